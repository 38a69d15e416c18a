"""GPU parity: every entry point of libfocus.so, called through the C ABI
binding, against the CPU oracle on the same seeded inputs.

Bars: group ids equal except near-ties (oracle top-2 margin < 1e-3, where
either of the two top groups is accepted); perm and offsets bit-exact against
the oracle sort of the GPU's own ids; attention within max-abs 1e-2 and
mean-abs 1e-3 of the fp64 oracle (fp32 output; bf16 output adds its own
rounding).
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from group_gated_sparse_amd import focus, synth, workloads
from gpu_common import (check_attn, check_ids, dev, dev_bf16, host, sample_rows, say,
                        visited_pairs)

pytestmark = pytest.mark.gpu


def _qkv(rng, B, Hq, Hkv, n, d):
    q = synth.bf16_bits(rng.standard_normal((B, Hq, n, d), dtype=np.float32))
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    return q, k, v


def _run_attn(q, k, v, ids, K, w, scale, out_dtype=torch.float32, stream=None):
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    tid = dev(ids.astype(np.int32))
    perm, offs = focus.focus_group_sort(tid, K, stream=stream)
    out, lse = focus.focus_attn_fwd(tq, tk, tv, tid, perm, offs, K, w, scale,
                                    out_dtype=out_dtype, want_lse=True, stream=stream)
    torch.cuda.synchronize()
    return host(out.float()), host(lse), host(perm), host(offs)


# ---------------------------------------------------------------- attention
ATTN_CASES = [
    # (name, B, Hq, Hkv, n, d, K, w)
    ("n1", 1, 1, 1, 1, 64, 3, 0),
    ("ragged_n77_d32", 1, 2, 1, 77, 32, 3, 5),
    ("w0_d64", 2, 2, 2, 200, 64, 4, 0),
    ("K_gt_n", 1, 2, 2, 40, 64, 64, 3),
    ("single_group", 1, 2, 1, 300, 128, 1, 17),
    ("gqa3_ragged", 1, 6, 2, 333, 128, 5, 40),
    ("gqa8_d128", 1, 16, 2, 520, 128, 7, 64),
    ("gqa16", 1, 16, 1, 260, 64, 6, 30),
    ("wide_window", 1, 2, 2, 150, 32, 4, 149),
    ("many_tiles", 2, 3, 3, 1100, 64, 9, 100),
    # query tiles spanning more than the 7 groups a plan record holds (the
    # kernel derives the segments itself and masks every key tile)
    ("many_groups_per_tile", 1, 2, 2, 1000, 64, 64, 8),
    ("many_groups_d128", 1, 4, 4, 900, 128, 64, 10),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_focus_attn_matches_oracle(case):
    name, B, Hq, Hkv, n, d, K, w = case
    say(f"[attn] {name}: B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} K={K} w={w}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    scale = 1.0 / math.sqrt(d)
    out, lse, perm, offs = _run_attn(q, k, v, ids, K, w, scale)
    ref, rlse, _ = oracle.attn(q, k, v, ids, w, scale)
    check_attn(out.reshape(-1, d), ref.reshape(-1, d), name)
    assert np.max(np.abs(lse - rlse)) < 1e-3
    rperm, roffs = oracle.group_sort(ids, K)
    assert np.array_equal(perm, rperm) and np.array_equal(offs, roffs)


def test_focus_attn_bf16_output():
    say("[attn] bf16 output")
    rng = np.random.default_rng(21)
    B, Hq, Hkv, n, d, K, w = 1, 8, 2, 700, 128, 6, 90
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    out, _, _, _ = _run_attn(q, k, v, ids, K, w, 0.088, out_dtype=torch.bfloat16)
    ref, _, _ = oracle.attn(q, k, v, ids, w, 0.088)
    check_attn(out.reshape(-1, d), ref.reshape(-1, d), "bf16 out", bf16_out=True)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_dense_causal_matches_oracle(d):
    say(f"[dense] d={d}")
    rng = np.random.default_rng(d)
    B, Hq, Hkv, n = 2, 4, 2, 517
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    scale = 1.0 / math.sqrt(d)
    out, lse = focus.dense_causal_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale,
                                           out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    ref, rlse, _ = oracle.attn(q, k, v, np.zeros((B, n), np.int32), 0, scale)
    check_attn(host(out).reshape(-1, d), ref.reshape(-1, d), f"dense d={d}")
    assert np.max(np.abs(host(lse) - rlse)) < 1e-3


def test_single_group_and_wide_window_equal_dense():
    """K = 1 and w >= n-1 both reduce the pattern to full causal attention."""
    say("[attn] K=1 and w>=n-1 against the dense kernel")
    rng = np.random.default_rng(5)
    B, Hq, Hkv, n, d = 1, 8, 8, 640, 64
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    dense, _ = focus.dense_causal_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), 0.125,
                                           out_dtype=torch.float32)
    a, _, _, _ = _run_attn(q, k, v, np.zeros((B, n), np.int32), 1, 37, 0.125)
    b, _, _, _ = _run_attn(q, k, v, rng.integers(0, 5, size=(B, n), dtype=np.int32), 5, n - 1,
                           0.125)
    dn = host(dense)
    assert np.max(np.abs(a - dn)) < 1e-2 and np.max(np.abs(b - dn)) < 1e-5


def test_deterministic_and_stream_independent():
    say("[attn] determinism / non-default stream")
    rng = np.random.default_rng(9)
    B, Hq, Hkv, n, d, K, w = 1, 8, 1, 900, 128, 8, 64
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    a = _run_attn(q, k, v, ids, K, w, 0.09)
    b = _run_attn(q, k, v, ids, K, w, 0.09)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = _run_attn(q, k, v, ids, K, w, 0.09, stream=s)
    s.synchronize()
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)


def test_side_stream_call_keeps_the_buffers_it_allocates():
    """A call enqueued on a side stream while the default stream stays
    current: the binding allocates the sort's and the attention's workspaces
    and outputs and drops the workspaces on return, while the kernels still
    run on the side stream. Large tensors allocated and filled on the default
    stream right after each call must not land on those blocks (the binding
    records the side stream on them), so the results equal an eager run on
    the default stream bit for bit."""
    say("[attn] side-stream call, default stream allocating meanwhile")
    rng = np.random.default_rng(4242)
    B, Hq, Hkv, n, d, K, w = 1, 16, 2, 8192, 128, 8, 256
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    tq, tk, tv, tid = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(ids)
    perm, offs = focus.focus_group_sort(tid, K)
    ref, ref_lse = focus.focus_attn_fwd(tq, tk, tv, tid, perm, offs, K, w, 0.1,
                                        out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse, ref_perm = host(ref), host(ref_lse), host(perm)
    del perm, offs
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    nbytes = focus.focus_attn_workspace_bytes(B, Hq, Hkv, n, d, K, w)
    junk = []
    perm_s, offs_s = focus.focus_group_sort(tid, K, stream=side)
    junk.append(torch.full((1 << 20,), -1, dtype=torch.int32, device=tq.device))
    out_s, lse_s = focus.focus_attn_fwd(tq, tk, tv, tid, perm_s, offs_s, K, w, 0.1,
                                        out_dtype=torch.float32, want_lse=True, stream=side)
    for _ in range(3):
        junk.append(torch.full((nbytes // 4,), float("nan"), dtype=torch.float32,
                               device=tq.device))
    main.wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(host(perm_s), ref_perm)
    assert np.array_equal(host(out_s), ref) and np.array_equal(host(lse_s), ref_lse)


def test_two_calls_equal_one():
    """focus_attn_window (on a second stream, no group data, started before
    the groups are sorted) then focus_attn_long_range_merge ==
    focus_attn_fwd, bit for bit."""
    say("[attn] split calls")
    rng = np.random.default_rng(10)
    B, Hq, Hkv, n, d, K, w = 1, 4, 4, 480, 64, 5, 33
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    tq, tk, tv, tid = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(ids)
    perm, offs = focus.focus_group_sort(tid, K)
    one, lse1 = focus.focus_attn_fwd(tq, tk, tv, tid, perm, offs, K, w, 0.125,
                                     out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    ws = torch.empty(focus.focus_attn_workspace_bytes(B, Hq, Hkv, n, d, K, w), dtype=torch.uint8,
                     device="cuda")
    two = torch.empty_like(one)
    lse2 = torch.empty_like(lse1)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    focus.focus_attn_window(tq, tk, tv, K, w, 0.125, workspace=ws, out=two, lse=lse2, stream=side)
    perm2, offs2 = focus.focus_group_sort(tid, K, stream=main)
    main.wait_stream(side)
    focus.focus_attn_long_range_merge(tq, tk, tv, tid, perm2, offs2, K, w, 0.125, workspace=ws,
                                      out=two, lse=lse2, stream=main)
    torch.cuda.synchronize()
    assert torch.equal(one, two) and torch.equal(lse1, lse2)


def test_three_calls_equal_one():
    """focus_attn_window on a second stream, beside it the sort then
    focus_attn_long_range_prepare on the main stream, then
    focus_attn_long_range_apply once both are done == focus_attn_fwd, bit for
    bit; the prepared workspace serves a second apply with other q."""
    say("[attn] prepare / apply calls")
    rng = np.random.default_rng(11)
    B, Hq, Hkv, n, d, K, w = 2, 8, 2, 1000, 128, 7, 40
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    ids[1, 300:700] = 2   # one long group run
    tq, tk, tv, tid = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(ids)
    perm, offs = focus.focus_group_sort(tid, K)
    one, lse1 = focus.focus_attn_fwd(tq, tk, tv, tid, perm, offs, K, w, 0.1,
                                     out_dtype=torch.float32, want_lse=True)
    tq2 = dev_bf16(_qkv(rng, B, Hq, Hkv, n, d)[0])
    one2, _ = focus.focus_attn_fwd(tq2, tk, tv, tid, perm, offs, K, w, 0.1,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    ws = torch.empty(focus.focus_attn_workspace_bytes(B, Hq, Hkv, n, d, K, w), dtype=torch.uint8,
                     device="cuda")
    two = torch.empty_like(one)
    lse2 = torch.empty_like(lse1)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    focus.focus_attn_window(tq, tk, tv, K, w, 0.1, workspace=ws, out=two, lse=lse2, stream=side)
    perm2, offs2 = focus.focus_group_sort(tid, K, stream=main)
    focus.focus_attn_long_range_prepare(tq, tk, tv, tid, perm2, offs2, K, w, 0.1, workspace=ws,
                                        out=two, lse=lse2, stream=main)
    main.wait_stream(side)
    focus.focus_attn_long_range_apply(tq, tk, tv, tid, perm2, offs2, K, w, 0.1, workspace=ws,
                                      out=two, lse=lse2, stream=main)
    torch.cuda.synchronize()
    assert torch.equal(one, two) and torch.equal(lse1, lse2)
    # the prepared part depends only on k, v and the groups: a new window
    # pass for other q, then apply again
    three = torch.empty_like(one)
    focus.focus_attn_window(tq2, tk, tv, K, w, 0.1, workspace=ws, out=three)
    focus.focus_attn_long_range_apply(tq2, tk, tv, tid, perm2, offs2, K, w, 0.1, workspace=ws,
                                      out=three)
    torch.cuda.synchronize()
    assert torch.equal(one2, three)


# ---------------------------------------------------------------- sort
@pytest.mark.parametrize("B,n,K", [(1, 1, 1), (1, 5, 64), (3, 1000, 7), (2, 4097, 64), (1, 65536, 64)])
def test_group_sort_bit_exact(B, n, K):
    say(f"[sort] B={B} n={n} K={K}")
    rng = np.random.default_rng(n + K)
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    if n > 100:
        ids[:, 10:60] = 3 % K
    perm, offs = focus.focus_group_sort(dev(ids), K)
    torch.cuda.synchronize()
    rperm, roffs = oracle.group_sort(ids, K)
    assert np.array_equal(host(perm), rperm) and np.array_equal(host(offs), roffs)


# ---------------------------------------------------------------- assign
ASSIGN_CASES = [
    # (name, B, n, d_model, d_proj, K, bias)
    ("k1", 1, 50, 64, 16, 1, False),
    ("tiny_k4", 1, 256, 64, 32, 4, False),
    ("ragged_tokens_k7", 3, 101, 100, 20, 7, True),
    ("k33", 1, 300, 256, 64, 33, True),
    ("k64_dproj200", 2, 128, 512, 200, 64, False),
]


@pytest.mark.parametrize("case", ASSIGN_CASES, ids=[c[0] for c in ASSIGN_CASES])
def test_assign_matches_oracle(case):
    name, B, n, d_model, d_proj, K, use_bias = case
    say(f"[assign] {name}")
    rng = np.random.default_rng(len(name) * 7 + K)
    h = rng.standard_normal((B, n, d_model), dtype=np.float32)
    P = (rng.standard_normal((d_model, d_proj), dtype=np.float32) / np.float32(np.sqrt(d_model)))
    C = rng.standard_normal((K, d_proj), dtype=np.float32)
    C /= np.linalg.norm(C, axis=1, keepdims=True)
    bias = (rng.standard_normal(K).astype(np.float32) * np.float32(0.2)) if use_bias else None
    ids, margin = focus.focus_assign(dev(h), dev(P), dev(C), None if bias is None else dev(bias))
    torch.cuda.synchronize()
    rids, rmargin = oracle.assign(h, P, C, bias)
    check_ids(host(ids).ravel(), rids.ravel(), rmargin.ravel(), h.reshape(-1, d_model), P, C, bias,
              name)
    gm, rm = host(margin).ravel(), rmargin.ravel()
    fin = np.isfinite(rm)
    assert np.array_equal(np.isfinite(gm), fin)
    assert np.max(np.abs(gm[fin] - rm[fin]), initial=0.0) < 1e-4


# ---------------------------------------------------------------- workloads
@pytest.mark.parametrize("wl", [workloads.TINY, workloads.GPT2], ids=lambda w: w.name)
def test_whole_path_small_workloads(wl):
    """assign -> sort -> attention on the full small workloads, all rows."""
    say(f"[path] {wl.name}")
    x = synth.make_inputs(wl)
    out, lse, ids, perm, offs = focus.focus_forward(
        dev(x["hidden"]), dev(x["P"]), dev(x["C"]), None if x["bias"] is None else dev(x["bias"]),
        dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), wl.w, wl.softmax_scale,
        out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    gids = host(ids)
    rids, rmargin = oracle.assign(x["hidden"], x["P"], x["C"], x["bias"])
    check_ids(gids.ravel(), rids.ravel(), rmargin.ravel(), x["hidden"].reshape(-1, wl.d_model),
              x["P"], x["C"], x["bias"], wl.name)
    rperm, roffs = oracle.group_sort(gids, wl.K)
    assert np.array_equal(host(perm), rperm) and np.array_equal(host(offs), roffs)
    ref, rlse, vis = oracle.attn(x["q"], x["k"], x["v"], gids, wl.w, wl.softmax_scale)
    check_attn(host(out).reshape(-1, wl.d), ref.reshape(-1, wl.d), wl.name)
    assert int(vis[:, 0].sum()) == visited_pairs(gids, wl.w)


@pytest.mark.parametrize("wl", [workloads.ZIPF7B, workloads.LONG64K, workloads.GQA70B,
                                pytest.param(workloads.LONG1M,
                                             marks=pytest.mark.timeout(900))],
                         ids=lambda w: w.name)
def test_whole_path_full_size_sampled(wl):
    """The benchmark's launch sequence at full size (window pass on a second
    stream while assign and sort run, then the long-range merge; bf16
    output), checked on sampled tokens and rows: ids against the oracle on
    4096 tokens, perm/offsets bit-exact on all tokens, attention on the
    start, window edge, end and random rows of every head. A second merge of
    the same window partial with fp32 output and lse gets the strict bar."""
    say(f"[full] {wl.name}: drawing inputs")
    x = synth.make_inputs(wl)
    B, n, K, w, d, Hq = wl.B, wl.n, wl.K, wl.w, wl.d, wl.Hq
    hidden, P, C = dev(x["hidden"]), dev(x["P"]), dev(x["C"])
    bias = None if x["bias"] is None else dev(x["bias"])
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    say(f"[full] {wl.name}: running the path")
    ws = torch.empty(max(focus.focus_attn_workspace_bytes(B, Hq, wl.Hkv, n, d, K, w), 1),
                     dtype=torch.uint8, device=q.device)
    out = torch.empty((B, Hq, n, d), dtype=torch.bfloat16, device=q.device)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    side.wait_stream(main)
    focus.focus_attn_window(q, k, v, K, w, wl.softmax_scale, workspace=ws, out=out, stream=side)
    ids, margin = focus.focus_assign(hidden, P, C, bias, want_margin=True, stream=main)
    perm, offs = focus.focus_group_sort(ids, K, stream=main)
    main.wait_stream(side)
    focus.focus_attn_long_range_merge(q, k, v, ids, perm, offs, K, w, wl.softmax_scale,
                                      workspace=ws, out=out, stream=main)
    out32 = torch.empty((B, Hq, n, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device)
    focus.focus_attn_long_range_merge(q, k, v, ids, perm, offs, K, w, wl.softmax_scale,
                                      workspace=ws, out=out32, lse=lse, stream=main)
    torch.cuda.synchronize()
    del hidden, q, k, v, ws
    gids = host(ids)

    rng = np.random.default_rng(zlib.crc32(wl.name.encode()))
    tok = np.unique(np.concatenate([[0, B * n - 1], rng.integers(0, B * n, size=4096)]))
    rids, rmargin = oracle.assign(x["hidden"], x["P"], x["C"], x["bias"], tokens=tok)
    check_ids(gids.ravel()[tok], rids.ravel(), rmargin.ravel(),
              x["hidden"].reshape(-1, wl.d_model)[tok], x["P"], x["C"], x["bias"], wl.name)
    gm, rm = host(margin).ravel()[tok], rmargin.ravel()
    assert np.max(np.abs(gm - rm)) < 1e-4
    rperm, roffs = oracle.group_sort(gids, K)
    assert np.array_equal(host(perm), rperm) and np.array_equal(host(offs), roffs)

    # at least 8192 rows: every head, rows 0 .. w edges, the last rows, the
    # first and last token of every group, and random rows
    rows = sample_rows(rng, B, Hq, n, w, per_head=max(16, 8192 // Hq), ids=gids)
    ref, rlse, _ = oracle.attn(x["q"], x["k"], x["v"], gids, w, wl.softmax_scale, rows=rows)
    got16 = host(out.float()).reshape(-1, d)[rows]
    check_attn(got16, ref.reshape(-1, d), f"{wl.name} bf16 out", bf16_out=True)
    got32 = host(out32).reshape(-1, d)[rows]
    check_attn(got32, ref.reshape(-1, d), f"{wl.name} fp32 out")
    assert np.max(np.abs(host(lse).ravel()[rows] - rlse.ravel())) < 1e-3


@pytest.mark.parametrize("qscale", [0.0, 6.0, 8.0],
                         ids=["flat_scores", "sharp_scores_x6", "sharp_scores_x8"])
def test_focus_attn_extreme_score_ranges(qscale):
    """q = 0 (every kept key equally weighted) and q scaled by 6 or 8 (logits
    with a standard deviation near 6 or 8, so the reference max moves often,
    most weights underflow and a few keys carry each row): both passes and
    the merge against the oracle, at the same bar as every other case."""
    say(f"[attn] q scaled by {qscale}")
    rng = np.random.default_rng(int(qscale) + 50)
    B, Hq, Hkv, n, d, K, w = 1, 8, 2, 900, 128, 5, 70
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    q = synth.bf16_bits(synth.bf16_to_f32(q) * np.float32(qscale))
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    out, lse, _, _ = _run_attn(q, k, v, ids, K, w, 1.0 / math.sqrt(d))
    ref, rlse, _ = oracle.attn(q, k, v, ids, w, 1.0 / math.sqrt(d))
    check_attn(out.reshape(-1, d), ref.reshape(-1, d), f"q x {qscale}")
    assert np.max(np.abs(lse - rlse)) < 1e-3


@pytest.mark.parametrize("where", ["window", "long_range", "mixed"])
def test_focus_attn_one_dominant_key(where):
    """Each query row is built as 2 k_j for one kept key j (its logit is about
    22.6 against others of standard deviation 2), so nearly all of the row's
    weight sits on that key and the output is close to v_j: the case where a
    mismatch between the weights applied to V and the normaliser shows most.
    The key is taken inside the window, among the same-group keys beyond it,
    or either way at random."""
    say(f"[attn] one dominant key ({where})")
    rng = np.random.default_rng(zlib.crc32(("dominant_" + where).encode()))
    B, Hq, Hkv, n, d, K, w = 1, 8, 2, 700, 128, 4, 40
    _, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    kf = synth.bf16_to_f32(k)
    qf = np.zeros((B, Hq, n, d), dtype=np.float32)
    for i in range(n):
        near = np.arange(max(0, i - w), i + 1)
        far = np.nonzero(ids[0, :max(0, i - w)] == ids[0, i])[0]
        use_far = where == "long_range" or (where == "mixed" and rng.random() < 0.5)
        pool = far if (use_far and far.size) else near
        for h in range(Hq):
            j = int(rng.choice(pool))
            qf[0, h, i] = 2.0 * kf[0, h // (Hq // Hkv), j]
    q = synth.bf16_bits(qf)
    scale = 1.0 / math.sqrt(d)
    out, lse, _, _ = _run_attn(q, k, v, ids, K, w, scale)
    ref, rlse, _ = oracle.attn(q, k, v, ids, w, scale)
    check_attn(out.reshape(-1, d), ref.reshape(-1, d), f"dominant key ({where})")
    assert np.max(np.abs(lse - rlse)) < 1e-3


@pytest.mark.parametrize("case", [("copies_gqa8", 1, 16, 2, 700, 128, 7, 64),
                                  ("copies_ragged_d64", 2, 3, 3, 333, 64, 5, 20)],
                         ids=lambda c: c[0])
def test_long_range_copy_path_equals_in_place(case):
    """With one group per token the long-range pass reads key rows in place;
    focus_attn_fwd_sorted_kv takes the group-sorted copies it uses otherwise
    (two groups per token, or one head's K rows spanning 2^31 bytes or more).
    Both load the same rows into each key tile, so the outputs agree bit for
    bit, and both match the oracle."""
    name, B, Hq, Hkv, n, d, K, w = case
    say(f"[attn] {name}: B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} K={K} w={w}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    scale = 1.0 / math.sqrt(d)
    out_a, lse_a, _, _ = _run_attn(q, k, v, ids, K, w, scale)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    tid = dev(ids)
    perm, offs = focus.focus_group_sort(tid, K)
    ws = torch.empty(focus.focus_attn_sorted_kv_workspace_bytes(B, Hq, Hkv, n, d, K, w),
                     dtype=torch.uint8, device=tq.device)
    out_b, lse_b = focus.focus_attn_fwd_sorted_kv(tq, tk, tv, tid, perm, offs, K, w, scale,
                                                  out_dtype=torch.float32, want_lse=True,
                                                  workspace=ws)
    torch.cuda.synchronize()
    out_b, lse_b = host(out_b), host(lse_b)
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)
    ref, rlse, _ = oracle.attn(q, k, v, ids, w, scale)
    check_attn(out_b.reshape(-1, d), ref.reshape(-1, d), name)
    assert np.max(np.abs(lse_b - rlse)) < 1e-3
