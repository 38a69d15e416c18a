"""GPU parity of the top-k membership variant (each token in its top-m
groups; far pairs kept when the tokens share any group, each pair once),
called through the C ABI binding, against the CPU oracle.

Bars as for the top-1 path: ids equal the oracle's except near-ties (there
each chosen group must score within the tie band of the oracle's group of
the same rank); perm and offsets bit-exact against the oracle sort of the
GPU's own ids; attention within max-abs 1e-2 and mean-abs 1e-3 of the fp64
oracle; lse within 1e-3.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from group_gated_sparse_amd import focus, synth, workloads
from gpu_common import TIE_BAND, check_attn, dev, dev_bf16, host, sample_rows, say

pytestmark = pytest.mark.gpu


def _qkv(rng, B, Hq, Hkv, n, d):
    q = synth.bf16_bits(rng.standard_normal((B, Hq, n, d), dtype=np.float32))
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    return q, k, v


def _member_ids(rng, B, n, K, m):
    """m distinct groups per token, uniformly at random."""
    return np.stack([np.stack([rng.choice(K, size=m, replace=False) for _ in range(n)])
                     for _ in range(B)]).astype(np.int32)


def check_topk_ids(gids, rids, hidden_rows, P, C, bias, what):
    """gids, rids: [tokens, m]. Equal where every rank decision of the
    oracle is clear of the tie band; elsewhere the GPU's groups are distinct
    and each scores (fp64) within the band of the oracle's same-rank score."""
    h = hidden_rows.astype(np.float64)
    s = (h @ P.astype(np.float64)) @ C.astype(np.float64).T
    if bias is not None:
        s = s + bias.astype(np.float64)
    m = gids.shape[1]
    srt = -np.sort(-s, axis=1)
    gaps = srt[:, :-1] - srt[:, 1:] if s.shape[1] > 1 else np.full((s.shape[0], 0), np.inf)
    clear = (gaps[:, :m] > TIE_BAND).all(axis=1)
    diff = np.nonzero((gids != rids).any(axis=1))[0]
    say(f"  {what}: {diff.size} of {gids.shape[0]} tokens differ; {int((~clear).sum())} near ties")
    assert clear[diff].sum() == 0, f"{what}: ids differ on clear tokens {diff[clear[diff]][:8]}"
    for t in diff:
        assert len(set(gids[t].tolist())) == m
        got = s[t, gids[t]]
        assert np.all(np.abs(got - srt[t, :m]) <= TIE_BAND), f"{what}: token {t} off rank"


# ---------------------------------------------------------------- assign
ASSIGN_CASES = [
    # (name, B, n, d_model, d_proj, K, m, bias)
    ("k2_m2", 1, 70, 64, 16, 2, 2, False),
    ("k4_m2", 2, 300, 128, 32, 4, 2, True),
    ("k33_m2", 1, 300, 256, 64, 33, 2, True),
    ("k64_m2_dproj200", 2, 128, 512, 200, 64, 2, False),
    ("k7_m1", 3, 101, 100, 20, 7, 1, True),
]


@pytest.mark.parametrize("case", ASSIGN_CASES, ids=[c[0] for c in ASSIGN_CASES])
def test_assign_topk_matches_oracle(case):
    name, B, n, d_model, d_proj, K, m, use_bias = case
    say(f"[assign top-k] {name}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    h = rng.standard_normal((B, n, d_model), dtype=np.float32)
    P = rng.standard_normal((d_model, d_proj), dtype=np.float32) / np.float32(np.sqrt(d_model))
    C = rng.standard_normal((K, d_proj), dtype=np.float32)
    C /= np.linalg.norm(C, axis=1, keepdims=True)
    bias = (rng.standard_normal(K).astype(np.float32) * np.float32(0.2)) if use_bias else None
    tb = None if bias is None else dev(bias)
    ids, margin = focus.focus_assign_topk(dev(h), dev(P), dev(C), m, tb)
    torch.cuda.synchronize()
    rids, rmargin = oracle.assign_topk(h, P, C, m, bias)
    gids = host(ids).reshape(B * n, m)
    check_topk_ids(gids, rids.reshape(B * n, m), h.reshape(-1, d_model), P, C, bias, name)
    gm, rm = host(margin).ravel(), rmargin.ravel()
    fin = np.isfinite(rm)
    assert np.array_equal(np.isfinite(gm), fin)
    assert np.max(np.abs(gm[fin] - rm[fin]), initial=0.0) < 1e-4
    if m == 1:   # the top-1 entry point gives the same bits
        ids1, margin1 = focus.focus_assign(dev(h), dev(P), dev(C), tb)
        torch.cuda.synchronize()
        assert np.array_equal(host(ids1).ravel(), gids.ravel())
        assert np.array_equal(host(margin1), host(margin))


# ---------------------------------------------------------------- sort
@pytest.mark.parametrize("B,n,K", [(1, 1, 2), (2, 3000, 4), (1, 5000, 64)])
def test_group_sort_of_entries_bit_exact(B, n, K):
    say(f"[sort entries] B={B} n={n} K={K}")
    rng = np.random.default_rng(n + K)
    ids = _member_ids(rng, B, n, K, 2)
    perm, offs = focus.focus_group_sort(dev(ids), K)
    torch.cuda.synchronize()
    rperm, roffs = oracle.group_sort_multi(ids, K)
    assert np.array_equal(host(perm), rperm) and np.array_equal(host(offs), roffs)


# ---------------------------------------------------------------- attention
def _run_topk(q, k, v, ids, K, m, w, scale, out_dtype=torch.float32):
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    tid = dev(ids)
    perm, offs = focus.focus_group_sort(tid, K)
    out, lse = focus.focus_attn_topk_fwd(tq, tk, tv, tid, perm, offs, K, m, w, scale,
                                         out_dtype=out_dtype, want_lse=True)
    torch.cuda.synchronize()
    return host(out.float()), host(lse), host(perm), host(offs)


TOPK_CASES = [
    # (name, B, Hq, Hkv, n, d, K, m, w)
    ("n1", 1, 1, 1, 1, 64, 2, 2, 0),
    ("ragged_n77_d32", 1, 2, 1, 77, 32, 4, 2, 5),
    ("w0_d64", 2, 2, 2, 200, 64, 4, 2, 0),
    ("all_groups_k2", 1, 2, 1, 300, 128, 2, 2, 17),
    ("K_gt_n", 1, 2, 2, 40, 64, 64, 2, 3),
    ("gqa3_ragged", 1, 6, 2, 333, 128, 5, 2, 40),
    ("gqa8_d128", 1, 16, 2, 520, 128, 7, 2, 64),
    ("many_tiles", 2, 3, 3, 1100, 64, 9, 2, 100),
    ("k4_long_d128", 1, 8, 8, 2000, 128, 4, 2, 64),
    ("m1", 1, 4, 2, 300, 64, 5, 1, 20),
    # the entry passes (K >= 5) at d = 32 (64-key tiles) with a ragged second half, and at w = 0
    ("entries_d32_ragged", 1, 4, 2, 150, 32, 6, 2, 9),
    ("entries_w0_b2", 2, 4, 4, 260, 64, 12, 2, 0),
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_focus_attn_topk_matches_oracle(case):
    name, B, Hq, Hkv, n, d, K, m, w = case
    say(f"[attn top-k] {name}: B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} K={K} m={m} w={w}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = _member_ids(rng, B, n, K, m)
    scale = 1.0 / math.sqrt(d)
    if m > 1:
        out, lse, perm, offs = _run_topk(q, k, v, ids, K, m, w, scale)
    else:
        out, lse, perm, offs = _run_topk_m1(q, k, v, ids[..., 0].copy(), K, w, scale)
    ref, rlse, _ = oracle.attn_multi(q, k, v, ids, w, scale)
    check_attn(out.reshape(-1, d), ref.reshape(-1, d), name)
    assert np.max(np.abs(lse - rlse)) < 1e-3
    rperm, roffs = oracle.group_sort_multi(ids, K)
    assert np.array_equal(perm, rperm) and np.array_equal(offs, roffs)


def _run_topk_m1(q, k, v, ids2d, K, w, scale):
    """m = 1 through the top-k entry point (ids (B, n, 1)) and, bit for bit,
    the same result as focus_attn_fwd."""
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    tid = dev(ids2d)
    perm, offs = focus.focus_group_sort(tid, K)
    out, lse = focus.focus_attn_topk_fwd(tq, tk, tv, tid.view(*tid.shape, 1), perm, offs, K, 1,
                                         w, scale, out_dtype=torch.float32, want_lse=True)
    out1, lse1 = focus.focus_attn_fwd(tq, tk, tv, tid, perm, offs, K, w, scale,
                                      out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out1) and torch.equal(lse, lse1)
    return host(out), host(lse), host(perm), host(offs)


def test_topk_bf16_output_and_all_groups_equal_dense():
    say("[attn top-k] bf16 output; m = K against the dense kernel")
    rng = np.random.default_rng(31)
    B, Hq, Hkv, n, d, K, w = 1, 8, 2, 700, 128, 6, 90
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = _member_ids(rng, B, n, K, 2)
    out, _, _, _ = _run_topk(q, k, v, ids, K, 2, w, 0.088, out_dtype=torch.bfloat16)
    ref, _, _ = oracle.attn_multi(q, k, v, ids, w, 0.088)
    check_attn(out.reshape(-1, d), ref.reshape(-1, d), "bf16 out", bf16_out=True)
    # K = m = 2: every pair shares both groups -> full causal attention
    ids2 = _member_ids(rng, B, n, 2, 2)
    a, la, _, _ = _run_topk(q, k, v, ids2, 2, 2, 50, 0.088)
    dense, dlse = focus.dense_causal_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), 0.088,
                                              out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    assert np.max(np.abs(a - host(dense))) < 1e-2 and np.max(np.abs(la - host(dlse))) < 1e-3


def test_topk_two_calls_equal_one():
    """focus_attn_window (second stream, before the sort) then
    focus_attn_topk_long_range_merge == focus_attn_topk_fwd, bit for bit."""
    say("[attn top-k] split calls")
    rng = np.random.default_rng(32)
    B, Hq, Hkv, n, d, K, m, w = 1, 8, 2, 900, 128, 4, 2, 70
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = _member_ids(rng, B, n, K, m)
    tq, tk, tv, tid = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(ids)
    perm, offs = focus.focus_group_sort(tid, K)
    one, lse1 = focus.focus_attn_topk_fwd(tq, tk, tv, tid, perm, offs, K, m, w, 0.1,
                                          out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    ws = torch.empty(focus.focus_attn_topk_workspace_bytes(B, Hq, Hkv, n, d, K, m, w),
                     dtype=torch.uint8, device="cuda")
    two = torch.empty_like(one)
    lse2 = torch.empty_like(lse1)
    side, main = torch.cuda.Stream(), torch.cuda.current_stream()
    side.wait_stream(main)
    focus.focus_attn_window(tq, tk, tv, K, w, 0.1, workspace=ws, out=two, lse=lse2, stream=side)
    perm2, offs2 = focus.focus_group_sort(tid, K, stream=main)
    main.wait_stream(side)
    focus.focus_attn_topk_long_range_merge(tq, tk, tv, tid, perm2, offs2, K, m, w, 0.1,
                                           workspace=ws, out=two, lse=lse2, stream=main)
    torch.cuda.synchronize()
    assert torch.equal(one, two) and torch.equal(lse1, lse2)


@pytest.mark.parametrize("K", [4, 6], ids=["set_pass", "entry_passes"])
def test_topk_apply_repeats_on_one_window_partial(K):
    """The long-range calls only read the window partial: merging twice from
    one window pass gives the same result twice, equal to focus_attn_topk_fwd
    (both long-range forms)."""
    say(f"[attn top-k] apply twice, K={K}")
    rng = np.random.default_rng(40 + K)
    B, Hq, Hkv, n, d, m, w = 1, 4, 2, 700, 64, 2, 30
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = _member_ids(rng, B, n, K, m)
    tq, tk, tv, tid = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(ids)
    perm, offs = focus.focus_group_sort(tid, K)
    one, lse1 = focus.focus_attn_topk_fwd(tq, tk, tv, tid, perm, offs, K, m, w, 0.125,
                                          out_dtype=torch.float32, want_lse=True)
    ws = torch.empty(focus.focus_attn_topk_workspace_bytes(B, Hq, Hkv, n, d, K, m, w),
                     dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(one) for _ in range(2)]
    lses = [torch.empty_like(lse1) for _ in range(2)]
    focus.focus_attn_window(tq, tk, tv, K, w, 0.125, workspace=ws, out=outs[0], lse=lses[0])
    for o, l in zip(outs, lses):
        focus.focus_attn_topk_long_range_merge(tq, tk, tv, tid, perm, offs, K, m, w, 0.125,
                                               workspace=ws, out=o, lse=l)
    torch.cuda.synchronize()
    for o, l in zip(outs, lses):
        assert torch.equal(o, one) and torch.equal(l, lse1)


def test_topk_three_calls_equal_one():
    """focus_attn_window (second stream) beside the sort and
    focus_attn_topk_long_range_prepare, then focus_attn_topk_long_range_apply
    == focus_attn_topk_fwd, bit for bit."""
    say("[attn top-k] prepare / apply calls")
    rng = np.random.default_rng(33)
    B, Hq, Hkv, n, d, K, m, w = 1, 8, 2, 700, 64, 6, 2, 50
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = _member_ids(rng, B, n, K, m)
    tq, tk, tv, tid = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(ids)
    perm, offs = focus.focus_group_sort(tid, K)
    one, lse1 = focus.focus_attn_topk_fwd(tq, tk, tv, tid, perm, offs, K, m, w, 0.1,
                                          out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    ws = torch.empty(focus.focus_attn_topk_workspace_bytes(B, Hq, Hkv, n, d, K, m, w),
                     dtype=torch.uint8, device="cuda")
    two = torch.empty_like(one)
    lse2 = torch.empty_like(lse1)
    side, main = torch.cuda.Stream(), torch.cuda.current_stream()
    side.wait_stream(main)
    focus.focus_attn_window(tq, tk, tv, K, w, 0.1, workspace=ws, out=two, lse=lse2, stream=side)
    perm2, offs2 = focus.focus_group_sort(tid, K, stream=main)
    focus.focus_attn_topk_long_range_prepare(tq, tk, tv, tid, perm2, offs2, K, m, w, 0.1,
                                             workspace=ws, out=two, lse=lse2, stream=main)
    main.wait_stream(side)
    focus.focus_attn_topk_long_range_apply(tq, tk, tv, tid, perm2, offs2, K, m, w, 0.1,
                                           workspace=ws, out=two, lse=lse2, stream=main)
    torch.cuda.synchronize()
    assert torch.equal(one, two) and torch.equal(lse1, lse2)


# ---------------------------------------------------------------- workloads
def test_whole_path_small_top2():
    """assign (top-2) -> sort of entries -> attention, all rows, on the
    small workload shape with m = 2."""
    wl = workloads.TINY.with_(name="tiny_top2_n256", m=2)
    say(f"[path top-k] {wl.name}")
    x = synth.make_inputs(wl)
    out, lse, ids, perm, offs = focus.focus_forward(
        dev(x["hidden"]), dev(x["P"]), dev(x["C"]), None if x["bias"] is None else dev(x["bias"]),
        dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), wl.w, wl.softmax_scale, m=2,
        out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    gids = host(ids)
    rids, _ = oracle.assign_topk(x["hidden"], x["P"], x["C"], 2, x["bias"])
    check_topk_ids(gids.reshape(-1, 2), rids.reshape(-1, 2), x["hidden"].reshape(-1, wl.d_model),
                   x["P"], x["C"], x["bias"], wl.name)
    rperm, roffs = oracle.group_sort_multi(gids, wl.K)
    assert np.array_equal(host(perm), rperm) and np.array_equal(host(offs), roffs)
    ref, rlse, _ = oracle.attn_multi(x["q"], x["k"], x["v"], gids, wl.w, wl.softmax_scale)
    check_attn(host(out).reshape(-1, wl.d), ref.reshape(-1, wl.d), wl.name)
    assert np.max(np.abs(host(lse) - rlse)) < 1e-3


@pytest.mark.parametrize("wl", [workloads.TOP2_K4, workloads.TOP2_K32], ids=lambda w: w.name)
def test_whole_path_top2_full_size_sampled(wl):
    """The benchmark's top-2 launch sequence at full size (window pass on a
    second stream while assign and sort run, then the long-range merge; bf16
    output, then fp32 with lse from the same window partial), checked on
    sampled tokens and rows."""
    say(f"[full top-k] {wl.name}: drawing inputs")
    x = synth.make_inputs(wl)
    B, n, K, w, d, Hq, m = wl.B, wl.n, wl.K, wl.w, wl.d, wl.Hq, wl.m
    hidden, P, C = dev(x["hidden"]), dev(x["P"]), dev(x["C"])
    bias = None if x["bias"] is None else dev(x["bias"])
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    say(f"[full top-k] {wl.name}: running the path")
    ws = torch.empty(max(focus.focus_attn_topk_workspace_bytes(B, Hq, wl.Hkv, n, d, K, m, w), 1),
                     dtype=torch.uint8, device=q.device)
    out = torch.empty((B, Hq, n, d), dtype=torch.bfloat16, device=q.device)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    side.wait_stream(main)
    focus.focus_attn_window(q, k, v, K, w, wl.softmax_scale, workspace=ws, out=out, stream=side)
    ids, margin = focus.focus_assign_topk(hidden, P, C, m, bias, stream=main)
    perm, offs = focus.focus_group_sort(ids, K, stream=main)
    main.wait_stream(side)
    focus.focus_attn_topk_long_range_merge(q, k, v, ids, perm, offs, K, m, w, wl.softmax_scale,
                                           workspace=ws, out=out, stream=main)
    out32 = torch.empty((B, Hq, n, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device)
    focus.focus_attn_topk_long_range_merge(q, k, v, ids, perm, offs, K, m, w, wl.softmax_scale,
                                           workspace=ws, out=out32, lse=lse, stream=main)
    torch.cuda.synchronize()
    del hidden, q, k, v, ws
    gids = host(ids)

    rng = np.random.default_rng(zlib.crc32(wl.name.encode()))
    tok = np.unique(np.concatenate([[0, B * n - 1], rng.integers(0, B * n, size=4096)]))
    rids, rmargin = oracle.assign_topk(x["hidden"], x["P"], x["C"], m, x["bias"], tokens=tok)
    check_topk_ids(gids.reshape(-1, m)[tok], rids, x["hidden"].reshape(-1, wl.d_model)[tok],
                   x["P"], x["C"], x["bias"], wl.name)
    assert np.max(np.abs(host(margin).ravel()[tok] - rmargin)) < 1e-4
    rperm, roffs = oracle.group_sort_multi(gids, K)
    assert np.array_equal(host(perm), rperm) and np.array_equal(host(offs), roffs)

    rows = sample_rows(rng, B, Hq, n, w, per_head=max(16, 4096 // Hq), ids=gids)
    ref, rlse, _ = oracle.attn_multi(x["q"], x["k"], x["v"], gids, w, wl.softmax_scale, rows=rows)
    check_attn(host(out.float()).reshape(-1, d)[rows], ref.reshape(-1, d),
               f"{wl.name} bf16 out", bf16_out=True)
    check_attn(host(out32).reshape(-1, d)[rows], ref.reshape(-1, d), f"{wl.name} fp32 out")
    assert np.max(np.abs(host(lse).ravel()[rows] - rlse.ravel())) < 1e-3


def test_topk_deterministic_and_stream_independent():
    say("[attn top-k] determinism / non-default stream")
    rng = np.random.default_rng(33)
    B, Hq, Hkv, n, d, K, m, w = 1, 8, 1, 1500, 128, 6, 2, 64
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    ids = _member_ids(rng, B, n, K, m)
    a = _run_topk(q, k, v, ids, K, m, w, 0.09)
    b = _run_topk(q, k, v, ids, K, m, w, 0.09)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tq, tk, tv, tid = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(ids)
        perm, offs = focus.focus_group_sort(tid, K, stream=s)
        out, lse = focus.focus_attn_topk_fwd(tq, tk, tv, tid, perm, offs, K, m, w, 0.09,
                                             out_dtype=torch.float32, want_lse=True, stream=s)
    s.synchronize()
    c = (host(out), host(lse))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
