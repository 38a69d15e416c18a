"""GPU parity of the training-time soft-gated attention (every causal pair;
pairs beyond the window weighted by sigmoid(lambda g_i . g_j) inside the
softmax), called through the C ABI binding, against the fp64 CPU oracle.

Bar: as for the inference path, max-abs 1e-2 and mean-abs 1e-3 on the output
(fp32; bf16 output adds its own rounding), lse within 1e-3. The gate itself
adds little: the affinity is formed from a bf16 hi/lo split of the fp32
soft assignments (about 2^-16 relative) and the sigmoid in fp32.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from group_gated_sparse_amd import focus, synth, workloads
from gpu_common import check_attn, dev, dev_bf16, host, sample_rows, say

pytestmark = pytest.mark.gpu


def _qkv(rng, B, Hq, Hkv, n, d):
    q = synth.bf16_bits(rng.standard_normal((B, Hq, n, d), dtype=np.float32))
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    return q, k, v


def _soft(rng, B, n, K, sharp=2.0):
    x = rng.standard_normal((B, n, K)) * sharp
    e = np.exp(x - x.max(-1, keepdims=True))
    return (e / e.sum(-1, keepdims=True)).astype(np.float32)


CASES = [
    # (name, B, Hq, Hkv, n, d, K, w, lam)
    ("n1", 1, 1, 1, 1, 64, 4, 0, 5.0),
    ("ragged_d32_k4", 1, 2, 1, 77, 32, 4, 5, 8.0),
    ("w0_d64_k20", 2, 2, 2, 200, 64, 20, 0, 6.0),
    ("lam0", 1, 2, 2, 150, 64, 8, 10, 0.0),
    ("neg_lam_k7", 1, 4, 2, 333, 128, 7, 40, -12.0),
    ("k32_gqa8", 1, 16, 2, 520, 128, 32, 64, 10.0),
    ("k64_d128", 1, 4, 4, 700, 128, 64, 30, 20.0),
    ("k64_d32", 1, 2, 1, 300, 32, 64, 7, 3.0),
    ("k33_d64_many_tiles", 2, 3, 3, 1100, 64, 33, 100, 9.0),
    ("wide_window", 1, 2, 2, 150, 128, 16, 149, 7.0),
    # four and eight heads per workgroup: gates shared between waves
    ("k16_g4_d64", 1, 8, 2, 400, 64, 16, 20, 6.0),
    ("k8_g8_d32", 1, 8, 1, 300, 32, 8, 10, 4.0),
    ("k64_g8_d128", 1, 8, 1, 450, 128, 64, 33, 15.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_soft_gate_matches_oracle(case):
    name, B, Hq, Hkv, n, d, K, w, lam = case
    say(f"[soft gate] {name}: B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} K={K} w={w} lambda={lam}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    G = _soft(rng, B, n, K)
    scale = 1.0 / math.sqrt(d)
    out, lse = focus.focus_soft_gate_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(G), w,
                                              scale, lam, out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.soft_gate_attn(q, k, v, G, w, scale, lam)
    check_attn(host(out).reshape(-1, d), ref.reshape(-1, d), name)
    assert np.max(np.abs(host(lse) - rlse)) < 1e-3


def test_soft_gate_bf16_output_and_wide_window_equals_dense():
    say("[soft gate] bf16 output; w >= n-1 against the dense kernel")
    rng = np.random.default_rng(41)
    B, Hq, Hkv, n, d, K = 1, 8, 2, 640, 128, 24
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    G = _soft(rng, B, n, K)
    tq, tk, tv, tG = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(G)
    out, _ = focus.focus_soft_gate_attn_fwd(tq, tk, tv, tG, 50, 0.09, 5.0)
    ref, _ = oracle.soft_gate_attn(q, k, v, G, 50, 0.09, 5.0)
    torch.cuda.synchronize()
    check_attn(host(out.float()).reshape(-1, d), ref.reshape(-1, d), "bf16 out", bf16_out=True)
    wide, _ = focus.focus_soft_gate_attn_fwd(tq, tk, tv, tG, n - 1, 0.09, 5.0,
                                             out_dtype=torch.float32)
    dense, _ = focus.dense_causal_attn_fwd(tq, tk, tv, 0.09, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.max(np.abs(host(wide) - host(dense))) < 1e-2


def test_soft_gate_full_size_sampled():
    """The measured configuration: the 70B layer shape (B=1, Hq=64, Hkv=8,
    n=32768, d=128, w=1024) with K=32 Sinkhorn soft assignments of the
    workload's hidden states (10 rounds, tau=1) and lambda = 8; sampled rows
    of every head against the oracle."""
    wl = workloads.GQA70B
    say(f"[soft gate full] {wl.name}: drawing inputs")
    x = synth.make_inputs(wl)
    S = focus.focus_assign_scores(dev(x["hidden"]), dev(x["P"]), dev(x["C"]),
                                  None if x["bias"] is None else dev(x["bias"]))
    G = focus.focus_sinkhorn(S, 1.0, 10)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    out, lse = focus.focus_soft_gate_attn_fwd(q, k, v, G, wl.w, wl.softmax_scale, 8.0,
                                              out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    g_host = host(G)
    del q, k, v, S
    rng = np.random.default_rng(42)
    rows = sample_rows(rng, wl.B, wl.Hq, wl.n, wl.w, per_head=16)
    ref, rlse = oracle.soft_gate_attn(x["q"], x["k"], x["v"], g_host, wl.w, wl.softmax_scale,
                                      8.0, rows=rows)
    check_attn(host(out).reshape(-1, wl.d)[rows], ref.reshape(-1, wl.d), f"{wl.name} soft gate")
    assert np.max(np.abs(host(lse).ravel()[rows] - rlse)) < 1e-3


def test_soft_gate_deterministic_and_workspace_reusable():
    say("[soft gate] determinism")
    rng = np.random.default_rng(43)
    B, Hq, Hkv, n, d, K = 1, 8, 2, 900, 128, 20
    q, k, v = _qkv(rng, B, Hq, Hkv, n, d)
    G = _soft(rng, B, n, K)
    tq, tk, tv, tG = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(G)
    ws = torch.empty(focus.focus_soft_gate_attn_workspace_bytes(B, n, K), dtype=torch.uint8,
                     device="cuda")
    a, la = focus.focus_soft_gate_attn_fwd(tq, tk, tv, tG, 40, 0.09, 6.0, workspace=ws,
                                           out_dtype=torch.float32, want_lse=True)
    b, lb = focus.focus_soft_gate_attn_fwd(tq, tk, tv, tG, 40, 0.09, 6.0, workspace=ws,
                                           out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
