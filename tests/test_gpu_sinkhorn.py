"""GPU parity of the training-time soft assignment: raw scores
(focus_assign_scores) and Sinkhorn normalisation (focus_sinkhorn), called
through the C ABI binding, against the CPU oracle.

Bars. Scores: within the error bound of the GPU's bf16 hi/lo split and of
both sides' fp32 sums (score_error_bound below) of the oracle's fp32 scores. Sinkhorn: the oracle runs in
fp64 on the GPU's own scores; every GPU value within 2e-4 relative (plus
1e-7 absolute for values near zero) of it. The bound comes from fp32
arithmetic: each pass forms row and column sums of at most a few hundred
sequential fp32 additions (rows per lane, then fixed-order trees), about
1e-5 relative, and each of the iters + 1 passes adds at most that much
(Sinkhorn scaling does not amplify relative errors); rows sum to 1 within
1e-5.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from group_gated_sparse_amd import focus, synth, workloads
from gpu_common import dev, host, say

pytestmark = pytest.mark.gpu

REL, ABS = 2e-4, 1e-7


def check_G(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > REL * np.abs(ref) + ABS
    rel = np.max(err / (np.abs(ref) + 1e-30))
    say(f"  {what}: max-abs {err.max():.3e} max-rel {rel:.3e}")
    assert not bad.any(), f"{what}: {bad.sum()} values beyond tolerance"
    assert np.max(np.abs(got.sum(-1, dtype=np.float64) - 1.0)) < 1e-5


def score_error_bound(h, P, C):
    """Bound on |GPU score - oracle score|. The GPU forms h (P C^T) from a
    two-term bf16 split of h and of W = P C^T, each term exact to 2^-17
    relative, and drops lo*lo: each product h_m W_mk is off by at most
    3 * 2^-17 of |h_m W_mk|. Both sides then add d_model products in fp32
    (at most d_model * 2^-24 relative to the sum of magnitudes each), and
    the oracle's own (h P) C^T order adds a like term over d_proj."""
    W = P.astype(np.float64) @ C.astype(np.float64).T
    mag = np.abs(h.astype(np.float64)) @ np.abs(W)
    d_model, d_proj = P.shape
    return mag * (3 * 2.0 ** -17 + 2 * (d_model + d_proj) * 2.0 ** -24) + 1e-6


def _scores(rng, B, n, K, spread):
    return (rng.standard_normal((B, n, K)) * spread).astype(np.float32)


SINK_CASES = [
    # (name, B, n, K, tau, iters, spread)
    ("n1_k1", 1, 1, 1, 1.0, 3, 1.0),
    ("k1", 2, 100, 1, 1.0, 2, 1.0),
    ("k2", 1, 513, 2, 1.0, 6, 1.0),
    ("zero_iters_k7", 1, 333, 7, 0.5, 0, 2.0),
    ("ragged_k32", 1, 1001, 32, 1.0, 10, 1.5),
    ("k64_b3", 3, 777, 64, 0.7, 5, 1.0),
    ("k3_many_blocks", 1, 300001, 3, 1.0, 4, 1.0),
    ("k33_small_n", 2, 17, 33, 2.0, 20, 3.0),
    ("k16_long", 1, 70000, 16, 1.0, 30, 1.0),
    # long sequences (one thread per row): 16-, 32- and 64-wide rows, ragged ends
    ("rows_k20", 1, 300007, 20, 1.0, 5, 1.0),
    ("rows_k50_b2", 2, 140001, 50, 0.8, 3, 1.5),
    ("rows_k64", 1, 262144, 64, 1.0, 8, 1.0),
]


@pytest.mark.parametrize("case", SINK_CASES, ids=[c[0] for c in SINK_CASES])
def test_sinkhorn_matches_oracle(case):
    name, B, n, K, tau, iters, spread = case
    say(f"[sinkhorn] {name}: B={B} n={n} K={K} tau={tau} iters={iters}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    S = _scores(rng, B, n, K, spread)
    G = focus.focus_sinkhorn(dev(S), tau, iters)
    torch.cuda.synchronize()
    ref = oracle.sinkhorn(S, tau, iters)
    check_G(host(G), ref, name)


def test_sinkhorn_unaligned_rows():
    """Scores and G that start 4 bytes off a 16-byte boundary (one score per
    lane instead of four) give the oracle's result too."""
    say("[sinkhorn] 4-byte aligned buffers")
    rng = np.random.default_rng(6)
    B, n, K = 1, 3000, 32
    S = _scores(rng, B, n, K, 1.0)
    buf = torch.empty(B * n * K + 1, dtype=torch.float32, device="cuda")
    out = torch.empty(B * n * K + 1, dtype=torch.float32, device="cuda")
    s_view = buf[1:].view(B, n, K)
    g_view = out[1:].view(B, n, K)
    s_view.copy_(dev(S))
    focus.focus_sinkhorn(s_view, 1.0, 6, G=g_view)
    torch.cuda.synchronize()
    check_G(host(g_view), oracle.sinkhorn(S, 1.0, 6), "unaligned")


def test_sinkhorn_is_deterministic_and_workspace_reusable():
    say("[sinkhorn] determinism")
    rng = np.random.default_rng(3)
    S = dev(_scores(rng, 2, 5000, 24, 1.0))
    ws = torch.empty(focus.focus_sinkhorn_workspace_bytes(2, 5000, 24, 7), dtype=torch.uint8,
                     device="cuda")
    a = focus.focus_sinkhorn(S, 0.9, 7, workspace=ws)
    b = focus.focus_sinkhorn(S, 0.9, 7, workspace=ws)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = focus.focus_sinkhorn(S, 0.9, 7, workspace=ws, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_assign_scores_match_oracle_and_argmax():
    say("[scores] ragged K = 7 and K = 40, with bias")
    rng = np.random.default_rng(4)
    for (B, n, d_model, d_proj, K) in [(2, 301, 96, 24, 7), (1, 500, 256, 64, 40)]:
        h = rng.standard_normal((B, n, d_model), dtype=np.float32)
        P = rng.standard_normal((d_model, d_proj), dtype=np.float32) / np.float32(np.sqrt(d_model))
        C = rng.standard_normal((K, d_proj), dtype=np.float32)
        bias = rng.standard_normal(K).astype(np.float32) * np.float32(0.2)
        S = focus.focus_assign_scores(dev(h), dev(P), dev(C), dev(bias))
        ids, _ = focus.focus_assign(dev(h), dev(P), dev(C), dev(bias))
        torch.cuda.synchronize()
        got = host(S)
        ref = oracle.assign_scores(h, P, C, bias)
        err = np.abs(got - ref)
        bound = score_error_bound(h, P, C)
        say(f"  K={K}: max-abs {err.max():.3e}, max err/bound {np.max(err / bound):.3f}")
        assert (err <= bound).all()
        # the same kernel arithmetic picks the ids: argmax of the scores
        srt = np.sort(got, axis=-1)
        clear = srt[..., -1] > srt[..., -2]
        assert np.array_equal(np.argmax(got, axis=-1)[clear], host(ids)[clear])


@pytest.mark.parametrize("wl,iters", [(workloads.GQA70B, 10), (workloads.LONG1M, 10)],
                         ids=lambda x: getattr(x, "name", str(x)))
def test_soft_assignment_full_size(wl, iters):
    """The measured configuration: scores of the workload's hidden states,
    then Sinkhorn with tau = 1, every value checked against the oracle."""
    say(f"[sinkhorn full] {wl.name}: drawing inputs")
    x = synth.make_inputs(wl, with_qkv=False)
    S = focus.focus_assign_scores(dev(x["hidden"]), dev(x["P"]), dev(x["C"]),
                                  None if x["bias"] is None else dev(x["bias"]))
    G = focus.focus_sinkhorn(S, 1.0, iters)
    torch.cuda.synchronize()
    s_host = host(S)
    rng = np.random.default_rng(5)
    tok = rng.integers(0, wl.B * wl.n, size=2048)
    ref_s = oracle.assign_scores(x["hidden"].reshape(-1, 1, wl.d_model)[tok], x["P"], x["C"],
                                 x["bias"])[:, 0]
    err = np.abs(s_host.reshape(-1, wl.K)[tok] - ref_s)
    bound = score_error_bound(x["hidden"].reshape(-1, wl.d_model)[tok], x["P"], x["C"])
    say(f"  scores on 2048 tokens: max-abs {err.max():.3e}, max err/bound {np.max(err / bound):.3f}")
    assert (err <= bound).all()
    check_G(host(G), oracle.sinkhorn(s_host, 1.0, iters), wl.name)
