"""Pins of the training-time soft-gated attention oracle.

Reading (Japanese page §2.1-§2.2, Korean page §2.1): every causal pair is
computed; pairs inside the window keep their plain weight, pairs further
apart are weighted by sigmoid(lambda * g_i . g_j), the group affinity of the
two tokens' soft assignments, and the softmax is renormalised over the
weighted pairs. Pins: special cases that reduce to torch's fp64
scaled_dot_product_attention with an additive mask built from the window
alone (the gate constant), brute force in pure Python, and the GQA map.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from test_oracle_attn import _f64, _qkv, _sdpa_causal


def _soft(rng, B, n, K, sharp=2.0):
    x = rng.standard_normal((B, n, K)) * sharp
    e = np.exp(x - x.max(-1, keepdims=True))
    return (e / e.sum(-1, keepdims=True)).astype(np.float32)


def _sdpa_far_bias(q, k, v, scale, w, bias):
    """torch fp64 SDPA, causal, with `bias` added to the logits of pairs
    further apart than w (bias: scalar or [B][n][n])."""
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    i = np.arange(n)
    far = (i[:, None] - i[None, :]) > w
    causal = i[None, :] <= i[:, None]
    mask = np.where(causal, 0.0, -np.inf) + np.where(far, 1.0, 0.0) * bias
    mask = np.array(np.broadcast_to(mask, (B, n, n))[:, None])
    qt = torch.from_numpy(_f64(q))
    kt = torch.from_numpy(_f64(k)).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(_f64(v)).repeat_interleave(Hq // Hkv, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(np.ascontiguousarray(mask)), scale=scale)
    return out.numpy()


def test_wide_window_is_causal_attention():
    rng = np.random.default_rng(31)
    q, k, v = _qkv(rng, 1, 4, 2, 60, 16)
    G = _soft(rng, 1, 60, 5)
    out, _ = oracle.soft_gate_attn(q, k, v, G, 59, 0.25, 7.0)
    assert np.max(np.abs(out - _sdpa_causal(q, k, v, 0.25))) < 1e-12


def test_zero_lambda_halves_far_pairs():
    """lambda = 0: sigmoid(0) = 1/2 on every far pair, whatever G."""
    rng = np.random.default_rng(32)
    q, k, v = _qkv(rng, 2, 2, 1, 70, 8)
    G = _soft(rng, 2, 70, 4)
    out, _ = oracle.soft_gate_attn(q, k, v, G, 5, 0.3, 0.0)
    ref = _sdpa_far_bias(q, k, v, 0.3, 5, math.log(0.5))
    assert np.max(np.abs(out - ref)) < 1e-12


@pytest.mark.parametrize("K,lam", [(4, 3.0), (16, -20.0)])
def test_uniform_assignment_gives_a_constant_gate(K, lam):
    """Uniform soft assignments: every affinity is 1/K, so far pairs get the
    constant gate sigmoid(lambda / K)."""
    rng = np.random.default_rng(33 + K)
    q, k, v = _qkv(rng, 1, 2, 2, 50, 8)
    G = np.full((1, 50, K), 1.0 / K, np.float32)
    out, lse = oracle.soft_gate_attn(q, k, v, G, 3, 0.5, lam)
    gate = 1.0 / (1.0 + math.exp(-lam * float(np.float32(1.0 / K)) ** 2 * K))
    ref = _sdpa_far_bias(q, k, v, 0.5, 3, math.log(gate))
    assert np.max(np.abs(out - ref)) < 1e-12


def test_general_gate_against_sdpa_with_affinity_bias():
    rng = np.random.default_rng(34)
    q, k, v = _qkv(rng, 1, 3, 1, 40, 8)
    G = _soft(rng, 1, 40, 6)
    lam = 4.0
    aff = G[0].astype(np.float64) @ G[0].astype(np.float64).T
    bias = -np.log1p(np.exp(-lam * aff))          # log sigmoid
    out, _ = oracle.soft_gate_attn(q, k, v, G, 2, 0.35, lam)
    ref = _sdpa_far_bias(q, k, v, 0.35, 2, bias[None])
    assert np.max(np.abs(out - ref)) < 1e-12


@pytest.mark.parametrize("n,w,lam,seed", [(1, 0, 1.0, 1), (9, 0, 5.0, 2), (17, 3, -2.0, 3),
                                          (24, 5, 12.0, 4)])
def test_brute_force(n, w, lam, seed):
    rng = np.random.default_rng(300 + seed)
    q, k, v = _qkv(rng, 1, 2, 1, n, 4)
    G = _soft(rng, 1, n, 3)
    out, _ = oracle.soft_gate_attn(q, k, v, G, w, 0.5, lam)
    ref = brute.soft_gate_attention(q[0].tolist(), k[0].tolist(), v[0].tolist(),
                                    G[0].astype(np.float64).tolist(), w, 0.5, lam)
    assert np.max(np.abs(out[0] - np.array(ref))) < 1e-12


def test_gqa_map_and_lse():
    rng = np.random.default_rng(35)
    q, k, v = _qkv(rng, 1, 6, 2, 30, 8)
    G = _soft(rng, 1, 30, 4)
    a, la = oracle.soft_gate_attn(q, k, v, G, 4, 0.3, 2.0)
    b, lb = oracle.soft_gate_attn(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), G, 4,
                                  0.3, 2.0)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    # lse: log of the gated weight sum (window part only at w >= n - 1)
    _, lw = oracle.soft_gate_attn(q, k, v, G, 29, 0.3, 2.0)
    qf, kf = _f64(q)[0, 0], _f64(k)[0, 0]
    s = 0.3 * qf @ kf.T
    i = 7
    assert abs(lw[0, 0, i] - np.log(np.exp(s[i, :i + 1]).sum())) < 1e-12
