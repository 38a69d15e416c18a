"""Pins of the attention oracle against things other than itself.

Each pin targets a plausible mistake: the causal bound, the window bound,
the same-group test, the GQA head map, the softmax normalisation and the
two-part split of the Korean page §2.3 (window part + intra-group long-range
part, joined by log-sum-exp).
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import brute
from group_gated_sparse_amd import synth


def _qkv(rng, B, Hq, Hkv, n, d, qscale=1.0):
    q = synth.bf16_bits(rng.standard_normal((B, Hq, n, d), dtype=np.float32) * np.float32(qscale))
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    return q, k, v


def _f64(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


def _sdpa_causal(q, k, v, scale):
    """torch's fp64 scaled_dot_product_attention with a causal mask (library routine)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(_f64(q))
    kt = torch.from_numpy(_f64(k)).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(_f64(v)).repeat_interleave(Hq // Hkv, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return out.numpy()


@pytest.mark.parametrize("w", [0, 3, 17])
def test_single_group_is_dense_causal(w):
    """K = 1: every earlier token shares the group, so the pattern is full causal."""
    rng = np.random.default_rng(11 + w)
    q, k, v = _qkv(rng, 2, 4, 2, 70, 16)
    ids = np.zeros((2, 70), np.int32)
    out, lse, vis = oracle.attn(q, k, v, ids, w, 0.25)
    ref = _sdpa_causal(q, k, v, 0.25)
    assert np.max(np.abs(out - ref)) < 1e-12
    i = np.arange(70)
    assert (vis == (i + 1)[None, None, :]).all()


def test_wide_window_is_dense_causal():
    """w >= n-1: the window alone covers every causal pair, whatever the groups."""
    rng = np.random.default_rng(5)
    q, k, v = _qkv(rng, 1, 3, 3, 45, 8)
    ids = rng.integers(0, 5, size=(1, 45), dtype=np.int32)
    for w in (44, 200):
        out, lse, _ = oracle.attn(q, k, v, ids, w, 0.5)
        assert np.max(np.abs(out - _sdpa_causal(q, k, v, 0.5))) < 1e-12


def test_lse_is_log_sum_exp_over_allowed_scores():
    rng = np.random.default_rng(6)
    n, d, w = 40, 8, 4
    q, k, v = _qkv(rng, 1, 2, 1, n, d)
    ids = rng.integers(0, 3, size=(1, n), dtype=np.int32)
    _, lse, _ = oracle.attn(q, k, v, ids, w, 0.3)
    s = 0.3 * np.einsum("hid,jd->hij", _f64(q)[0], _f64(k)[0, 0])
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    keep = (j <= i) & ((i - j <= w) | (ids[0][:, None] == ids[0][None, :]))
    ref = logsumexp(np.where(keep[None], s, -np.inf), axis=2)
    assert np.max(np.abs(lse[0] - ref)) < 1e-12


def test_window_zero_is_causal_attention_within_each_group():
    """w = 0 leaves only same-group causal pairs: run textbook causal attention
    on each group's gathered subsequence."""
    rng = np.random.default_rng(7)
    n, d = 60, 16
    q, k, v = _qkv(rng, 1, 2, 2, n, d)
    ids = rng.integers(0, 4, size=(1, n), dtype=np.int32)
    out, _, _ = oracle.attn(q, k, v, ids, 0, 0.25)
    ref = np.zeros_like(out)
    for g in range(4):
        pos = np.nonzero(ids[0] == g)[0]
        if pos.size == 0:
            continue
        ref[:, :, pos] = _sdpa_causal(q[:, :, pos], k[:, :, pos], v[:, :, pos], 0.25)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_distinct_groups_and_no_window_returns_v():
    """Each token alone in its group and w = 0: the only kept pair is (i, i)."""
    rng = np.random.default_rng(8)
    n, d = 12, 8
    q, k, v = _qkv(rng, 1, 2, 1, n, d)
    ids = rng.permutation(20)[:n].astype(np.int32)[None]
    out, lse, vis = oracle.attn(q, k, v, ids, 0, 1.0)
    assert (vis == 1).all()
    assert np.array_equal(out[0, 0], _f64(v)[0, 0]) and np.array_equal(out[0, 1], _f64(v)[0, 0])


def test_row_zero_returns_v0():
    rng = np.random.default_rng(9)
    q, k, v = _qkv(rng, 2, 2, 2, 30, 8)
    ids = rng.integers(0, 3, size=(2, 30), dtype=np.int32)
    out, _, _ = oracle.attn(q, k, v, ids, 5, 0.7)
    assert np.array_equal(out[:, :, 0], _f64(v)[:, :, 0])


CASES = [
    # (n, d, Hq, Hkv, K, w, seed)
    (1, 4, 1, 1, 1, 0, 1),
    (2, 4, 2, 1, 3, 0, 2),
    (9, 4, 2, 2, 12, 0, 3),     # K > n: empty groups
    (17, 8, 2, 1, 3, 1, 4),
    (23, 4, 3, 3, 5, 3, 5),
    (31, 8, 4, 2, 2, 7, 6),
    (40, 4, 2, 2, 6, 40, 7),    # w >= n
    (48, 4, 1, 1, 4, 2, 8),
]


@pytest.mark.parametrize("n,d,Hq,Hkv,K,w,seed", CASES)
def test_brute_force_pair_enumeration(n, d, Hq, Hkv, K, w, seed):
    rng = np.random.default_rng(100 + seed)
    q, k, v = _qkv(rng, 1, Hq, Hkv, n, d)
    ids = rng.integers(0, K, size=(1, n), dtype=np.int32)
    out, _, vis = oracle.attn(q, k, v, ids, w, 1.0 / math.sqrt(d))
    bout, bw = brute.attention(q[0].tolist(), k[0].tolist(), v[0].tolist(), ids[0].tolist(),
                               w, 1.0 / math.sqrt(d))
    assert np.max(np.abs(out[0] - np.array(bout))) < 1e-12
    bw = np.array(bw)
    assert (vis[0] == (bw > 0).sum(axis=2)).all()
    for h in range(Hq):
        for i in range(n):
            wt = oracle.attn_weights(q, k, ids, w, 1.0 / math.sqrt(d), 0, h, i)
            assert np.max(np.abs(wt - bw[h, i])) < 1e-12


def test_weights_sum_to_one_and_vanish_outside_the_pattern():
    rng = np.random.default_rng(12)
    n, d, w = 50, 8, 3
    q, k, v = _qkv(rng, 1, 2, 1, n, d, qscale=3.0)
    ids = rng.integers(0, 4, size=(1, n), dtype=np.int32)
    for h in range(2):
        for i in range(n):
            wt = oracle.attn_weights(q, k, ids, w, 1.0, 0, h, i)
            allowed = np.array([j <= i and (i - j <= w or ids[0, j] == ids[0, i])
                                for j in range(n)])
            assert abs(wt.sum() - 1.0) < 1e-12
            assert (wt[~allowed] == 0.0).all()
            assert (wt[allowed] > 0.0).all()


def test_group_label_bijection_leaves_output_unchanged():
    rng = np.random.default_rng(13)
    q, k, v = _qkv(rng, 2, 2, 2, 64, 8)
    ids = rng.integers(0, 6, size=(2, 64), dtype=np.int32)
    relabel = rng.permutation(6).astype(np.int32)
    a, la, _ = oracle.attn(q, k, v, ids, 4, 0.4)
    b, lb, _ = oracle.attn(q, k, v, relabel[ids], 4, 0.4)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_two_part_split_matches_single_softmax():
    """Korean page §2.3 splits the pattern into a local-window part and an
    intra-group long-range part; the log-sum-exp merge of the two must equal
    the single softmax over their union."""
    rng = np.random.default_rng(14)
    q, k, v = _qkv(rng, 2, 4, 2, 150, 16)
    ids = rng.integers(0, 5, size=(2, 150), dtype=np.int32)
    for w in (0, 7, 31, 149):
        a, la, _ = oracle.attn(q, k, v, ids, w, 0.25)
        b, lb = oracle.attn_two_phase(q, k, v, ids, w, 0.25)
        assert np.max(np.abs(a - b)) < 1e-12 and np.max(np.abs(la - lb)) < 1e-12


def test_gqa_head_map_equals_repeated_kv():
    """q head h reads kv head h // (Hq/Hkv): same as MHA with k, v repeated."""
    rng = np.random.default_rng(15)
    q, k, v = _qkv(rng, 1, 6, 2, 40, 8)
    ids = rng.integers(0, 3, size=(1, 40), dtype=np.int32)
    a, _, _ = oracle.attn(q, k, v, ids, 5, 0.3)
    b, _, _ = oracle.attn(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), ids, 5, 0.3)
    assert np.array_equal(a, b)


def test_row_subset_matches_full_run():
    rng = np.random.default_rng(16)
    q, k, v = _qkv(rng, 2, 3, 1, 33, 8)
    ids = rng.integers(0, 4, size=(2, 33), dtype=np.int32)
    full, lse, vis = oracle.attn(q, k, v, ids, 2, 0.5)
    rows = rng.choice(2 * 3 * 33, size=25, replace=False)
    sub, slse, svis = oracle.attn(q, k, v, ids, 2, 0.5, rows=rows)
    assert np.array_equal(sub, full.reshape(-1, 8)[rows])
    assert np.array_equal(slse, lse.ravel()[rows]) and np.array_equal(svis, vis.ravel()[rows])


def _long_range_pairs(ids_row, w):
    """Same-group pairs with i - j > w, counted group by group with a sorted search."""
    total = 0
    for g in np.unique(ids_row):
        pos = np.nonzero(ids_row == g)[0]
        total += int(np.searchsorted(pos, pos - w, side="left").sum())
    return total


@pytest.mark.parametrize("n,w,K", [(1, 0, 1), (64, 0, 3), (200, 13, 7), (300, 299, 4), (257, 400, 2)])
def test_visited_pairs_closed_form(n, w, K):
    """|A_i| summed = window band n(w+1) - w(w+1)/2 (w < n) plus same-group
    pairs further than w apart (Japanese page §2.2's n*w and n^2/K terms)."""
    rng = np.random.default_rng(n + w)
    ids = rng.integers(0, K, size=(1, n), dtype=np.int32)
    q, k, v = _qkv(rng, 1, 1, 1, n, 4)
    _, _, vis = oracle.attn(q, k, v, ids, w, 1.0)
    ww = min(w, n - 1)
    band = n * (ww + 1) - ww * (ww + 1) // 2
    assert int(vis.sum()) == band + _long_range_pairs(ids[0], w)
    assert oracle.pair_count(ids, w) == int(vis.sum())
    if K == 1:
        assert int(vis.sum()) == n * (n + 1) // 2
