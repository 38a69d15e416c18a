"""Pins of the multi-membership oracle (each token in its top-m groups).

The Korean page §2.3 and the Japanese page §2.2 let a token join its top-k
groups at inference (the Korean page §3.4 and the Japanese page §3.3 use
k = 2 with K = 4); a far pair is kept when the two tokens share any group,
and each kept pair enters the softmax once. Each pin below targets a
plausible mistake: a pair shared through two groups counted twice, the
second group ignored, the wrong order or tie rule of the top-m choice, the
margin taken between the wrong ranks.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
from test_oracle_attn import _qkv, _sdpa_causal


def _inputs(rng, B, n, d_model, d_proj, K):
    h = rng.standard_normal((B, n, d_model), dtype=np.float32)
    P = rng.standard_normal((d_model, d_proj), dtype=np.float32) / np.float32(np.sqrt(d_model))
    C = rng.standard_normal((K, d_proj), dtype=np.float32)
    C /= np.linalg.norm(C, axis=1, keepdims=True)
    return h, P, C


def test_topk_matches_fp64_ranking_outside_tie_band():
    rng = np.random.default_rng(21)
    h, P, C = _inputs(rng, 2, 300, 96, 24, 9)
    bias = rng.standard_normal(9).astype(np.float32) * np.float32(0.3)
    ids, margin = oracle.assign_topk(h, P, C, 3, bias)
    s = (h.astype(np.float64) @ P.astype(np.float64)) @ C.astype(np.float64).T + bias
    order = np.argsort(-s, axis=-1, kind="stable")
    srt = np.take_along_axis(s, order, axis=-1)
    gaps = srt[..., :-1] - srt[..., 1:]            # gaps[r] = s_(r+1) - s_(r+2)
    clear = (gaps[..., :3] > 1e-3).all(axis=-1)
    assert clear.mean() > 0.8
    assert np.array_equal(ids[clear], order[..., :3][clear])
    assert np.max(np.abs(margin - gaps[..., 2])) < 1e-4
    assert (margin >= 0).all()


def test_topk_first_choice_is_top1_and_m1_is_top1():
    rng = np.random.default_rng(22)
    h, P, C = _inputs(rng, 1, 120, 32, 8, 6)
    ids1, m1 = oracle.assign(h, P, C)
    idk, mk = oracle.assign_topk(h, P, C, 1)
    assert np.array_equal(idk[..., 0], ids1) and np.array_equal(mk, m1)
    id2, _ = oracle.assign_topk(h, P, C, 2)
    assert np.array_equal(id2[..., 0], ids1)
    assert (id2[..., 0] != id2[..., 1]).all()


def test_topk_exact_ties_take_lowest_index_and_m_equals_K():
    h = np.ones((1, 3, 2), np.float32)
    P = np.eye(2, dtype=np.float32)
    C = np.array([[0.0, 1.0], [1.0, 0.0], [0.6, 0.8], [0.0, 1.0]], np.float32)
    # scores 1, 1, 1.4, 1: group 2 first, then the tie 0 / 1 / 3 in index order
    ids, margin = oracle.assign_topk(h, P, C, 2)
    assert (ids == np.array([2, 0])).all() and (margin == 0).all()
    ids, margin = oracle.assign_topk(h, P, C, 4)
    assert (ids == np.array([2, 0, 1, 3])).all() and np.isinf(margin).all()


def test_multi_sort_is_stable_sort_of_entries():
    rng = np.random.default_rng(23)
    B, n, m, K = 2, 300, 2, 5
    ids = np.stack([np.stack([rng.choice(K, size=m, replace=False) for _ in range(n)])
                    for _ in range(B)]).astype(np.int32)
    perm, off = oracle.group_sort_multi(ids, K)
    flat = ids.reshape(B, n * m)
    for b in range(B):
        assert np.array_equal(perm[b], np.argsort(flat[b], kind="stable"))
        for g in range(K):
            seg = perm[b, off[b, g]:off[b, g + 1]]
            assert (flat[b, seg] == g).all()
            assert (np.diff(seg // m) > 0).all()        # one entry per token, positions increase
    assert (off[:, -1] == n * m).all()


def test_single_membership_equals_top1_pattern():
    rng = np.random.default_rng(24)
    q, k, v = _qkv(rng, 2, 4, 2, 90, 8)
    ids = rng.integers(0, 5, size=(2, 90), dtype=np.int32)
    a, la, va = oracle.attn(q, k, v, ids, 6, 0.3)
    b, lb, vb = oracle.attn_multi(q, k, v, ids[..., None], 6, 0.3)
    assert np.array_equal(a, b) and np.array_equal(la, lb) and np.array_equal(va, vb)


@pytest.mark.parametrize("w", [0, 5])
def test_all_groups_is_dense_causal(w):
    """m = K: every pair shares every group, so the pattern is full causal
    attention (torch's fp64 SDPA), and no pair is counted more than once."""
    rng = np.random.default_rng(25 + w)
    q, k, v = _qkv(rng, 1, 4, 2, 64, 16)
    ids = np.stack([rng.permutation(3) for _ in range(64)])[None].astype(np.int32)
    out, lse, vis = oracle.attn_multi(q, k, v, ids, w, 0.25)
    ref = _sdpa_causal(q, k, v, 0.25)
    assert np.max(np.abs(out - ref)) < 1e-12
    assert (vis == (np.arange(64) + 1)[None, None, :]).all()


CASES = [
    # (n, d, Hq, Hkv, K, m, w, seed)
    (1, 4, 1, 1, 2, 2, 0, 1),
    (13, 4, 2, 1, 4, 2, 0, 2),
    (24, 8, 2, 2, 4, 2, 2, 3),
    (31, 4, 3, 1, 6, 3, 4, 4),
    (40, 4, 1, 1, 5, 2, 1, 5),
]


@pytest.mark.parametrize("n,d,Hq,Hkv,K,m,w,seed", CASES)
def test_brute_force_set_enumeration(n, d, Hq, Hkv, K, m, w, seed):
    rng = np.random.default_rng(200 + seed)
    q, k, v = _qkv(rng, 1, Hq, Hkv, n, d)
    ids = np.stack([rng.choice(K, size=m, replace=False) for _ in range(n)])[None].astype(np.int32)
    out, _, vis = oracle.attn_multi(q, k, v, ids, w, 1.0 / math.sqrt(d))
    bout, bcnt = brute.attention_sets(q[0].tolist(), k[0].tolist(), v[0].tolist(),
                                      ids[0].tolist(), w, 1.0 / math.sqrt(d))
    assert np.max(np.abs(out[0] - np.array(bout))) < 1e-12
    assert (vis[0] == np.array(bcnt)).all()


def _far_pairs(pos, w):
    """Pairs (i, j) of a position-sorted list with i - j > w."""
    return int(np.searchsorted(pos, pos - w, side="left").sum())


@pytest.mark.parametrize("n,w,K", [(64, 0, 4), (300, 11, 4), (257, 20, 6), (200, 199, 4)])
def test_pair_count_inclusion_exclusion(n, w, K):
    """m = 2: kept pairs = window band + far pairs sharing a group, where a
    pair sharing both groups (same group set) is subtracted once (inclusion-
    exclusion), checked against the row counts of the attention oracle."""
    rng = np.random.default_rng(n + 7 * w)
    ids = np.stack([rng.choice(K, size=2, replace=False) for _ in range(n)])[None].astype(np.int32)
    ww = min(w, n - 1)
    band = n * (ww + 1) - ww * (ww + 1) // 2
    far = 0
    for g in range(K):
        far += _far_pairs(np.nonzero((ids[0] == g).any(axis=1))[0], w)
    key = np.sort(ids[0], axis=1)
    for a in range(K):
        for c in range(a + 1, K):
            far -= _far_pairs(np.nonzero((key[:, 0] == a) & (key[:, 1] == c))[0], w)
    q, k, v = _qkv(rng, 1, 1, 1, n, 4)
    _, _, vis = oracle.attn_multi(q, k, v, ids, w, 1.0)
    assert int(vis.sum()) == band + far
    assert oracle.pair_count_multi(ids, w) == band + far
