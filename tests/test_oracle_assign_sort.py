"""Pins of the assignment and grouping oracles.

Assignment: the Japanese page §2.1 projects h_i and compares it with the K
centroids in centroid space; §2.2 takes a hard top-k group at inference
(top-1 here). Grouping: a stable sort of tokens by group id.
"""
import numpy as np
import pytest

import oracle
from group_gated_sparse_amd import synth, workloads


def _inputs(rng, B, n, d_model, d_proj, K):
    h = rng.standard_normal((B, n, d_model), dtype=np.float32)
    P = rng.standard_normal((d_model, d_proj), dtype=np.float32) / np.float32(np.sqrt(d_model))
    C = rng.standard_normal((K, d_proj), dtype=np.float32)
    C /= np.linalg.norm(C, axis=1, keepdims=True)
    return h, P, C


def test_assign_matches_fp64_argmax_outside_tie_band():
    rng = np.random.default_rng(1)
    h, P, C = _inputs(rng, 2, 300, 96, 24, 9)
    bias = rng.standard_normal(9).astype(np.float32) * np.float32(0.3)
    ids, margin = oracle.assign(h, P, C, bias)
    s = (h.astype(np.float64) @ P.astype(np.float64)) @ C.astype(np.float64).T + bias
    srt = np.sort(s, axis=-1)
    m64 = srt[..., -1] - srt[..., -2]
    clear = m64 > 1e-3
    assert clear.mean() > 0.9
    assert np.array_equal(ids[clear], np.argmax(s, axis=-1)[clear])
    assert np.max(np.abs(margin - m64)) < 1e-4
    assert (margin >= 0).all()


def test_assign_is_equivariant_under_centroid_permutation():
    """Reordering the rows of C reorders the scores exactly, so ids follow."""
    rng = np.random.default_rng(2)
    h, P, C = _inputs(rng, 1, 200, 64, 16, 7)
    ids, margin = oracle.assign(h, P, C)
    pi = rng.permutation(7)
    ids2, margin2 = oracle.assign(h, P, C[pi])
    assert np.array_equal(pi[ids2], ids)
    assert np.array_equal(margin, margin2)


def test_assign_single_group_and_dominant_bias():
    rng = np.random.default_rng(3)
    h, P, C = _inputs(rng, 2, 50, 32, 8, 1)
    ids, margin = oracle.assign(h, P, C)
    assert (ids == 0).all() and np.isinf(margin).all()
    h, P, C = _inputs(rng, 1, 50, 32, 8, 5)
    bias = np.zeros(5, np.float32)
    bias[3] = 1e4
    ids, _ = oracle.assign(h, P, C, bias)
    assert (ids == 3).all()


def test_assign_exact_tie_takes_lowest_index():
    h = np.ones((1, 4, 2), np.float32)
    P = np.eye(2, dtype=np.float32)
    C = np.array([[0.0, 1.0], [1.0, 0.0], [0.6, 0.8], [0.0, 1.0]], np.float32)
    # scores: 1, 1, 1.4, 1 for every token -> group 2; tie 0 vs 1 vs 3 below it
    ids, margin = oracle.assign(h, P, C)
    assert (ids == 2).all()
    ids, margin = oracle.assign(h, P, C[[0, 1, 3]])
    assert (ids == 0).all() and (margin == 0).all()


def test_assign_token_subset_matches_full():
    rng = np.random.default_rng(4)
    h, P, C = _inputs(rng, 3, 40, 32, 8, 6)
    full, fm = oracle.assign(h, P, C)
    toks = rng.choice(120, size=30, replace=False)
    sub, sm = oracle.assign(h, P, C, tokens=toks)
    assert np.array_equal(sub, full.ravel()[toks]) and np.array_equal(sm, fm.ravel()[toks])


@pytest.mark.parametrize("B,n,K", [(1, 1, 1), (1, 5, 9), (3, 100, 4), (2, 1000, 64), (1, 77, 1)])
def test_sort_matches_stable_argsort(B, n, K):
    rng = np.random.default_rng(B * 1000 + n + K)
    ids = rng.integers(0, K, size=(B, n), dtype=np.int32)
    if n > 10:
        ids[:, : n // 3] = ids[:, :1]  # long runs of one group
    perm, off = oracle.group_sort(ids, K)
    for b in range(B):
        assert np.array_equal(perm[b], np.argsort(ids[b], kind="stable"))
        cnt = np.bincount(ids[b], minlength=K)
        assert np.array_equal(off[b], np.concatenate([[0], np.cumsum(cnt)]))
        assert (np.diff(ids[b][perm[b]]) >= 0).all()
        for g in range(K):
            seg = perm[b, off[b, g]:off[b, g + 1]]
            assert (np.diff(seg) > 0).all() and (ids[b, seg] == g).all()


def test_sort_rejects_ids_outside_range():
    with pytest.raises(ValueError):
        oracle.group_sort(np.array([[0, 4, 1]], np.int32), 4)


def test_tiny_workload_assign_is_deterministic_and_balanced():
    wl = workloads.TINY
    x = synth.make_inputs(wl)
    ids, _ = oracle.assign(x["hidden"], x["P"], x["C"], x["bias"])
    cnt = np.bincount(ids.ravel(), minlength=wl.K)
    assert cnt.sum() == wl.n and (cnt > 0).all()
    y = synth.make_inputs(wl)
    assert synth.digest(x) == synth.digest(y)
