"""Pins of the Sinkhorn soft-assignment oracle (training-time step).

The Korean page §2.2 and the Japanese page §2.1 / §2.3 make the n x K
token-to-group assignment matrix doubly stochastic with Sinkhorn
normalisation: every token's row sums to 1 and every group receives the
same total, n / K. Each pin targets a plausible mistake: the wrong axis or
target of a normalisation, the temperature dropped, the last scaling not
applied, the first row step skipped.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _scores(rng, B, n, K, spread=1.0):
    return (rng.standard_normal((B, n, K)) * spread).astype(np.float32)


def test_zero_iterations_is_row_softmax():
    """Rows first: with no column step, G is the softmax of scores / tau
    over the groups (scipy)."""
    rng = np.random.default_rng(1)
    S = _scores(rng, 2, 50, 7, 2.0)
    G = oracle.sinkhorn(S, 0.7, 0)
    assert np.max(np.abs(G - softmax(S.astype(np.float64) / 0.7, axis=-1))) < 1e-14


def test_additive_scores_give_uniform_assignment():
    """scores[t][k] = a_t + b_k: A is an outer product, the column step makes
    every column equal, and the next row step gives exactly 1/K."""
    rng = np.random.default_rng(2)
    a = rng.integers(-40, 40, size=40) / 16.0      # on a grid: the sums are exact in fp32
    b = rng.integers(-40, 40, size=5) / 8.0
    S = (a[:, None] + b[None, :]).astype(np.float32)[None]
    for it in (1, 4):
        G = oracle.sinkhorn(S, 1.0, it)
        assert np.max(np.abs(G - 0.2)) < 1e-12


def test_two_by_two_limit_closed_form():
    """n = K = 2 (column target 1): diagonal scalings keep the cross ratio
    a11 a22 / (a12 a21), so the doubly stochastic limit is [[p, 1-p], [1-p, p]]
    with p / (1 - p) = sqrt(a11 a22 / (a12 a21))."""
    S = np.array([[[0.3, -1.1], [0.8, 0.25]]], np.float32)
    A = np.exp(S[0].astype(np.float64) / 0.5)
    r = np.sqrt(A[0, 0] * A[1, 1] / (A[0, 1] * A[1, 0]))
    p = r / (1 + r)
    G = oracle.sinkhorn(S, 0.5, 200)[0]
    assert np.max(np.abs(G - np.array([[p, 1 - p], [1 - p, p]]))) < 1e-12


def test_cross_ratios_are_those_of_exp_scores():
    """Every Sinkhorn step is a diagonal scaling of A = exp(S / tau), so all
    cross ratios G_ik G_jl / (G_il G_jk) stay exp((S_ik + S_jl - S_il - S_jk) / tau)."""
    rng = np.random.default_rng(3)
    S = _scores(rng, 1, 30, 6)
    tau = 0.8
    G = oracle.sinkhorn(S, tau, 5)[0]
    S64 = S[0].astype(np.float64)
    for (i, j, k, l) in [(0, 1, 0, 1), (3, 17, 2, 5), (29, 4, 5, 0)]:
        got = G[i, k] * G[j, l] / (G[i, l] * G[j, k])
        want = np.exp((S64[i, k] + S64[j, l] - S64[i, l] - S64[j, k]) / tau)
        assert abs(got / want - 1) < 1e-12


def test_marginals_rows_exact_columns_converge():
    rng = np.random.default_rng(4)
    n, K = 300, 8
    S = _scores(rng, 2, n, K, 1.5)
    errs = []
    for it in (1, 3, 10, 60):
        G = oracle.sinkhorn(S, 1.0, it)
        assert np.max(np.abs(G.sum(-1) - 1)) < 1e-12
        errs.append(np.max(np.abs(G.sum(1) - n / K)))
    assert errs[-1] < 1e-9 and errs[0] > errs[-1]
    assert all(errs[i + 1] <= errs[i] for i in range(len(errs) - 1))


def test_row_shift_and_column_permutation():
    """Adding a constant to a row of scores changes nothing (rows are
    normalised first); permuting the groups permutes the columns."""
    rng = np.random.default_rng(5)
    S = (rng.integers(-96, 96, size=(1, 64, 6)) / 64.0).astype(np.float32)   # grid values
    G = oracle.sinkhorn(S, 1.0, 4)
    shift = np.round(rng.standard_normal((1, 64, 1)) * 4).astype(np.float32)   # sums exact in fp32
    assert np.max(np.abs(oracle.sinkhorn(S + shift, 1.0, 4) - G)) < 1e-12
    pi = rng.permutation(6)
    assert np.max(np.abs(oracle.sinkhorn(S[..., pi], 1.0, 4) - G[..., pi])) < 1e-14


def test_assign_scores_match_fp64_and_argmax():
    rng = np.random.default_rng(6)
    h = rng.standard_normal((2, 120, 48)).astype(np.float32)
    P = (rng.standard_normal((48, 16)) / np.sqrt(48)).astype(np.float32)
    C = rng.standard_normal((9, 16)).astype(np.float32)
    bias = rng.standard_normal(9).astype(np.float32)
    S = oracle.assign_scores(h, P, C, bias)
    ref = (h.astype(np.float64) @ P.astype(np.float64)) @ C.astype(np.float64).T + bias
    assert np.max(np.abs(S - ref)) < 1e-4
    ids, _ = oracle.assign(h, P, C, bias)
    assert np.array_equal(np.argmax(S, axis=-1), ids)
