"""Work counts used to turn measured times into throughput.

Visited pairs follow the Focus pair count (Japanese page "Focus: Learning
Which Attention Pairs Matter", technical summary §2.2: O(n^2/K + n*w) pairs
at inference): the causal window band plus same-group pairs further apart
than the window. Flops per visited pair = 4*d (2*d for q·k, 2*d for p·v);
exp/max/sum are not counted.
"""
import numpy as np

MI355X_BF16_DENSE_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz (no sparsity)
MI355X_HBM_GBPS = 8000.0


def window_pairs(n: int, w: int) -> int:
    """sum_i (min(i, w) + 1): pairs with 0 <= i - j <= w, per query head."""
    ww = min(w, n - 1)
    return n * (ww + 1) - ww * (ww + 1) // 2


def long_range_pairs(ids_row: np.ndarray, w: int) -> int:
    """Same-group pairs (i, j) with i - j > w in one sequence, per query head."""
    order = np.argsort(ids_row, kind="stable")
    g = ids_row[order]
    bounds = np.flatnonzero(np.diff(g)) + 1
    total = 0
    for seg in np.split(order, bounds):
        total += int(np.searchsorted(seg, seg - w, side="left").sum())
    return total


def pair_counts(ids: np.ndarray, w: int):
    """(window pairs, long-range pairs) summed over the batch, per query head."""
    B, n = ids.shape
    win = B * window_pairs(n, w)
    lr = sum(long_range_pairs(ids[b], w) for b in range(B))
    return win, lr


def long_range_pairs_multi(ids_tok: np.ndarray, w: int):
    """Top-m membership, one sequence (ids_tok [n][m], distinct groups per
    token): (kept far pairs, far pairs visited). A far pair is kept when the
    tokens share a group; the long-range pass visits every far pair inside
    each group's segment, so a pair sharing s groups is visited s times and
    kept once. For m <= 2, kept = visited - (far pairs whose tokens have the
    same two groups)."""
    n, m = ids_tok.shape
    if m > 2:
        raise ValueError("m <= 2")
    visited = 0
    for g in np.unique(ids_tok):
        seg = np.flatnonzero((ids_tok == g).any(axis=1))
        visited += int(np.searchsorted(seg, seg - w, side="left").sum())
    if m == 1:
        return visited, visited
    key = np.sort(ids_tok, axis=1).astype(np.int64)
    code = key[:, 0] * 1024 + key[:, 1]
    order = np.argsort(code, kind="stable")
    c = code[order]
    twice = 0
    for seg in np.split(order, np.flatnonzero(np.diff(c)) + 1):
        twice += int(np.searchsorted(seg, seg - w, side="left").sum())
    return visited - twice, visited


def pair_counts_multi(ids: np.ndarray, w: int):
    """(window pairs, kept long-range pairs, visited long-range pairs) over
    the batch, per query head; ids [B][n][m]."""
    B, n, _ = ids.shape
    win = B * window_pairs(n, w)
    kept = visited = 0
    for b in range(B):
        k, v = long_range_pairs_multi(ids[b], w)
        kept += k
        visited += v
    return win, kept, visited


def attn_flops(pairs: int, Hq: int, d: int) -> float:
    return 4.0 * d * pairs * Hq
