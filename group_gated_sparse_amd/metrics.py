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


def attn_flops(pairs: int, Hq: int, d: int) -> float:
    return 4.0 * d * pairs * Hq
