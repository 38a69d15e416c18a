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


# ---- Computed pairs: the (query, key) products the attention kernels' MFMAs
# ---- actually form, masked ones included, to separate masking waste from
# ---- kernel speed. They follow the kernels' tiling: a workgroup takes TT
# ---- tokens x G query heads (G = the largest of 8, 4, 2, 1 dividing Hq/Hkv,
# ---- TT = 128 / G) and visits key tiles of BN keys (32 for d = 64 and 128,
# ---- 64 for d = 32).

def heads_per_workgroup(Hq: int, Hkv: int) -> int:
    hpk = Hq // Hkv
    for g in (8, 4, 2, 1):
        if hpk % g == 0:
            return g
    return 1


def tile_keys(d: int) -> int:
    return 64 if d == 32 else 32


def window_computed_pairs(n: int, w: int, TT: int, BN: int) -> int:
    """Per query head: key tiles of [max(0, q0 - w), last query] for every
    tile of TT tokens, times TT rows."""
    q0 = np.arange(0, n, TT, dtype=np.int64)
    kend = np.minimum(n, q0 + TT)
    kstart = np.maximum(0, q0 - w)
    ntl = (kend - kstart + BN - 1) // BN
    return int(ntl.sum()) * BN * TT


def long_range_computed_pairs(ids: np.ndarray, perm: np.ndarray, offsets: np.ndarray, w: int,
                              TT: int, BN: int) -> int:
    """One group per token. Per query head, summed over the batch: for each
    tile of TT sorted tokens and each group g among them, the key tiles of
    g's segment below the first slot whose position is >= (largest query
    position of g in the tile) - w, times TT rows. ids [B][n], perm [B][n]
    positions, offsets [B][K+1]."""
    B, ne = perm.shape
    total = 0
    for b in range(B):
        pb, ob_, ib = perm[b].astype(np.int64), offsets[b].astype(np.int64), ids[b]
        for s0 in range(0, ne, TT):
            s1 = min(ne, s0 + TT)
            gf, gl = int(ib[pb[s0]]), int(ib[pb[s1 - 1]])
            for g in range(gf, gl + 1):
                ob, oe = int(ob_[g]), int(ob_[g + 1])
                qlo, qhi = max(s0, ob), min(s1, oe)
                if qlo >= qhi:
                    continue
                maxpos = int(pb[qhi - 1])
                kend = ob + int(np.searchsorted(pb[ob:qhi], maxpos - w, side="left"))
                total += (kend - ob + BN - 1) // BN
    return total * BN * TT


def entry_long_range_computed_pairs(ids: np.ndarray, perm: np.ndarray, offsets: np.ndarray,
                                    w: int, TT: int, BN: int) -> int:
    """Two groups per token, the entry passes (K >= 5). Keys: the n*2
    membership entries e = t*2 + c sorted by group (perm [B][2n], offsets
    [B][K+1]; ids [B][2n] flat). Queries: for c = 0, 1 the entries of
    membership index c in key order, cut into tiles of TT; for each tile and
    each group g among its rows, the key tiles of g's segment below the first
    slot whose position is >= (largest position of the tile's rows of g) - w.
    Per query head, summed over the batch, times TT rows."""
    B, ne = perm.shape
    total = 0
    for b in range(B):
        pb, ob_, ib = perm[b].astype(np.int64), offsets[b].astype(np.int64), ids[b]
        for c in (0, 1):
            q = pb[(pb & 1) == c]
            for s0 in range(0, len(q), TT):
                rows = q[s0:s0 + TT]
                grp = ib[rows]
                for g in range(int(grp[0]), int(grp[-1]) + 1):
                    mine = rows[grp == g]
                    if len(mine) == 0:
                        continue
                    ob, oe = int(ob_[g]), int(ob_[g + 1])
                    bound = 2 * (int(mine[-1]) // 2 - w)
                    kend = ob + int(np.searchsorted(pb[ob:oe], bound, side="left"))
                    total += (kend - ob + BN - 1) // BN
    return total * BN * TT


def uses_set_pass(K: int, m: int) -> bool:
    """Two groups per token with K <= 4: the long-range pass runs over the
    tokens sorted by membership set (each kept pair visited once)."""
    return m == 2 and K <= 4


def set_long_range_computed_pairs(ids: np.ndarray, K: int, w: int, TT: int, BN: int) -> int:
    """Per query head, summed over the batch, for the set pass (ids
    [B][n][2]): tokens stably sorted by the index of their group pair; for
    each tile of TT sorted tokens and each set sharing a group with some
    token of the tile, the key tiles of that set's segment below the first
    slot whose position is >= (largest position in the tile) - w, times TT."""
    B, n, _ = ids.shape
    pairs = [(a, b) for a in range(K) for b in range(a + 1, K)]
    code = {p: i for i, p in enumerate(pairs)}
    masks = np.array([(1 << a) | (1 << b) for a, b in pairs], dtype=np.int64)
    total = 0
    for bb in range(B):
        lo = np.minimum(ids[bb, :, 0], ids[bb, :, 1])
        hi = np.maximum(ids[bb, :, 0], ids[bb, :, 1])
        sid = np.array([code[(int(x), int(y))] for x, y in zip(lo, hi)], dtype=np.int64)
        perm = np.argsort(sid, kind="stable")
        offs = np.concatenate([[0], np.cumsum(np.bincount(sid, minlength=len(pairs)))])
        tmask = masks[sid]
        for s0 in range(0, n, TT):
            rows = perm[s0:s0 + TT]
            umask = int(np.bitwise_or.reduce(tmask[rows]))
            maxpos = int(rows.max())
            for t in range(len(pairs)):
                if not masks[t] & umask:
                    continue
                seg = perm[offs[t]:offs[t + 1]]
                keys = int(np.searchsorted(seg, maxpos - w, side="left"))
                total += (keys + BN - 1) // BN
    return total * BN * TT
