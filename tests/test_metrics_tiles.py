"""Computed-pair counts (the key tiles the attention kernels visit) against a
direct per-tile enumeration and hand-computed cases."""
import numpy as np
import pytest

from group_gated_sparse_amd import metrics


def brute_window(n, w, TT, BN):
    total = 0
    for q0 in range(0, n, TT):
        lo, hi = max(0, q0 - w), min(n, q0 + TT)
        total += -(-(hi - lo) // BN)
    return total * BN * TT


def brute_long_range(ids_flat, perm, offsets, w, TT, BN):
    """Per sorted tile and group present: count the segment's slots whose
    position is below (largest query position of the group in the tile) - w
    by scanning them one by one."""
    total = 0
    for b in range(perm.shape[0]):
        ne = perm.shape[1]
        for s0 in range(0, ne, TT):
            rows = range(s0, min(ne, s0 + TT))
            groups = sorted({int(ids_flat[b][perm[b][s]]) for s in rows})
            for g in range(groups[0], groups[-1] + 1):
                ob, oe = int(offsets[b][g]), int(offsets[b][g + 1])
                mine = [s for s in rows if ob <= s < oe]
                if not mine:
                    continue
                maxpos = max(int(perm[b][s]) for s in mine)
                keys = 0
                for s in range(ob, max(mine) + 1):
                    if int(perm[b][s]) < maxpos - w:
                        keys += 1
                    else:
                        break
                total += -(-keys // BN)
    return total * BN * TT


def brute_entry_long_range(ids, w, TT, BN):
    """The entry passes' key tiles by direct enumeration, ids [B][n][2]: for
    membership index c, the tokens ordered by (their c-th group, position)
    are cut into tiles of TT; for each tile and each group g of its tokens,
    count the tokens having g as either group (in position order) whose
    position is below (largest position of the tile's tokens of g) - w, one by
    one."""
    total = 0
    B, n, _ = ids.shape
    for b in range(B):
        for c in (0, 1):
            order = sorted(range(n), key=lambda t: (int(ids[b, t, c]), t))
            for s0 in range(0, n, TT):
                rows = order[s0:s0 + TT]
                for g in sorted({int(ids[b, t, c]) for t in rows}):
                    maxpos = max(t for t in rows if ids[b, t, c] == g)
                    keys = 0
                    for t in range(n):
                        if g in (int(ids[b, t, 0]), int(ids[b, t, 1])):
                            if t < maxpos - w:
                                keys += 1
                            else:
                                break
                    total += -(-keys // BN)
    return total * BN * TT


def sort_entries(ids_flat, K):
    perm = np.argsort(ids_flat, axis=1, kind="stable").astype(np.int32)
    offs = np.stack([np.concatenate([[0], np.cumsum(np.bincount(r, minlength=K))]) for r in ids_flat])
    return perm, offs.astype(np.int32)


def test_window_hand_case():
    # n = 64, w = 32, 16-token tiles, 32-key tiles: 1 + 1 + 2 + 2 key tiles
    assert metrics.window_computed_pairs(64, 32, 16, 32) == 6 * 32 * 16


@pytest.mark.parametrize("n,w,TT,BN", [(1, 0, 16, 32), (77, 5, 16, 32), (300, 64, 32, 64),
                                       (1000, 128, 16, 32), (513, 1000, 64, 32)])
def test_window_matches_enumeration(n, w, TT, BN):
    got = metrics.window_computed_pairs(n, w, TT, BN)
    assert got == brute_window(n, w, TT, BN)
    assert got >= metrics.window_pairs(n, w)


@pytest.mark.parametrize("seed,B,n,K,w,TT", [(1, 1, 200, 4, 10, 16), (2, 2, 333, 8, 30, 16),
                                              (3, 1, 256, 3, 0, 32), (5, 1, 97, 64, 5, 16)])
def test_long_range_matches_enumeration(seed, B, n, K, w, TT):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, K, (B, n)).astype(np.int32)
    perm, offs = sort_entries(ids, K)
    BN = 32
    got = metrics.long_range_computed_pairs(ids, perm, offs, w, TT, BN)
    assert got == brute_long_range(ids, perm, offs, w, TT, BN)
    assert got >= metrics.pair_counts(ids, w)[1]


@pytest.mark.parametrize("seed,B,n,K,w,TT,BN", [(4, 1, 180, 6, 20, 16, 32), (6, 2, 300, 5, 0, 16, 32),
                                                 (7, 1, 257, 32, 12, 64, 64),
                                                 (8, 1, 130, 9, 3, 32, 32)])
def test_entry_long_range_matches_enumeration(seed, B, n, K, w, TT, BN):
    rng = np.random.default_rng(seed)
    ids = np.stack([np.stack([rng.choice(K, 2, replace=False) for _ in range(n)])
                    for _ in range(B)]).astype(np.int32)
    flat = ids.reshape(B, 2 * n)
    perm, offs = sort_entries(flat, K)
    got = metrics.entry_long_range_computed_pairs(flat, perm, offs, w, TT, BN)
    assert got == brute_entry_long_range(ids, w, TT, BN)
    # every far pair inside a group's segment is computed
    assert got >= metrics.pair_counts_multi(ids, w)[2]


def test_long_range_empty_when_window_covers_all():
    rng = np.random.default_rng(9)
    ids = rng.integers(0, 5, (1, 150)).astype(np.int32)
    perm, offs = sort_entries(ids, 5)
    assert metrics.long_range_computed_pairs(ids, perm, offs, 149, 16, 32) == 0


def test_heads_per_workgroup_and_tile_keys():
    assert metrics.heads_per_workgroup(64, 8) == 8
    assert metrics.heads_per_workgroup(12, 12) == 1
    assert metrics.heads_per_workgroup(24, 2) == 4
    assert metrics.heads_per_workgroup(12, 2) == 2
    assert metrics.tile_keys(32) == 64 and metrics.tile_keys(64) == 32 and metrics.tile_keys(128) == 32


def brute_set_long_range(ids, K, w, TT, BN):
    """The set pass's key tiles by direct enumeration: sort tokens by their
    pair of groups (lexicographic pair index, stable), then per tile of TT
    tokens and per set sharing a group with any of them, count that set's
    tokens (in position order) whose position is below (largest position in
    the tile) - w one by one."""
    total = 0
    pairs = [(a, b) for a in range(K) for b in range(a + 1, K)]
    for b in range(ids.shape[0]):
        n = ids.shape[1]
        key = [pairs.index(tuple(sorted((int(ids[b, t, 0]), int(ids[b, t, 1]))))) for t in range(n)]
        order = sorted(range(n), key=lambda t: (key[t], t))
        for s0 in range(0, n, TT):
            rows = order[s0:s0 + TT]
            groups = set()
            for t in rows:
                groups |= {int(ids[b, t, 0]), int(ids[b, t, 1])}
            maxpos = max(rows)
            for si, (x, y) in enumerate(pairs):
                if x not in groups and y not in groups:
                    continue
                keys = sum(1 for t in range(n) if key[t] == si and t < maxpos - w)
                total += -(-keys // BN)
    return total * BN * TT


@pytest.mark.parametrize("n,K,w,TT,BN", [(1, 2, 0, 16, 32), (90, 4, 5, 16, 32), (300, 3, 20, 32, 64),
                                         (500, 4, 40, 16, 32)])
def test_set_long_range_matches_enumeration(n, K, w, TT, BN):
    rng = np.random.default_rng(n + K)
    ids = np.stack([np.stack([rng.choice(K, size=2, replace=False) for _ in range(n)])])
    got = metrics.set_long_range_computed_pairs(ids, K, w, TT, BN)
    assert got == brute_set_long_range(ids, K, w, TT, BN)
    kept, _ = metrics.long_range_pairs_multi(ids[0], w)
    assert got >= kept
