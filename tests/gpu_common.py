"""Shared helpers of the GPU tests: moving seeded inputs to the device and
comparing device results with the oracle at the agreed tolerances."""
import math
import sys

import numpy as np
import torch

# Attention parity bound on the same bf16-rounded inputs (fp32 output):
ATTN_MAX_ABS = 1e-2
ATTN_MEAN_ABS = 1e-3
# Assignment: ids may differ only where the oracle's top-2 margin is below this.
TIE_BAND = 1e-3


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def sample_rows(rng, B, Hq, n, w, per_head=48, heads=None, ids=None):
    """Flattened (b*Hq+h)*n+i rows: the start, the window edge, the end and random rows;
    with ids (B, n) or (B, n, m) also the first and last token of every group."""
    heads = range(Hq) if heads is None else heads
    fixed = {0, 1, min(n - 1, max(0, w - 1)), min(n - 1, w), min(n - 1, w + 1), n - 2, n - 1}
    rows = []
    for b in range(B):
        edges = set()
        if ids is not None:
            ib = np.asarray(ids[b]).reshape(n, -1)
            for g in np.unique(ib):
                pos = np.nonzero((ib == g).any(axis=1))[0]
                edges |= {int(pos[0]), int(pos[-1])}
        for h in heads:
            picks = set(i for i in fixed if 0 <= i < n) | edges
            picks |= set(rng.integers(0, n, size=min(per_head, n)).tolist())
            rows += [(b * Hq + h) * n + i for i in sorted(picks)]
    return np.array(rows, dtype=np.int64)


def check_attn(got: np.ndarray, ref: np.ndarray, what: str, bf16_out: bool = False):
    """got, ref: [rows, d]. fp32 output: max-abs <= 1e-2 and mean-abs <= 1e-3.
    bf16 output adds the output rounding (half an ulp, <= |ref| * 2^-8)."""
    err = np.abs(got.astype(np.float64) - ref)
    if bf16_out:
        allow = ATTN_MAX_ABS + np.abs(ref) * 2.0 ** -8
        bad = err > allow
    else:
        bad = err > ATTN_MAX_ABS
    say(f"  {what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond tolerance, max err {err.max()}"
    assert err.mean() <= ATTN_MEAN_ABS, f"{what}: mean-abs {err.mean()} > {ATTN_MEAN_ABS}"


def check_ids(gpu_ids, ora_ids, ora_margin, hidden_rows, P, C, bias, what):
    """Ids equal the oracle's except near-ties (oracle margin < TIE_BAND) where
    the GPU id must be one of the two top-scoring groups (scored in fp64)."""
    diff = np.nonzero(gpu_ids != ora_ids)[0]
    say(f"  {what}: {diff.size} of {gpu_ids.size} ids differ from the oracle; "
        f"{int((ora_margin < TIE_BAND).sum())} tokens in the tie band")
    if diff.size == 0:
        return
    assert (ora_margin[diff] < TIE_BAND).all(), \
        f"{what}: ids differ outside the tie band at {diff[ora_margin[diff] >= TIE_BAND][:8]}"
    h = hidden_rows[diff].astype(np.float64)
    s = (h @ P.astype(np.float64)) @ C.astype(np.float64).T
    if bias is not None:
        s = s + bias.astype(np.float64)
    top2 = np.argsort(-s, axis=1, kind="stable")[:, :2]
    assert ((top2 == gpu_ids[diff][:, None]).any(axis=1)).all(), f"{what}: id not in top-2"


def visited_pairs(ids: np.ndarray, w: int) -> int:
    """sum over b, i of |A_i| per query head (window band + same-group far pairs)."""
    B, n = ids.shape
    ww = min(w, n - 1)
    total = B * (n * (ww + 1) - ww * (ww + 1) // 2)
    for b in range(B):
        for g in np.unique(ids[b]):
            pos = np.nonzero(ids[b] == g)[0]
            total += int(np.searchsorted(pos, pos - w, side="left").sum())
    return total


def approx_equal_or_raise(a, b, tol, what):
    m = float(np.max(np.abs(a - b))) if a.size else 0.0
    if not m <= tol:
        raise AssertionError(f"{what}: max diff {m} > {tol}")
    return m


def is_finite(x) -> bool:
    return bool(np.isfinite(x).all())


__all__ = ["say", "dev", "dev_bf16", "host", "sample_rows", "check_attn", "check_ids",
           "visited_pairs", "math", "ATTN_MAX_ABS", "ATTN_MEAN_ABS", "TIE_BAND"]
