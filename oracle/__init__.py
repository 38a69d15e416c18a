"""CPU oracle for the Focus group-gated attention forward pass (numpy front end).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers. The product path never
imports this package, and this package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C: fp32 assignment, stable
counting sort, fp64 masked softmax attention) and ``brute.py`` (pure-Python
pair enumeration for tiny cases). Every function cites the page passage it
follows in its docstring or in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (-O2 -fopenmp -ffp-contract=off)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    lib.oracle_assign.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p, _i64,
                                  _p, _p, ctypes.c_int]
    lib.oracle_assign.restype = ctypes.c_int
    lib.oracle_group_sort.argtypes = [_p, _i64, _i64, _i64, _p, _p]
    lib.oracle_group_sort.restype = ctypes.c_int
    lib.oracle_attn.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                ctypes.c_double, _p, _i64, _p, _p, _p, ctypes.c_int]
    lib.oracle_attn.restype = ctypes.c_int
    lib.oracle_attn_two_phase.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64,
                                          _i64, ctypes.c_double, _p, _i64, _p, _p,
                                          ctypes.c_int]
    lib.oracle_attn_two_phase.restype = ctypes.c_int
    lib.oracle_attn_weights.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                        ctypes.c_double, _i64, _i64, _i64, _p]
    lib.oracle_attn_weights.restype = ctypes.c_int
    lib.oracle_pair_count.argtypes = [_p, _i64, _i64, _i64, ctypes.c_int]
    lib.oracle_pair_count.restype = _i64
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_assign_topk.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _p,
                                       _i64, _p, _p, ctypes.c_int]
    lib.oracle_assign_topk.restype = ctypes.c_int
    lib.oracle_attn_multi.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                      ctypes.c_double, _p, _i64, _p, _p, _p, ctypes.c_int]
    lib.oracle_attn_multi.restype = ctypes.c_int
    lib.oracle_pair_count_multi.argtypes = [_p, _i64, _i64, _i64, _i64, ctypes.c_int]
    lib.oracle_pair_count_multi.restype = _i64
    lib.oracle_assign_scores.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p,
                                         ctypes.c_int]
    lib.oracle_assign_scores.restype = ctypes.c_int
    lib.oracle_sinkhorn.argtypes = [_p, _i64, _i64, _i64, ctypes.c_double, _i64, _p]
    lib.oracle_sinkhorn.restype = ctypes.c_int
    lib.oracle_soft_gate_attn.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                          ctypes.c_double, ctypes.c_double, _p, _i64, _p, _p,
                                          ctypes.c_int]
    lib.oracle_soft_gate_attn.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def assign(hidden, P, C, bias=None, tokens=None, nthreads: int = 0):
    """Hard top-1 group of each token: argmax_k (h·P)·C_k + bias_k, fp32.

    Japanese page, technical summary §2.1 (projection into centroid space)
    and §2.2 (hard assignment at inference). ``hidden`` is (B, n, d_model);
    ``tokens`` optionally lists flattened b*n+t indices. Returns (ids, margin),
    margin = top-1 minus top-2 score (+inf when K == 1).
    """
    hidden = _c(hidden, np.float32)
    P = _c(P, np.float32)
    C = _c(C, np.float32)
    bias = _c(bias, np.float32)
    B, n, d_model = hidden.shape
    d_proj = P.shape[1]
    K = C.shape[0]
    assert P.shape == (d_model, d_proj) and C.shape == (K, d_proj)
    if tokens is not None:
        tokens = _c(tokens, np.int64).ravel()
        count = tokens.size
    else:
        count = B * n
    ids = np.empty(count, dtype=np.int32)
    margin = np.empty(count, dtype=np.float32)
    rc = _load().oracle_assign(_ptr(hidden), _ptr(P), _ptr(C), _ptr(bias), B, n, d_model, d_proj,
                               K, _ptr(tokens), count if tokens is not None else 0,
                               _ptr(ids), _ptr(margin), nthreads)
    if rc != 0:
        raise ValueError("oracle_assign rejected its arguments")
    if tokens is None:
        ids = ids.reshape(B, n)
        margin = margin.reshape(B, n)
    return ids, margin


def group_sort(ids, K: int):
    """Stable counting sort of tokens by group: (perm (B, n), offsets (B, K+1))."""
    ids = _c(ids, np.int32)
    B, n = ids.shape
    perm = np.empty((B, n), dtype=np.int32)
    offsets = np.empty((B, K + 1), dtype=np.int32)
    if _load().oracle_group_sort(_ptr(ids), B, n, K, _ptr(perm), _ptr(offsets)) != 0:
        raise ValueError("oracle_group_sort rejected its arguments (ids outside [0, K)?)")
    return perm, offsets


def _attn_common(q, k, v, ids):
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    ids = _c(ids, np.int32)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, n, d) and v.shape == k.shape and ids.shape == (B, n)
    return q, k, v, ids, B, Hq, Hkv, n, d


def attn(q, k, v, ids, w: int, scale: float, rows=None, nthreads: int = 0):
    """Exact softmax attention over A_i = {j <= i : i-j <= w or same group}.

    Korean page §2.1/§2.3, Japanese page §2.1/§2.2. q (B,Hq,n,d), k/v
    (B,Hkv,n,d) as bf16 bit patterns (uint16); ids (B, n). ``rows`` lists
    flattened (b*Hq+h)*n+i rows (default: all). Returns (out fp64 [rows, d]
    or (B,Hq,n,d), lse fp64, visited int64).
    """
    q, k, v, ids, B, Hq, Hkv, n, d = _attn_common(q, k, v, ids)
    if rows is not None:
        rows = _c(rows, np.int64).ravel()
        count = rows.size
    else:
        count = B * Hq * n
    out = np.empty((count, d), dtype=np.float64)
    lse = np.empty(count, dtype=np.float64)
    visited = np.empty(count, dtype=np.int64)
    rc = _load().oracle_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(ids), B, Hq, Hkv, n, d, int(w),
                             float(scale), _ptr(rows), count if rows is not None else 0,
                             _ptr(out), _ptr(lse), _ptr(visited), nthreads)
    if rc != 0:
        raise ValueError("oracle_attn rejected its arguments")
    if rows is None:
        return out.reshape(B, Hq, n, d), lse.reshape(B, Hq, n), visited.reshape(B, Hq, n)
    return out, lse, visited


def attn_two_phase(q, k, v, ids, w: int, scale: float, rows=None, nthreads: int = 0):
    """Window part and intra-group long-range part merged by log-sum-exp
    (Korean page §2.3's two-part split). Same returns as ``attn`` minus visited."""
    q, k, v, ids, B, Hq, Hkv, n, d = _attn_common(q, k, v, ids)
    if rows is not None:
        rows = _c(rows, np.int64).ravel()
        count = rows.size
    else:
        count = B * Hq * n
    out = np.empty((count, d), dtype=np.float64)
    lse = np.empty(count, dtype=np.float64)
    rc = _load().oracle_attn_two_phase(_ptr(q), _ptr(k), _ptr(v), _ptr(ids), B, Hq, Hkv, n, d,
                                       int(w), float(scale), _ptr(rows),
                                       count if rows is not None else 0, _ptr(out), _ptr(lse),
                                       nthreads)
    if rc != 0:
        raise ValueError("oracle_attn_two_phase rejected its arguments")
    if rows is None:
        return out.reshape(B, Hq, n, d), lse.reshape(B, Hq, n)
    return out, lse


def attn_weights(q, k, ids, w: int, scale: float, b: int, h: int, i: int):
    """Softmax weights of row (b, h, i) over all n keys (0 outside A_i)."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    ids = _c(ids, np.int32)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    wts = np.empty(n, dtype=np.float64)
    rc = _load().oracle_attn_weights(_ptr(q), _ptr(k), _ptr(ids), B, Hq, Hkv, n, d, int(w),
                                     float(scale), b, h, i, _ptr(wts))
    if rc != 0:
        raise ValueError("oracle_attn_weights rejected its arguments")
    return wts


def pair_count(ids, w: int, nthreads: int = 0) -> int:
    """sum over b, i of |A_i| (pairs per query head), by direct enumeration."""
    ids = _c(ids, np.int32)
    B, n = ids.shape
    r = _load().oracle_pair_count(_ptr(ids), B, n, int(w), nthreads)
    if r < 0:
        raise ValueError("oracle_pair_count rejected its arguments")
    return int(r)


# ---- multi-membership (top-m groups per token) -------------------------------
# Korean page §2.3 / Japanese page §2.2: at inference a token may join its top-k
# groups (k = 2 at K = 4 in the Korean page §3.4 and the Japanese page §3.3);
# a far pair is then kept when the two tokens share any group.

def assign_topk(hidden, P, C, m: int, bias=None, tokens=None, nthreads: int = 0):
    """Top-m groups per token by the fp32 scores of assign(): ids (B, n, m)
    in decreasing score order (exact ties to the lowest index) and margin
    s_(m) - s_(m+1) (+inf when K == m)."""
    hidden = _c(hidden, np.float32)
    P = _c(P, np.float32)
    C = _c(C, np.float32)
    bias = _c(bias, np.float32)
    B, n, d_model = hidden.shape
    d_proj = P.shape[1]
    K = C.shape[0]
    assert P.shape == (d_model, d_proj) and C.shape == (K, d_proj)
    if tokens is not None:
        tokens = _c(tokens, np.int64).ravel()
        count = tokens.size
    else:
        count = B * n
    ids = np.empty((count, m), dtype=np.int32)
    margin = np.empty(count, dtype=np.float32)
    rc = _load().oracle_assign_topk(_ptr(hidden), _ptr(P), _ptr(C), _ptr(bias), B, n, d_model,
                                    d_proj, K, int(m), _ptr(tokens),
                                    count if tokens is not None else 0, _ptr(ids), _ptr(margin),
                                    nthreads)
    if rc != 0:
        raise ValueError("oracle_assign_topk rejected its arguments")
    if tokens is None:
        ids = ids.reshape(B, n, m)
        margin = margin.reshape(B, n)
    return ids, margin


def group_sort_multi(ids, K: int):
    """Stable sort of membership entries by group. ids (B, n, m); entry
    e = t*m + c is token t's c-th group. Returns (perm (B, n*m) of entry
    indices, offsets (B, K+1)): each group's entries are one segment in
    increasing position."""
    ids = _c(ids, np.int32)
    B, n, m = ids.shape
    return group_sort(ids.reshape(B, n * m), K)


def _attn_multi_common(q, k, v, ids):
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    ids = _c(ids, np.int32)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, n, d) and v.shape == k.shape
    assert ids.ndim == 3 and ids.shape[:2] == (B, n)
    return q, k, v, ids, B, Hq, Hkv, n, d, ids.shape[2]


def attn_multi(q, k, v, ids, w: int, scale: float, rows=None, nthreads: int = 0):
    """Exact softmax attention over
    A_i = {j <= i : i-j <= w or groups(i) and groups(j) intersect}, ids (B, n, m);
    otherwise as attn()."""
    q, k, v, ids, B, Hq, Hkv, n, d, m = _attn_multi_common(q, k, v, ids)
    if rows is not None:
        rows = _c(rows, np.int64).ravel()
        count = rows.size
    else:
        count = B * Hq * n
    out = np.empty((count, d), dtype=np.float64)
    lse = np.empty(count, dtype=np.float64)
    visited = np.empty(count, dtype=np.int64)
    rc = _load().oracle_attn_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(ids), m, B, Hq, Hkv, n, d,
                                   int(w), float(scale), _ptr(rows),
                                   count if rows is not None else 0, _ptr(out), _ptr(lse),
                                   _ptr(visited), nthreads)
    if rc != 0:
        raise ValueError("oracle_attn_multi rejected its arguments")
    if rows is None:
        return out.reshape(B, Hq, n, d), lse.reshape(B, Hq, n), visited.reshape(B, Hq, n)
    return out, lse, visited


def pair_count_multi(ids, w: int, nthreads: int = 0) -> int:
    """sum over b, i of |A_i| for the multi-membership pattern (ids (B, n, m))."""
    ids = _c(ids, np.int32)
    B, n, m = ids.shape
    r = _load().oracle_pair_count_multi(_ptr(ids), m, B, n, int(w), nthreads)
    if r < 0:
        raise ValueError("oracle_pair_count_multi rejected its arguments")
    return int(r)


# ---- soft assignment with Sinkhorn normalisation (training-time step) -------
# Korean page §2.2 and Japanese page §2.1 / §2.3: the token-to-group
# assignment matrix is made doubly stochastic (rows sum to 1, every group gets
# the same total n / K).

def assign_scores(hidden, P, C, bias=None, nthreads: int = 0):
    """Raw fp32 scores (h P) C^T + bias, (B, n, K), summed as in assign()."""
    hidden = _c(hidden, np.float32)
    P = _c(P, np.float32)
    C = _c(C, np.float32)
    bias = _c(bias, np.float32)
    B, n, d_model = hidden.shape
    d_proj = P.shape[1]
    K = C.shape[0]
    assert P.shape == (d_model, d_proj) and C.shape == (K, d_proj)
    S = np.empty((B, n, K), dtype=np.float32)
    rc = _load().oracle_assign_scores(_ptr(hidden), _ptr(P), _ptr(C), _ptr(bias), B, n, d_model,
                                      d_proj, K, _ptr(S), nthreads)
    if rc != 0:
        raise ValueError("oracle_assign_scores rejected its arguments")
    return S


def sinkhorn(scores, tau: float, iters: int):
    """Sinkhorn-Knopp soft assignment G (B, n, K) fp64 of A = exp(scores/tau):
    rows first, then `iters` rounds of (columns to n/K, rows to 1)."""
    scores = _c(scores, np.float32)
    B, n, K = scores.shape
    G = np.empty((B, n, K), dtype=np.float64)
    if _load().oracle_sinkhorn(_ptr(scores), B, n, K, float(tau), int(iters), _ptr(G)) != 0:
        raise ValueError("oracle_sinkhorn rejected its arguments")
    return G


def soft_gate_attn(q, k, v, G, w: int, scale: float, lam: float, rows=None, nthreads: int = 0):
    """Training-time soft-gated attention (Japanese page §2.1-§2.2, Korean
    page §2.1): every causal pair, weight gate_ij * exp(scale q_i.k_j) with
    gate 1 inside the window (i - j <= w) and sigmoid(lam * g_i.g_j) beyond.
    G (B, n, K) fp32 soft assignments. Returns (out, lse) like attn()."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    G = _c(G, np.float32)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    K = G.shape[2]
    assert k.shape == (B, Hkv, n, d) and v.shape == k.shape and G.shape[:2] == (B, n)
    if rows is not None:
        rows = _c(rows, np.int64).ravel()
        count = rows.size
    else:
        count = B * Hq * n
    out = np.empty((count, d), dtype=np.float64)
    lse = np.empty(count, dtype=np.float64)
    rc = _load().oracle_soft_gate_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(G), B, Hq, Hkv, n, d, K,
                                       int(w), float(scale), float(lam), _ptr(rows),
                                       count if rows is not None else 0, _ptr(out), _ptr(lse),
                                       nthreads)
    if rc != 0:
        raise ValueError("oracle_soft_gate_attn rejected its arguments")
    if rows is None:
        return out.reshape(B, Hq, n, d), lse.reshape(B, Hq, n)
    return out, lse
