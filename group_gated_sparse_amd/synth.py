"""Seeded synthetic inputs for the Focus forward pass.

This module only draws inputs. It holds none of the method's arithmetic
(no projection, no centroid scores, no argmax, no sort, no attention), so it
can feed both the HIP path and the CPU oracle.

Recipe: three independent numpy streams, ``default_rng([seed, 0])`` for P and
C, ``default_rng([seed, 1])`` for hidden, ``default_rng([seed, 2])`` for q, k, v
(so attention-only callers need not draw the hidden states):
  1. P  (d_model x d_proj, fp32)
       "gauss":       standard_normal * float32(1/sqrt(d_model))
       "orthonormal": Q factor of a standard_normal (d_model x d_proj) matrix
  2. C  (K x d_proj, fp32)
       "gauss":       standard_normal, each row divided by its fp32 norm
       "orthonormal": transpose of the Q factor of a standard_normal (d_proj x K)
  3. hidden (B x n x d_model, fp32 standard_normal), drawn per batch element in
     chunks of 4096 rows
  4. q (B x Hq x n x d), k, v (B x Hkv x n x d): fp32 standard_normal, q times
     q_prescale, then rounded to bf16 (round to nearest, ties to even); one
     (b, head) slab at a time.
The per-group logit bias is not drawn: for "orthonormal" P and C the K
centroid logits of a token with N(0, I) hidden state are i.i.d. N(0, 1), so the
probability that group k wins the argmax under bias b is
    p_k(b) = integral phi(x - b_k) prod_{j != k} Phi(x - b_j) dx,
and ``gauss_max_bias`` solves p_k(b) = target_k by fixed-point iteration.
"""
from __future__ import annotations

import hashlib
from typing import Dict, Optional

import numpy as np
from scipy.special import log_ndtr

from .workloads import Workload

HIDDEN_CHUNK_ROWS = 4096


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs here are finite normal samples, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact fp32 values they encode."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_target(K: int, s: float) -> np.ndarray:
    p = (np.arange(1, K + 1, dtype=np.float64)) ** (-s)
    return p / p.sum()


def gauss_max_win_prob(b: np.ndarray, step: float = 2e-3) -> np.ndarray:
    """P(argmax_k (x_k + b_k) = k) for i.i.d. standard normal x_k."""
    b = np.asarray(b, dtype=np.float64)
    x = np.arange(b.min() - 9.0, b.max() + 9.0, step)
    logcdf = log_ndtr(x[None, :] - b[:, None])            # K x X
    total = logcdf.sum(axis=0)                             # sum_j log Phi(x - b_j)
    dens = np.exp(-0.5 * (x[None, :] - b[:, None]) ** 2 - 0.5 * np.log(2 * np.pi))
    integrand = dens * np.exp(total[None, :] - logcdf)
    return np.trapezoid(integrand, x, axis=1)


def gauss_max_bias(target: np.ndarray, iters: int = 2000, tol: float = 1e-9) -> np.ndarray:
    """Bias b with gauss_max_win_prob(b) = target (damped fixed point, mean 0)."""
    target = np.asarray(target, dtype=np.float64)
    b = np.zeros_like(target)
    for _ in range(iters):
        p = np.maximum(gauss_max_win_prob(b), 1e-300)
        delta = np.log(target) - np.log(p)
        if np.max(np.abs(delta)) < tol:
            break
        b = b + 0.3 * delta
        b -= b.mean()
    return b


def _orthonormal_columns(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    g = rng.standard_normal((rows, cols), dtype=np.float32).astype(np.float64)
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return q


def draw_centroid_space(wl: Workload, rng: np.random.Generator):
    """Steps 1-2: P and C (fp32)."""
    if wl.pc_kind == "gauss":
        P = rng.standard_normal((wl.d_model, wl.d_proj), dtype=np.float32) \
            * np.float32(1.0 / np.sqrt(wl.d_model))
        C = rng.standard_normal((wl.K, wl.d_proj), dtype=np.float32)
        C = C / np.linalg.norm(C, axis=1, keepdims=True).astype(np.float32)
    elif wl.pc_kind == "orthonormal":
        if wl.K > wl.d_proj or wl.d_proj > wl.d_model:
            raise ValueError("orthonormal P/C need K <= d_proj <= d_model")
        P = _orthonormal_columns(rng, wl.d_model, wl.d_proj)
        C = _orthonormal_columns(rng, wl.d_proj, wl.K).T
    else:
        raise ValueError(f"unknown pc_kind {wl.pc_kind!r}")
    return np.ascontiguousarray(P, dtype=np.float32), np.ascontiguousarray(C, dtype=np.float32)


def logit_bias(wl: Workload) -> Optional[np.ndarray]:
    if wl.bias_target is None:
        return None
    if wl.pc_kind != "orthonormal":
        raise ValueError("a calibrated bias needs orthonormal P and C")
    if wl.bias_target == "zipf":
        return gauss_max_bias(zipf_target(wl.K, wl.zipf_s)).astype(np.float32)
    raise ValueError(f"unknown bias_target {wl.bias_target!r}")


def draw_hidden(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    h = np.empty((wl.B, wl.n, wl.d_model), dtype=np.float32)
    for b in range(wl.B):
        for r0 in range(0, wl.n, HIDDEN_CHUNK_ROWS):
            r1 = min(wl.n, r0 + HIDDEN_CHUNK_ROWS)
            h[b, r0:r1] = rng.standard_normal((r1 - r0, wl.d_model), dtype=np.float32)
    return h


def draw_qkv(wl: Workload, rng: np.random.Generator):
    q = np.empty((wl.B, wl.Hq, wl.n, wl.d), dtype=np.uint16)
    k = np.empty((wl.B, wl.Hkv, wl.n, wl.d), dtype=np.uint16)
    v = np.empty((wl.B, wl.Hkv, wl.n, wl.d), dtype=np.uint16)
    pre = np.float32(wl.q_prescale)
    for b in range(wl.B):
        for h in range(wl.Hq):
            x = rng.standard_normal((wl.n, wl.d), dtype=np.float32)
            if wl.q_prescale != 1.0:
                x = x * pre
            q[b, h] = bf16_bits(x)
    for t in (k, v):
        for b in range(wl.B):
            for h in range(wl.Hkv):
                t[b, h] = bf16_bits(rng.standard_normal((wl.n, wl.d), dtype=np.float32))
    return q, k, v


def make_inputs(wl: Workload, with_hidden: bool = True, with_qkv: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of one workload (each part from its own seeded stream)."""
    P, C = draw_centroid_space(wl, np.random.default_rng([wl.seed, 0]))
    out: Dict[str, np.ndarray] = {"P": P, "C": C, "bias": logit_bias(wl)}
    if with_hidden:
        out["hidden"] = draw_hidden(wl, np.random.default_rng([wl.seed, 1]))
    if with_qkv:
        out["q"], out["k"], out["v"] = draw_qkv(wl, np.random.default_rng([wl.seed, 2]))
    return out


def random_group_ids(rng: np.random.Generator, B: int, n: int, K: int,
                     probs: Optional[np.ndarray] = None) -> np.ndarray:
    """Group ids drawn directly (for attention-only cases), int32 in [0, K)."""
    if probs is None:
        return rng.integers(0, K, size=(B, n), dtype=np.int32)
    return rng.choice(K, size=(B, n), p=probs).astype(np.int32)


def digest(arrays: Dict[str, Optional[np.ndarray]]) -> str:
    h = hashlib.sha256()
    for key in sorted(arrays):
        a = arrays[key]
        h.update(key.encode())
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
