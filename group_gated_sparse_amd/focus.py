"""Thin ctypes binding of libfocus.so (C ABI in include/focus.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, turned into device pointers, and passed with the current HIP
stream. Every step of the computation runs in the library's HIP kernels; a
missing library raises instead of falling back to anything else.

q, k, v are torch.bfloat16 CUDA tensors (their bits are the ABI's uint16).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfocus.so")

FOCUS_OK = 0
FOCUS_BF16 = 0
FOCUS_F32 = 1
STATUS_NAMES = {0: "FOCUS_OK", 1: "FOCUS_ERR_INVALID_ARGUMENT", 2: "FOCUS_ERR_UNSUPPORTED",
                3: "FOCUS_ERR_WORKSPACE", 4: "FOCUS_ERR_DEVICE"}

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_f = ctypes.c_float

_SIGNATURES = {
    "focus_abi_version": ([], _i),
    "focus_last_error": ([], ctypes.c_char_p),
    "focus_assign_workspace_bytes": ([_i, _i], _sz),
    "focus_assign": ([_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _sz, _p], _i),
    "focus_group_sort_workspace_bytes": ([_i, _i, _i], _sz),
    "focus_group_sort": ([_p, _i, _i, _i, _p, _p, _p, _sz, _p], _i),
    "focus_group_sort_noalloc": ([_p, _i, _i, _i, _p, _p, _p], _i),
    "focus_attn_workspace_bytes": ([_i, _i, _i, _i, _i, _i, _i], _sz),
    "focus_attn_fwd": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _i, _p, _p,
                        _sz, _p], _i),
    "focus_attn_sorted_kv_workspace_bytes": ([_i, _i, _i, _i, _i, _i, _i], _sz),
    "focus_attn_fwd_sorted_kv": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _i,
                                  _p, _p, _sz, _p], _i),
    "focus_attn_window": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _i,
                               _p, _p, _sz, _p], _i),
    "focus_attn_long_range_merge": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p,
                                 _i, _p, _p, _sz, _p], _i),
    "focus_attn_long_range_prepare": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f,
                                       _p, _i, _p, _p, _sz, _p], _i),
    "focus_attn_long_range_apply": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p,
                                     _i, _p, _p, _sz, _p], _i),
    "dense_causal_attn_fwd": ([_p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _i, _p, _p], _i),
    "focus_assign_topk": ([_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _sz, _p], _i),
    "focus_attn_topk_workspace_bytes": ([_i, _i, _i, _i, _i, _i, _i, _i], _sz),
    "focus_attn_topk_fwd": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _i,
                             _p, _p, _sz, _p], _i),
    "focus_attn_topk_long_range_merge": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
                                          _f, _p, _i, _p, _p, _sz, _p], _i),
    "focus_attn_topk_long_range_prepare": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                                            _i, _f, _p, _i, _p, _p, _sz, _p], _i),
    "focus_attn_topk_long_range_apply": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
                                          _f, _p, _i, _p, _p, _sz, _p], _i),
    "focus_assign_scores": ([_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _sz, _p], _i),
    "focus_sinkhorn_workspace_bytes": ([_i, _i, _i, _i], _sz),
    "focus_sinkhorn": ([_p, _i, _i, _i, _f, _i, _p, _p, _sz, _p], _i),
    "focus_soft_gate_attn_workspace_bytes": ([_i, _i, _i], _sz),
    "focus_soft_gate_attn_fwd": ([_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _f, _p, _i, _p,
                                  _p, _sz, _p], _i),
}

_lib = None


class FocusError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib():
    """The loaded libfocus.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m group_gated_sparse_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check_status(status: int):
    if status != FOCUS_OK:
        raise FocusError(status, lib().focus_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _new(shape, dtype, device, stream) -> torch.Tensor:
    """A tensor the binding allocates for a call enqueued on `stream`.

    torch's caching allocator ties a block to the stream current at
    allocation; when the kernels run on another stream, record_stream keeps
    the block from being handed out again (e.g. a workspace dropped on
    return) until the work queued on that stream has passed it."""
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)
    return t


def _workspace(nbytes: int, device, given: Optional[torch.Tensor], stream=None):
    if nbytes == 0:
        return given
    if given is not None:
        _need(given, "workspace", torch.uint8)
        return given
    return _new(nbytes, torch.uint8, device, stream)


# ---------------------------------------------------------------------------
def focus_assign_workspace_bytes(d_model: int, K: int) -> int:
    return int(lib().focus_assign_workspace_bytes(d_model, K))


def focus_assign(hidden: torch.Tensor, P: torch.Tensor, C: torch.Tensor,
                 bias: Optional[torch.Tensor] = None, *, group_ids=None, margin=None,
                 want_margin: bool = True, workspace=None, stream=None
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Group id per token: argmax_k (h P) C_k^T + bias_k. hidden (B, n, d_model) fp32."""
    return _assign(hidden, P, C, bias, 1, group_ids, margin, want_margin, workspace, stream)


def focus_assign_topk(hidden: torch.Tensor, P: torch.Tensor, C: torch.Tensor, m: int,
                      bias: Optional[torch.Tensor] = None, *, group_ids=None, margin=None,
                      want_margin: bool = True, workspace=None, stream=None
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Top-m groups per token, best first: group_ids (B, n, m); margin = m-th
    minus (m+1)-th score."""
    return _assign(hidden, P, C, bias, m, group_ids, margin, want_margin, workspace, stream)


def _assign(hidden, P, C, bias, m, group_ids, margin, want_margin, workspace, stream):
    B, n, d_model = hidden.shape
    d_proj = P.shape[1]
    K = C.shape[0]
    _need(hidden, "hidden", torch.float32)
    _need(P, "P", torch.float32, (d_model, d_proj))
    _need(C, "C", torch.float32, (K, d_proj))
    if bias is not None:
        _need(bias, "bias", torch.float32, (K,))
    dev = hidden.device
    ids_shape = (B, n) if m == 1 else (B, n, m)
    if group_ids is None:
        group_ids = _new(ids_shape, torch.int32, dev, stream)
    _need(group_ids, "group_ids", torch.int32, ids_shape)
    if margin is None and want_margin:
        margin = _new((B, n), torch.float32, dev, stream)
    if margin is not None:
        _need(margin, "margin", torch.float32, (B, n))
    nbytes = focus_assign_workspace_bytes(d_model, K)
    ws = _workspace(nbytes, dev, workspace, stream)
    _check_status(lib().focus_assign_topk(_ptr(hidden), _ptr(P), _ptr(C), _ptr(bias), B, n,
                                          d_model, d_proj, K, int(m), _ptr(group_ids),
                                          _ptr(margin), _ptr(ws),
                                          0 if ws is None else ws.numel(), _stream(stream)))
    return group_ids, margin


def focus_assign_scores(hidden: torch.Tensor, P: torch.Tensor, C: torch.Tensor,
                        bias: Optional[torch.Tensor] = None, *, scores=None, workspace=None,
                        stream=None) -> torch.Tensor:
    """Raw scores (h P) C^T + bias, (B, n, K) fp32."""
    B, n, d_model = hidden.shape
    d_proj = P.shape[1]
    K = C.shape[0]
    _need(hidden, "hidden", torch.float32)
    _need(P, "P", torch.float32, (d_model, d_proj))
    _need(C, "C", torch.float32, (K, d_proj))
    if bias is not None:
        _need(bias, "bias", torch.float32, (K,))
    if scores is None:
        scores = _new((B, n, K), torch.float32, hidden.device, stream)
    _need(scores, "scores", torch.float32, (B, n, K))
    ws = _workspace(focus_assign_workspace_bytes(d_model, K), hidden.device, workspace, stream)
    _check_status(lib().focus_assign_scores(_ptr(hidden), _ptr(P), _ptr(C), _ptr(bias), B, n,
                                            d_model, d_proj, K, _ptr(scores), _ptr(ws),
                                            0 if ws is None else ws.numel(), _stream(stream)))
    return scores


def focus_sinkhorn_workspace_bytes(B: int, n: int, K: int, iters: int) -> int:
    return int(lib().focus_sinkhorn_workspace_bytes(B, n, K, iters))


def focus_sinkhorn(scores: torch.Tensor, tau: float, iters: int, *, G=None, workspace=None,
                   stream=None) -> torch.Tensor:
    """Sinkhorn soft assignment of exp(scores / tau): rows first, then
    `iters` rounds of (columns to n/K, rows to 1). scores (B, n, K) fp32."""
    _need(scores, "scores", torch.float32)
    B, n, K = scores.shape
    if G is None:
        G = _new(scores.shape, torch.float32, scores.device, stream)
    _need(G, "G", torch.float32, (B, n, K))
    ws = _workspace(focus_sinkhorn_workspace_bytes(B, n, K, iters), scores.device, workspace,
                    stream)
    _check_status(lib().focus_sinkhorn(_ptr(scores), B, n, K, float(tau), int(iters), _ptr(G),
                                       _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(stream)))
    return G


def focus_group_sort_workspace_bytes(B: int, n: int, K: int) -> int:
    return int(lib().focus_group_sort_workspace_bytes(B, n, K))


def focus_group_sort(group_ids: torch.Tensor, K: int, *, perm=None, group_offsets=None,
                     workspace=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stable grouping: (perm (B, n) sorted slot -> position, group_offsets (B, K+1)).
    Top-m ids (B, n, m) are sorted as their n*m membership entries t*m + c:
    perm (B, n*m) then holds entries."""
    _need(group_ids, "group_ids", torch.int32)
    if group_ids.dim() == 3:
        group_ids = group_ids.view(group_ids.shape[0], -1)
    B, n = group_ids.shape
    dev = group_ids.device
    if perm is None:
        perm = _new((B, n), torch.int32, dev, stream)
    if group_offsets is None:
        group_offsets = _new((B, K + 1), torch.int32, dev, stream)
    _need(perm, "perm", torch.int32, (B, n))
    _need(group_offsets, "group_offsets", torch.int32, (B, K + 1))
    nbytes = focus_group_sort_workspace_bytes(B, n, K)
    ws = _workspace(nbytes, dev, workspace, stream)
    _check_status(lib().focus_group_sort(_ptr(group_ids), B, n, K, _ptr(perm),
                                         _ptr(group_offsets), _ptr(ws),
                                         0 if ws is None else ws.numel(), _stream(stream)))
    return perm, group_offsets


def focus_group_sort_noalloc(group_ids: torch.Tensor, K: int, *, perm, group_offsets,
                             stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """focus_group_sort with the library's static scratch instead of a
    workspace: the call allocates nothing, so perm and group_offsets must be
    given. Calls overlapping on one GPU share that scratch and race."""
    _need(group_ids, "group_ids", torch.int32)
    if group_ids.dim() == 3:
        group_ids = group_ids.view(group_ids.shape[0], -1)
    B, n = group_ids.shape
    _need(perm, "perm", torch.int32, (B, n))
    _need(group_offsets, "group_offsets", torch.int32, (B, K + 1))
    _check_status(lib().focus_group_sort_noalloc(_ptr(group_ids), B, n, K, _ptr(perm),
                                                 _ptr(group_offsets), _stream(stream)))
    return perm, group_offsets


def focus_attn_workspace_bytes(B: int, Hq: int, Hkv: int, n: int, d_head: int, K: int,
                               window: int) -> int:
    return int(lib().focus_attn_workspace_bytes(B, Hq, Hkv, n, d_head, K, window))


def focus_attn_sorted_kv_workspace_bytes(B: int, Hq: int, Hkv: int, n: int, d_head: int, K: int,
                                         window: int) -> int:
    return int(lib().focus_attn_sorted_kv_workspace_bytes(B, Hq, Hkv, n, d_head, K, window))


def focus_attn_topk_workspace_bytes(B: int, Hq: int, Hkv: int, n: int, d_head: int, K: int,
                                    m: int, window: int) -> int:
    return int(lib().focus_attn_topk_workspace_bytes(B, Hq, Hkv, n, d_head, K, m, window))


def _attn_call(fn_name, q, k, v, group_ids, perm, group_offsets, K, window, scale, out,
               out_dtype, lse, want_lse, workspace, stream, needs_groups=True, m=None):
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, Hkv, n, d))
    _need(v, "v", torch.bfloat16, (B, Hkv, n, d))
    mm = 1 if m is None else m
    if needs_groups or group_ids is not None:
        _need(group_ids, "group_ids", torch.int32, (B, n) if m is None else (B, n, m))
    if needs_groups or perm is not None:
        _need(perm, "perm", torch.int32, (B, n * mm))
    if needs_groups or group_offsets is not None:
        _need(group_offsets, "group_offsets", torch.int32, (B, K + 1))
    if out is None:
        out = _new((B, Hq, n, d), out_dtype, q.device, stream)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _need(out, "out", out.dtype, (B, Hq, n, d))
    if lse is None and want_lse:
        lse = _new((B, Hq, n), torch.float32, q.device, stream)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq, n))
    if fn_name == "focus_attn_fwd_sorted_kv":
        nbytes = focus_attn_sorted_kv_workspace_bytes(B, Hq, Hkv, n, d, K, window)
    elif m is None:
        nbytes = focus_attn_workspace_bytes(B, Hq, Hkv, n, d, K, window)
    else:
        nbytes = focus_attn_topk_workspace_bytes(B, Hq, Hkv, n, d, K, m, window)
    ws = _workspace(nbytes, q.device, workspace, stream)
    dt = FOCUS_F32 if out.dtype == torch.float32 else FOCUS_BF16
    fn = getattr(lib(), fn_name)
    shape_args = (B, Hq, Hkv, n, d, K) if m is None else (B, Hq, Hkv, n, d, K, int(m))
    _check_status(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(group_ids), _ptr(perm), _ptr(group_offsets),
                     *shape_args, window, float(scale), _ptr(out), dt, _ptr(lse),
                     _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return out, lse, ws


def focus_attn_fwd(q, k, v, group_ids, perm, group_offsets, K: int, window: int, scale: float,
                   *, out=None, out_dtype=torch.bfloat16, lse=None, want_lse: bool = False,
                   workspace=None, stream=None):
    """Focus attention over the local window plus same-group long-range pairs.
    Returns (out, lse or None)."""
    out, lse, _ = _attn_call("focus_attn_fwd", q, k, v, group_ids, perm, group_offsets, K,
                             window, scale, out, out_dtype, lse, want_lse, workspace, stream)
    return out, lse


def focus_attn_fwd_sorted_kv(q, k, v, group_ids, perm, group_offsets, K: int, window: int,
                             scale: float, *, out=None, out_dtype=torch.bfloat16, lse=None,
                             want_lse: bool = False, workspace=None, stream=None):
    """focus_attn_fwd with the long-range pass reading group-sorted copies of
    K and V (gathered by its preparation) instead of key rows in place; the
    library takes this path by itself only for very long rows. Same result,
    bit for bit. Returns (out, lse or None)."""
    out, lse, _ = _attn_call("focus_attn_fwd_sorted_kv", q, k, v, group_ids, perm, group_offsets,
                             K, window, scale, out, out_dtype, lse, want_lse, workspace, stream)
    return out, lse


def focus_attn_window(q, k, v, K: int, window: int, scale: float, *, workspace,
                      out=None, out_dtype=torch.bfloat16, lse=None, want_lse: bool = False,
                      stream=None):
    """First pass of focus_attn_fwd: the local window. It reads no group data;
    it writes the window partial into workspace (or out/lse directly when no
    pair lies beyond the window)."""
    return _attn_call("focus_attn_window", q, k, v, None, None, None, K, window, scale, out,
                      out_dtype, lse, want_lse, workspace, stream, needs_groups=False)


def focus_attn_long_range_merge(q, k, v, group_ids, perm, group_offsets, K: int, window: int,
                                scale: float, *, workspace, out=None, out_dtype=torch.bfloat16,
                                lse=None, want_lse: bool = False, stream=None):
    """Second pass of focus_attn_fwd: same-group pairs beyond the window,
    merged with the window partial; writes out (and lse)."""
    return _attn_call("focus_attn_long_range_merge", q, k, v, group_ids, perm, group_offsets, K,
                      window, scale, out, out_dtype, lse, want_lse, workspace, stream)


def focus_attn_long_range_prepare(q, k, v, group_ids, perm, group_offsets, K: int, window: int,
                                  scale: float, *, workspace, out, out_dtype=torch.bfloat16,
                                  lse=None, stream=None):
    """First half of focus_attn_long_range_merge: the tile plan and order,
    one packed record per ordered tile (plan record, tile index, each row's
    entry and key-slot end, the first key tile's positions) and, when key
    rows of one head span 2^31 bytes or more, group-sorted K/V copies,
    written into workspace. It reads only k, v and the group data (pass the
    out and lse that the apply call will get), so it may run beside
    focus_attn_window."""
    _attn_call("focus_attn_long_range_prepare", q, k, v, group_ids, perm, group_offsets, K,
               window, scale, out, out_dtype, lse, False, workspace, stream)


def focus_attn_long_range_apply(q, k, v, group_ids, perm, group_offsets, K: int, window: int,
                                scale: float, *, workspace, out=None, out_dtype=torch.bfloat16,
                                lse=None, want_lse: bool = False, stream=None):
    """Second half of focus_attn_long_range_merge, after both
    focus_attn_long_range_prepare and focus_attn_window on this workspace:
    the intra-group attention merged with the window partial."""
    return _attn_call("focus_attn_long_range_apply", q, k, v, group_ids, perm, group_offsets, K,
                      window, scale, out, out_dtype, lse, want_lse, workspace, stream)


def focus_attn_topk_fwd(q, k, v, group_ids, perm, group_offsets, K: int, m: int, window: int,
                        scale: float, *, out=None, out_dtype=torch.bfloat16, lse=None,
                        want_lse: bool = False, workspace=None, stream=None):
    """Focus attention with m groups per token: far pairs are kept when the
    tokens share any group. group_ids (B, n, m); perm (B, n*m) of entries.
    Returns (out, lse or None)."""
    out, lse, _ = _attn_call("focus_attn_topk_fwd", q, k, v, group_ids, perm, group_offsets, K,
                             window, scale, out, out_dtype, lse, want_lse, workspace, stream,
                             m=m)
    return out, lse


def focus_attn_topk_long_range_merge(q, k, v, group_ids, perm, group_offsets, K: int, m: int,
                                     window: int, scale: float, *, workspace, out=None,
                                     out_dtype=torch.bfloat16, lse=None, want_lse: bool = False,
                                     stream=None):
    """Second pass of focus_attn_topk_fwd (after focus_attn_window with the
    same workspace): shared-group pairs beyond the window, one partial per
    membership entry, and the merge into out (and lse)."""
    return _attn_call("focus_attn_topk_long_range_merge", q, k, v, group_ids, perm,
                      group_offsets, K, window, scale, out, out_dtype, lse, want_lse, workspace,
                      stream, m=m)


def focus_attn_topk_long_range_prepare(q, k, v, group_ids, perm, group_offsets, K: int, m: int,
                                       window: int, scale: float, *, workspace, out,
                                       out_dtype=torch.bfloat16, lse=None, stream=None):
    """focus_attn_long_range_prepare for m groups per token."""
    _attn_call("focus_attn_topk_long_range_prepare", q, k, v, group_ids, perm, group_offsets, K,
               window, scale, out, out_dtype, lse, False, workspace, stream, m=m)


def focus_attn_topk_long_range_apply(q, k, v, group_ids, perm, group_offsets, K: int, m: int,
                                     window: int, scale: float, *, workspace, out=None,
                                     out_dtype=torch.bfloat16, lse=None, want_lse: bool = False,
                                     stream=None):
    """focus_attn_long_range_apply for m groups per token."""
    return _attn_call("focus_attn_topk_long_range_apply", q, k, v, group_ids, perm,
                      group_offsets, K, window, scale, out, out_dtype, lse, want_lse, workspace,
                      stream, m=m)


def dense_causal_attn_fwd(q, k, v, scale: float, *, out=None, out_dtype=torch.bfloat16,
                          lse=None, want_lse: bool = False, stream=None):
    """Plain causal attention baseline. Returns (out, lse or None)."""
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, Hkv, n, d))
    _need(v, "v", torch.bfloat16, (B, Hkv, n, d))
    if out is None:
        out = _new((B, Hq, n, d), out_dtype, q.device, stream)
    _need(out, "out", out.dtype, (B, Hq, n, d))
    if lse is None and want_lse:
        lse = _new((B, Hq, n), torch.float32, q.device, stream)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq, n))
    dt = FOCUS_F32 if out.dtype == torch.float32 else FOCUS_BF16
    _check_status(lib().dense_causal_attn_fwd(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, n, d,
                                              float(scale), _ptr(out), dt, _ptr(lse),
                                              _stream(stream)))
    return out, lse


def focus_soft_gate_attn_workspace_bytes(B: int, n: int, K: int) -> int:
    return int(lib().focus_soft_gate_attn_workspace_bytes(B, n, K))


def focus_soft_gate_attn_fwd(q, k, v, G, window: int, scale: float, lam: float, *, out=None,
                             out_dtype=torch.bfloat16, lse=None, want_lse: bool = False,
                             workspace=None, stream=None):
    """Training-time soft-gated attention: every causal pair; pairs beyond the
    window weighted by sigmoid(lam * g_i . g_j) inside the softmax. G (B, n, K)
    fp32 soft assignments. Returns (out, lse or None)."""
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, Hkv, n, d))
    _need(v, "v", torch.bfloat16, (B, Hkv, n, d))
    _need(G, "G", torch.float32)
    if G.dim() != 3 or tuple(G.shape[:2]) != (B, n):
        raise ValueError(f"G must have shape (B, n, K) = ({B}, {n}, K)")
    K = G.shape[2]
    if out is None:
        out = _new((B, Hq, n, d), out_dtype, q.device, stream)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _need(out, "out", out.dtype, (B, Hq, n, d))
    if lse is None and want_lse:
        lse = _new((B, Hq, n), torch.float32, q.device, stream)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq, n))
    ws = _workspace(focus_soft_gate_attn_workspace_bytes(B, n, K), q.device, workspace,
                    stream)
    dt = FOCUS_F32 if out.dtype == torch.float32 else FOCUS_BF16
    _check_status(lib().focus_soft_gate_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(G), B, Hq, Hkv,
                                                 n, d, K, window, float(scale), float(lam),
                                                 _ptr(out), dt, _ptr(lse), _ptr(ws),
                                                 0 if ws is None else ws.numel(),
                                                 _stream(stream)))
    return out, lse


def focus_forward(hidden, P, C, bias, q, k, v, window: int, scale: float, *, m: int = 1,
                  out_dtype=torch.bfloat16, want_lse: bool = False, stream=None):
    """The whole forward pass: assign -> group sort -> attention (m groups
    per token; m = 1 is the plain top-1 pattern)."""
    K = C.shape[0]
    if m == 1:
        ids, _ = focus_assign(hidden, P, C, bias, want_margin=False, stream=stream)
        perm, offs = focus_group_sort(ids, K, stream=stream)
        out, lse = focus_attn_fwd(q, k, v, ids, perm, offs, K, window, scale,
                                  out_dtype=out_dtype, want_lse=want_lse, stream=stream)
    else:
        ids, _ = focus_assign_topk(hidden, P, C, m, bias, want_margin=False, stream=stream)
        perm, offs = focus_group_sort(ids, K, stream=stream)
        out, lse = focus_attn_topk_fwd(q, k, v, ids, perm, offs, K, m, window, scale,
                                       out_dtype=out_dtype, want_lse=want_lse, stream=stream)
    return out, lse, ids, perm, offs
