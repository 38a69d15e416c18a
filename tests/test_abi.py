"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects invalid requests on the host before any HIP call
(no GPU is touched by these tests)."""
import ctypes
import os
import re
import subprocess

import pytest

from group_gated_sparse_amd import focus

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "focus.h")

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3

# Fake device addresses: only ever compared and range-checked on the host.
A = 0x10000000
Bp = 0x20000000
C_ = 0x30000000
D_ = 0x40000000
E_ = 0x50000000
F_ = 0x60000000
G_ = 0x70000000
H_ = 0x80000000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:focus_status|size_t|int|const char\*)\s+(\w+)\s*\(",
                                 text, re.M)))


def test_header_is_plain_c():
    subprocess.check_call(["gcc", "-std=c99", "-fsyntax-only", "-Wall", "-Werror", "-x", "c",
                           HEADER])


def test_library_exports_every_declared_symbol():
    lib = focus.lib()
    names = declared_functions()
    assert len(names) >= 20
    out = subprocess.check_output(["nm", "-D", "--defined-only", focus.LIB_PATH], text=True)
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    for name in names:
        assert name in exported, f"{name} is declared but not exported"
        assert getattr(lib, name) is not None
    assert lib.focus_abi_version() == 4


def _err():
    return focus.lib().focus_last_error().decode()


def _assign(**kw):
    args = dict(hidden=A, P=Bp, C=C_, bias=None, B=1, n=8, d_model=64, d_proj=16, K=4,
                ids=D_, margin=None, ws=E_, wsb=1 << 20, stream=None)
    args.update(kw)
    return focus.lib().focus_assign(args["hidden"], args["P"], args["C"], args["bias"], args["B"],
                                    args["n"], args["d_model"], args["d_proj"], args["K"],
                                    args["ids"], args["margin"], args["ws"], args["wsb"],
                                    args["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(hidden=None), INVALID, "hidden"),
    (dict(hidden=A + 4), INVALID, "aligned"),
    (dict(P=None), INVALID, "P"),
    (dict(ids=None), INVALID, "group_ids"),
    (dict(K=0), UNSUPPORTED, "K"),
    (dict(K=65), UNSUPPORTED, "K"),
    (dict(B=0), INVALID, "B"),
    (dict(n=0), INVALID, "n"),
    (dict(d_model=62), UNSUPPORTED, "multiple of 4"),
    (dict(d_proj=0), INVALID, "d_proj"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(wsb=16), WORKSPACE, "too small"),
    (dict(ids=A + 64), INVALID, "overlap"),
])
def test_assign_rejects(kw, code, msg):
    assert _assign(**kw) == code
    assert msg in _err()


def _assign_topk(m, **kw):
    args = dict(hidden=A, P=Bp, C=C_, bias=None, B=1, n=8, d_model=64, d_proj=16, K=4,
                ids=D_, margin=None, ws=E_, wsb=1 << 20, stream=None)
    args.update(kw)
    return focus.lib().focus_assign_topk(args["hidden"], args["P"], args["C"], args["bias"],
                                         args["B"], args["n"], args["d_model"], args["d_proj"],
                                         args["K"], m, args["ids"], args["margin"], args["ws"],
                                         args["wsb"], args["stream"])


@pytest.mark.parametrize("m,kw,code,msg", [
    (0, {}, UNSUPPORTED, "m must be"),
    (3, dict(K=8), UNSUPPORTED, "m must be"),
    (2, dict(K=1), INVALID, "must be <= K"),
    (2, dict(hidden=None), INVALID, "hidden"),
    (2, dict(wsb=16), WORKSPACE, "too small"),
    # ids [B][n][2] = 64 bytes from D_ - 48 reach into hidden at D_
    (2, dict(hidden=D_, ids=D_ - 48), INVALID, "overlap"),
])
def test_assign_topk_rejects(m, kw, code, msg):
    assert _assign_topk(m, **kw) == code
    assert msg in _err()


def test_workspace_sizes():
    lib = focus.lib()
    # two bf16 tables of [32 or 64][d_model rounded up to 64], each 256-byte aligned
    assert lib.focus_assign_workspace_bytes(64, 4) == 2 * 32 * 64 * 2
    assert lib.focus_assign_workspace_bytes(100, 40) == 2 * 64 * 128 * 2
    assert lib.focus_assign_workspace_bytes(64, 0) == 0
    # per-block group counts: B x ceil(n / 2048) x K int32, 256-byte aligned
    assert lib.focus_group_sort_workspace_bytes(2, 100, 8) == 256
    assert lib.focus_group_sort_workspace_bytes(1, 65536, 64) == 32 * 64 * 4
    # partial fp16 [B][Hq][n][d] + (lse, exponent) fp32 pairs [B][Hq][n] + 128 B plan per query
    # tile (here 64 tokens x 2 heads, 4 tiles) + int32 tile order [B][tiles] + one packed record
    # per tile (64 ints of plan record and tile index, 64 row entries, 64 row key ends, 64
    # positions of a 64-key tile: 256 ints), each region 256-byte aligned; key rows are read in
    # place, so no sorted copies of K and V are reserved
    in_place = 256 * 2 * 32 * 2 + 4096 + 4 * 128 + 256 + 4 * 256 * 4
    assert lib.focus_attn_workspace_bytes(1, 2, 1, 256, 32, 4, 32) == in_place
    # the sorted-copy path adds sorted bf16 K and V [B][Hkv][n][d] and int32 sorted positions
    # [B][n + 256]
    assert lib.focus_attn_sorted_kv_workspace_bytes(1, 2, 1, 256, 32, 4, 32) == (
        in_place + 2 * (256 * 32 * 2) + 512 * 4)
    assert lib.focus_attn_sorted_kv_workspace_bytes(1, 2, 1, 256, 32, 4, 255) == 0
    assert lib.focus_attn_sorted_kv_workspace_bytes(1, 2, 1, 256, 48, 4, 32) == 0
    # the bench workload (70B GQA, n = 32768): no 134 MB of sorted K and V on the in-place path
    big = lib.focus_attn_workspace_bytes(1, 64, 8, 32768, 128, 32, 1024)
    assert lib.focus_attn_sorted_kv_workspace_bytes(1, 64, 8, 32768, 128, 32, 1024) - big == (
        2 * 8 * 32768 * 128 * 2 + (32768 + 256) * 4)
    # no pair can be further apart than the window: no partial needed
    assert lib.focus_attn_workspace_bytes(1, 2, 1, 256, 32, 4, 255) == 0
    assert lib.focus_attn_workspace_bytes(1, 2, 1, 256, 48, 4, 32) == 0
    # top-k, m = 1: the same layout
    assert lib.focus_attn_topk_workspace_bytes(1, 2, 1, 256, 32, 4, 1, 32) == \
        lib.focus_attn_workspace_bytes(1, 2, 1, 256, 32, 4, 32)
    # m = 2, K = 5 (the entry passes): plan and order over the two halves of the query order
    # (4 tiles of 64 entries each), sorted K and V and the slots' (position, other group) words
    # over the 512 membership entries, then the query-order sort (membership index per key
    # slot, the sorted slots, 3 offsets, the sort's per-block counts), the query order's
    # entries and the first pass's partial (fp16 [B][Hq][n][d] and its pairs [B][Hq][n]); no
    # partial per entry
    assert lib.focus_attn_topk_workspace_bytes(1, 2, 1, 256, 32, 5, 2, 32) == (
        256 * 2 * 32 * 2 + 4096 + 8 * 128 + 256 + 2 * (512 * 32 * 2) + 768 * 4
        + 512 * 4 + 512 * 4 + 256 + 256 + 512 * 4 + 256 * 2 * 32 * 2 + 4096)
    # m = 2, K = 4 (six membership sets, the set pass): plan and order over the 256 tokens
    # (4 tiles), set-sorted K and V [B][Hkv][n][d], the slots' (position, group mask) words
    # [B][n + 256], then the set id per token, the set-sorted positions, the 7 set offsets and
    # the sort's per-block counts
    assert lib.focus_attn_topk_workspace_bytes(1, 2, 1, 256, 32, 4, 2, 32) == (
        256 * 2 * 32 * 2 + 4096 + 4 * 128 + 256 + 2 * (256 * 32 * 2) + 512 * 4 + 256 * 4
        + 256 * 4 + 256 + 256)
    assert lib.focus_attn_topk_workspace_bytes(1, 2, 1, 256, 32, 4, 3, 32) == 0
    assert lib.focus_attn_topk_workspace_bytes(1, 2, 1, 256, 32, 4, 2, 255) == 0


def _sort(**kw):
    args = dict(ids=A, B=1, n=16, K=4, perm=Bp, offs=C_, ws=D_, wsb=4096, stream=None)
    args.update(kw)
    return focus.lib().focus_group_sort(args["ids"], args["B"], args["n"], args["K"],
                                        args["perm"], args["offs"], args["ws"], args["wsb"],
                                        args["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(ids=None), INVALID, "group_ids"),
    (dict(perm=None), INVALID, "perm"),
    (dict(offs=None), INVALID, "group_offsets"),
    (dict(K=0), UNSUPPORTED, "K"),
    (dict(K=100), UNSUPPORTED, "K"),
    (dict(n=0), INVALID, "n"),
    (dict(perm=A + 8), INVALID, "overlap"),
    (dict(B=70000), UNSUPPORTED, "B must be"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(wsb=4), WORKSPACE, "too small"),
])
def test_group_sort_rejects(kw, code, msg):
    assert _sort(**kw) == code
    assert msg in _err()


def _attn(fn="focus_attn_fwd", **kw):
    args = dict(q=A, k=Bp, v=C_, ids=D_, perm=E_, offs=F_, B=1, Hq=4, Hkv=2, n=256, d=64, K=4,
                w=16, scale=0.125, out=G_, dt=0, lse=None, ws=H_, wsb=1 << 30, stream=None)
    args.update(kw)
    f = getattr(focus.lib(), fn)
    return f(args["q"], args["k"], args["v"], args["ids"], args["perm"], args["offs"], args["B"],
             args["Hq"], args["Hkv"], args["n"], args["d"], args["K"], args["w"], args["scale"],
             args["out"], args["dt"], args["lse"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("fn", ["focus_attn_fwd", "focus_attn_fwd_sorted_kv", "focus_attn_window",
                                "focus_attn_long_range_merge", "focus_attn_long_range_prepare",
                                "focus_attn_long_range_apply"])
@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), INVALID, "q"),
    (dict(k=Bp + 8), INVALID, "aligned"),
    (dict(out=None), INVALID, "out"),
    (dict(d=48), UNSUPPORTED, "d_head"),
    (dict(d=256), UNSUPPORTED, "d_head"),
    (dict(Hq=3), INVALID, "multiple"),
    (dict(K=0), UNSUPPORTED, "K"),
    (dict(K=65), UNSUPPORTED, "K"),
    (dict(w=-1), INVALID, "window"),
    (dict(n=0), INVALID, "n"),
    (dict(B=0), INVALID, "B"),
    (dict(scale=0.0), INVALID, "scale"),
    (dict(scale=-1.0), INVALID, "scale"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(scale=float("inf")), INVALID, "scale"),
    (dict(dt=7), INVALID, "out_dtype"),
    (dict(out=A + 1024), INVALID, "overlap"),
    (dict(lse=G_ + 64), INVALID, "overlap"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(wsb=1024), WORKSPACE, "too small"),
    (dict(ws=A + 4096), INVALID, "workspace must not overlap"),
])
def test_attn_rejects(fn, kw, code, msg):
    assert _attn(fn, **kw) == code
    assert msg in _err()


@pytest.mark.parametrize("fn", ["focus_attn_fwd", "focus_attn_fwd_sorted_kv",
                                "focus_attn_long_range_merge", "focus_attn_long_range_prepare",
                                "focus_attn_long_range_apply"])
@pytest.mark.parametrize("kw,msg", [(dict(ids=None), "group_ids"), (dict(perm=None), "perm"),
                                    (dict(offs=None), "group_offsets")])
def test_attn_passes_needing_groups_reject_missing_group_data(fn, kw, msg):
    assert _attn(fn, **kw) == INVALID
    assert msg in _err()


def _attn_topk(fn="focus_attn_topk_fwd", m=2, **kw):
    args = dict(q=A, k=Bp, v=C_, ids=D_, perm=E_, offs=F_, B=1, Hq=4, Hkv=2, n=256, d=64, K=4,
                w=16, scale=0.125, out=G_, dt=0, lse=None, ws=H_, wsb=1 << 30, stream=None)
    args.update(kw)
    f = getattr(focus.lib(), fn)
    return f(args["q"], args["k"], args["v"], args["ids"], args["perm"], args["offs"], args["B"],
             args["Hq"], args["Hkv"], args["n"], args["d"], args["K"], m, args["w"],
             args["scale"], args["out"], args["dt"], args["lse"], args["ws"], args["wsb"],
             args["stream"])


@pytest.mark.parametrize("fn", ["focus_attn_topk_fwd", "focus_attn_topk_long_range_merge",
                                "focus_attn_topk_long_range_prepare",
                                "focus_attn_topk_long_range_apply"])
@pytest.mark.parametrize("m,kw,code,msg", [
    (0, {}, UNSUPPORTED, "m must be"),
    (3, dict(K=8), UNSUPPORTED, "m must be"),
    (2, dict(K=1), INVALID, "must be <= K"),
    (2, dict(n=(1 << 23) + 1), UNSUPPORTED, "n * m"),
    (2, dict(ids=None), INVALID, "group_ids"),
    (2, dict(perm=None), INVALID, "perm"),
    (2, dict(d=48), UNSUPPORTED, "d_head"),
    (2, dict(scale=0.0), INVALID, "scale"),
    (2, dict(ws=None), WORKSPACE, "workspace"),
    # enough for m = 1 but not for the sorted K/V of m = 2 (K = 5: the entry passes)
    (2, dict(wsb=400000, K=5), WORKSPACE, "too small"),
    # K = 4 (the set pass): one byte short of its own size
    (2, dict(wsb=275711), WORKSPACE, "too small"),
])
def test_attn_topk_rejects(fn, m, kw, code, msg):
    if kw.get("wsb") == 400000:
        need1 = focus.lib().focus_attn_workspace_bytes(1, 4, 2, 256, 64, 5, 16)
        need2 = focus.lib().focus_attn_topk_workspace_bytes(1, 4, 2, 256, 64, 5, 2, 16)
        assert need1 <= 400000 < need2
    if kw.get("wsb") == 275711:
        assert focus.lib().focus_attn_topk_workspace_bytes(1, 4, 2, 256, 64, 4, 2, 16) == 275712
    assert _attn_topk(fn, m, **kw) == code
    assert msg in _err()


def _sink(**kw):
    args = dict(S=A, B=1, n=100, K=8, tau=1.0, iters=5, G=Bp, ws=C_, wsb=1 << 20, stream=None)
    args.update(kw)
    return focus.lib().focus_sinkhorn(args["S"], args["B"], args["n"], args["K"], args["tau"],
                                      args["iters"], args["G"], args["ws"], args["wsb"],
                                      args["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(S=None), INVALID, "scores"),
    (dict(G=None), INVALID, "G"),
    (dict(G=A + 64), INVALID, "overlap"),
    (dict(K=0), UNSUPPORTED, "K"),
    (dict(K=65), UNSUPPORTED, "K"),
    (dict(n=0), INVALID, "n"),
    (dict(B=70000), UNSUPPORTED, "B must be"),
    (dict(iters=-1), INVALID, "iters"),
    (dict(iters=10001), INVALID, "iters"),
    (dict(tau=0.0), INVALID, "tau"),
    (dict(tau=float("nan")), INVALID, "tau"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(wsb=16), WORKSPACE, "too small"),
    (dict(ws=A + 256), INVALID, "overlap"),
])
def test_sinkhorn_rejects(kw, code, msg):
    assert _sink(**kw) == code
    assert msg in _err()


def test_sinkhorn_workspace_size():
    lib = focus.lib()
    # column scales [B][K] + two buffers of per-workgroup column sums [B][nblk][K]
    # (128 rows per workgroup, at most 2048 workgroups), each region 256-byte aligned
    assert lib.focus_sinkhorn_workspace_bytes(1, 100, 8, 5) == 3 * 256
    assert lib.focus_sinkhorn_workspace_bytes(2, 32768, 32, 10) == 256 + 2 * (2 * 256 * 32 * 4)
    # 1M rows: 512-row workgroups, 2048 of them
    assert lib.focus_sinkhorn_workspace_bytes(1, 1 << 20, 64, 10) == 256 + 2 * (2048 * 64 * 4)
    assert lib.focus_sinkhorn_workspace_bytes(1, 100, 0, 5) == 0


def _sg(**kw):
    args = dict(q=A, k=Bp, v=C_, G=D_, B=1, Hq=4, Hkv=2, n=256, d=64, K=8, w=16, scale=0.125,
                lam=4.0, out=G_, dt=0, lse=None, ws=H_, wsb=1 << 20, stream=None)
    args.update(kw)
    return focus.lib().focus_soft_gate_attn_fwd(
        args["q"], args["k"], args["v"], args["G"], args["B"], args["Hq"], args["Hkv"], args["n"],
        args["d"], args["K"], args["w"], args["scale"], args["lam"], args["out"], args["dt"],
        args["lse"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(G=None), INVALID, "G"),
    (dict(G=D_ + 2), INVALID, "aligned"),
    (dict(lam=float("nan")), INVALID, "lambda"),
    (dict(lam=float("inf")), INVALID, "lambda"),
    (dict(K=0), UNSUPPORTED, "K"),
    (dict(K=65), UNSUPPORTED, "K"),
    (dict(d=48), UNSUPPORTED, "d_head"),
    (dict(q=None), INVALID, "q"),
    (dict(scale=0.0), INVALID, "scale"),
    (dict(out=D_), INVALID, "overlap"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(wsb=64), WORKSPACE, "too small"),
])
def test_soft_gate_rejects(kw, code, msg):
    assert _sg(**kw) == code
    assert msg in _err()


def test_soft_gate_workspace_size():
    lib = focus.lib()
    # bf16 hi and lo rows of the assignments, K padded to 16 / 32 / 64
    assert lib.focus_soft_gate_attn_workspace_bytes(1, 256, 8) == 256 * 4 * 16
    assert lib.focus_soft_gate_attn_workspace_bytes(2, 1000, 20) == 2 * 1000 * 4 * 32
    assert lib.focus_soft_gate_attn_workspace_bytes(1, 100, 33) == 25600
    assert lib.focus_soft_gate_attn_workspace_bytes(1, 100, 65) == 0


def test_assign_scores_rejects():
    f = focus.lib().focus_assign_scores
    assert f(A, Bp, C_, None, 1, 8, 64, 16, 4, None, E_, 1 << 20, None) == INVALID
    assert "scores" in _err()
    assert f(A, Bp, C_, None, 1, 8, 64, 16, 4, A + 64, E_, 1 << 20, None) == INVALID
    assert "overlap" in _err()
    assert f(A, Bp, C_, None, 1, 8, 64, 16, 0, D_, E_, 1 << 20, None) == UNSUPPORTED


def test_sorted_kv_call_needs_the_larger_workspace():
    """focus_attn_fwd_sorted_kv validates against its own, larger workspace
    size: the in-place size is rejected before anything is enqueued."""
    lib = focus.lib()
    small = lib.focus_attn_workspace_bytes(1, 4, 2, 256, 64, 4, 16)
    big = lib.focus_attn_sorted_kv_workspace_bytes(1, 4, 2, 256, 64, 4, 16)
    assert small < big
    assert _attn("focus_attn_fwd_sorted_kv", wsb=small) == WORKSPACE
    assert "too small" in _err()
    assert _attn("focus_attn_fwd_sorted_kv", wsb=big - 1) == WORKSPACE


def test_window_pass_takes_no_group_data():
    """The window pass reads no group data, so NULL ids / perm / offsets pass
    validation; a bad request is still rejected on its own merits (here the
    workspace is too small, after the group pointers were skipped)."""
    assert _attn("focus_attn_window", ids=None, perm=None, offs=None, wsb=1024) == WORKSPACE
    assert "too small" in _err()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), INVALID, "q"),
    (dict(d=16), UNSUPPORTED, "d_head"),
    (dict(Hkv=3), INVALID, "multiple"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(out=Bp), INVALID, "overlap"),
])
def test_dense_rejects(kw, code, msg):
    args = dict(q=A, k=Bp, v=C_, B=1, Hq=4, Hkv=2, n=256, d=64, scale=0.125, out=G_, dt=0,
                lse=None, stream=None)
    args.update(kw)
    rc = focus.lib().dense_causal_attn_fwd(args["q"], args["k"], args["v"], args["B"], args["Hq"],
                                           args["Hkv"], args["n"], args["d"], args["scale"],
                                           args["out"], args["dt"], args["lse"], args["stream"])
    assert rc == code
    assert msg in _err()


def test_error_text_is_thread_local():
    import threading
    assert _sort(K=0) == UNSUPPORTED
    seen = {}

    def other():
        seen["text"] = _err()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["text"] == "" and "K must be" in _err()
