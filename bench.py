"""Benchmark of the Focus forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--skip-cpu-baseline] [--skip-dense] [--cold-mall] [--graph]

One step = the whole hot path on one batch of seeded synthetic input already
resident in HBM, all through the C ABI: focus_assign -> focus_group_sort ->
focus_attn_long_range_prepare (the tile plan) on the main stream, with
focus_attn_window (the window pass, which needs no group data) enqueued on a
second stream right after focus_assign, so that both run together; then,
once both are done, focus_attn_long_range_apply on the main stream (together the calls are
focus_attn_fwd). --no-overlap runs all five calls in order on one stream.
The window pass either starts at once beside the assignment (schedule
"beside") or waits for the assignment to finish and then runs beside the sort
and prepare calls (schedule "after_assign"): where the assignment is short
next to the window pass, sharing the GPU with it stretches the assignment
so far that the chain assign -> sort -> prepare outlasts the window pass.
--schedule auto (the default) times a few steps of each after the warm-up
and keeps the faster; the timed steps then all use it (with --graph the
replayed graph is chosen the same way, from replays of each).
Workloads with m = 2 groups per token use focus_assign_topk, the sort of the
n*m membership entries and the focus_attn_topk_long_range_* calls instead.
W untimed warm-up steps, then K timed steps between two device
synchronisations. Per-call times come from HIP events recorded around each
call, on the stream it runs on, inside the timed loop.

Prints ONE JSON line. value = visited-pair TFLOP/s of the whole step
(4*d flops per allowed (query head, i, j) pair / step time). Also reported:
attention-only TFLOP/s, the dense causal baseline (dense_causal_attn_fwd) and
the speedups over it, the roofline of the dominant kernel, the pairs the
kernels' tiles compute (masked ones included) with the tile utilization and
computed-tile TFLOP/s of each pass, and the CPU oracle timed on a bounded
sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Focus attn visited-pair TFLOP/s + speedup vs dense causal, n=32K, 1 GPU"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="70b_gqa_n32768")
    ap.add_argument("--dense-iters", type=int, default=5)
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-dense", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle attention sample")
    ap.add_argument("--no-overlap", action="store_true",
                    help="run the window pass on the main stream, after the sort")
    ap.add_argument("--schedule", default="auto", choices=["auto", "beside", "after_assign"],
                    help="when the window pass starts on its stream: beside the assignment, "
                         "or after it; auto picks the faster after the warm-up")
    ap.add_argument("--op", default="attn", choices=["attn", "sinkhorn", "soft_gate"],
                    help="attn: the inference forward step (default); sinkhorn: the "
                         "training-time soft assignment (scores + Sinkhorn rounds); "
                         "soft_gate: the training-time soft-gated attention forward")
    ap.add_argument("--lam", type=float, default=8.0, help="gate slope (--op soft_gate)")
    ap.add_argument("--iters", type=int, default=10, help="Sinkhorn rounds (--op sinkhorn)")
    ap.add_argument("--tau", type=float, default=1.0, help="Sinkhorn temperature (--op sinkhorn)")
    ap.add_argument("--cold-mall", action="store_true",
                    help="write a 512 MiB buffer before each timed step (outside its events), "
                         "so the step starts with nothing of its inputs in the 256 MB "
                         "Infinity Cache; the step time is then the HIP-event time")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one whole step (both streams) into a HIP graph and time "
                         "its replays; value and ms_per_step are then the replayed step's, the "
                         "per-call times and the roofline come from the eager pass")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (a reference "
                         "dispatch for calibrating HBM byte counters)")
    return ap.parse_args()


TRAFFIC_SOURCES = ("group_gated_sparse_amd/csrc/attn.hip", "group_gated_sparse_amd/csrc/focus_internal.h",
                   "group_gated_sparse_amd/csrc/assign.hip", "group_gated_sparse_amd/csrc/sort.hip",
                   "group_gated_sparse_amd/csrc/sinkhorn.hip", "group_gated_sparse_amd/build.py")


def measured_traffic(key, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/hbm_traffic_<key>.txt, key = the workload's name, or
    "<op>_<workload>" for the training-time ops: FETCH_SIZE and WRITE_SIZE
    scaled by a plain-copy calibration), or None when there is none or it was
    taken on kernel sources other than the ones in this tree."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{key}.txt")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    sha, value = None, None
    for line in open(path):
        if line.startswith("sources_sha256:"):
            sha = line.split(":", 1)[1].strip()
        elif line.startswith(f"kernel {kernel}:"):
            value = float(line.split("hbm_bytes")[1].split()[0])
    return value if sha == h.hexdigest() else None


def copy_probe(torch, res):
    """One plain 1 GiB device-to-device copy after the timed work: a dispatch
    of known size for calibrating the HBM byte counters of a profiled run."""
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    res["copy_probe_bytes"] = src.numel() * 4
    del src, dst


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count}


def host_cpu():
    """The host CPU's model name and logical core count (the oracle's
    OpenMP thread count is reported separately as cores)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cores": os.cpu_count()}


def cpu_baseline(x, wl, target_s):
    """The oracle as it stands, on the host cores: full assignment and group
    sort, attention on a random row sample extrapolated per visited pair."""
    import oracle
    from group_gated_sparse_amd import metrics
    cores = oracle.max_threads()
    t0 = time.perf_counter()
    if wl.m == 1:
        ids, _ = oracle.assign(x["hidden"], x["P"], x["C"], x["bias"])
    else:
        ids, _ = oracle.assign_topk(x["hidden"], x["P"], x["C"], wl.m, x["bias"])
    t_assign = time.perf_counter() - t0
    t0 = time.perf_counter()
    if wl.m == 1:
        oracle.group_sort(ids, wl.K)
    else:
        oracle.group_sort_multi(ids, wl.K)
    t_sort = time.perf_counter() - t0
    attend = oracle.attn if wl.m == 1 else oracle.attn_multi
    rng = np.random.default_rng(7)
    total_rows = wl.B * wl.Hq * wl.n
    rows_done = 0
    pairs_done = 0
    t_attn = 0.0
    batch = 2048
    while t_attn < target_s and rows_done < total_rows:
        rows = rng.integers(0, total_rows, size=batch)
        t0 = time.perf_counter()
        _, _, vis = attend(x["q"], x["k"], x["v"], ids, wl.w, wl.softmax_scale, rows=rows)
        t_attn += time.perf_counter() - t0
        rows_done += batch
        pairs_done += int(vis.sum())
        if t_attn > 0:
            batch = int(min(max(batch, batch * (target_s - t_attn) / t_attn), 262144))
            batch = max(batch, 256)
    if wl.m == 1:
        win, lr = metrics.pair_counts(ids, wl.w)
    else:
        win, lr, _ = metrics.pair_counts_multi(ids, wl.w)
    pairs_all = (win + lr) * wl.Hq
    t_attn_all = t_attn * pairs_all / max(pairs_done, 1)
    step_s = t_assign + t_sort + t_attn_all
    flops = metrics.attn_flops(win + lr, wl.Hq, wl.d)
    return {
        "value": flops / step_s / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "host_cpu": host_cpu(),
        "kind": "oracle",
        "sample": (f"full fp32 assignment ({wl.B * wl.n} tokens, {t_assign:.2f} s) and group sort "
                   f"({t_sort:.3f} s); fp64 attention on {rows_done} random query rows "
                   f"({pairs_done} visited pairs, {t_attn:.2f} s) extrapolated per visited pair "
                   f"to all {pairs_all} pairs ({t_attn_all:.1f} s); step estimate {step_s:.1f} s"),
        "step_s": step_s,
    }


def bench_sinkhorn(args, wl):
    """Soft assignment step: focus_assign_scores then focus_sinkhorn (iters
    rounds), timed with HIP events per call; one JSON line."""
    import torch
    from group_gated_sparse_amd import focus, metrics, synth
    log(f"workload {wl.name}: generating hidden states")
    x = synth.make_inputs(wl, with_qkv=False)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    hidden, P, C = dev(x["hidden"]), dev(x["P"]), dev(x["C"])
    bias = None if x["bias"] is None else dev(x["bias"])
    B, n, K, T = wl.B, wl.n, wl.K, args.iters
    S = torch.empty((B, n, K), dtype=torch.float32, device="cuda")
    G = torch.empty_like(S)
    ws_a = torch.empty(focus.focus_assign_workspace_bytes(wl.d_model, K), dtype=torch.uint8,
                       device="cuda")
    ws_s = torch.empty(focus.focus_sinkhorn_workspace_bytes(B, n, K, T), dtype=torch.uint8,
                       device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        focus.focus_assign_scores(hidden, P, C, bias, scores=S, workspace=ws_a)
        if ev is not None:
            ev[1].record()
        focus.focus_sinkhorn(S, args.tau, T, G=G, workspace=ws_s)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    sc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    sk_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms = max(wall_ms, sc_ms + sk_ms)
    log(f"step {ms:.4f} ms: scores {sc_ms:.4f} ms, sinkhorn {sk_ms:.4f} ms ({T} rounds)")
    # algorithmic bytes of one Sinkhorn call: every pass reads the scores once,
    # the last also writes G
    sk_bytes = (T + 1) * B * n * K * 4 + B * n * K * 4
    # the scores kernel: one 32-group block of the split W^T per workgroup
    # pass up to 32 groups, two beyond
    sc_kernel = f"assign_argmax_kernel<{1 if K <= 32 else 2},0>"
    res = {
        "metric": "Sinkhorn soft assignment (scores + rounds), tokens/s, 1 GPU",
        "value": B * n / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "op": "sinkhorn", "B": B, "n": n, "K": K,
                   "d_model": wl.d_model, "d_proj": wl.d_proj, "iters": T, "tau": args.tau},
        "phase_ms": {"scores": sc_ms, "sinkhorn": sk_ms},
        "roofline": {"kernel": f"{sc_kernel} (scores)", "bound": "hbm",
                     "achieved": B * n * wl.d_model * 4 / (sc_ms * 1e-3) / 1e9,
                     "peak": metrics.MI355X_HBM_GBPS, "unit": "GB/s",
                     "frac": B * n * wl.d_model * 4 / (sc_ms * 1e-3) / 1e9 / metrics.MI355X_HBM_GBPS,
                     "traffic": measured_traffic(f"sinkhorn_{wl.name}", sc_kernel),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)"},
        "sinkhorn_roofline": {"kernel": "sinkhorn_pass_kernel x (iters + 1)", "bound": "hbm",
                              "achieved": sk_bytes / (sk_ms * 1e-3) / 1e9,
                              "peak": metrics.MI355X_HBM_GBPS, "unit": "GB/s",
                              "frac": sk_bytes / (sk_ms * 1e-3) / 1e9 / metrics.MI355X_HBM_GBPS,
                              "bytes_per_call": sk_bytes},
    }
    if args.copy_probe:
        copy_probe(torch, res)
    if not args.skip_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        rows = min(n, 4096)
        Sh = S.cpu().numpy()[:, :rows]
        oracle.sinkhorn(Sh, args.tau, T)
        t_s = (time.perf_counter() - t0) * n / rows
        t0 = time.perf_counter()
        oracle.assign_scores(x["hidden"][:, :rows], x["P"], x["C"], x["bias"])
        t_a = (time.perf_counter() - t0) * n / rows
        res["cpu_baseline"] = {"value": B * n / (t_s + t_a), "unit": "tokens/s",
                               "cores": oracle.max_threads(), "host_cpu": host_cpu(),
                               "kind": "oracle",
                               "sample": f"oracle scores and Sinkhorn ({T} rounds) on the first "
                                         f"{rows} tokens of each sequence, scaled by n / {rows}"}
    print(json.dumps(res), flush=True)


def bench_soft_gate(args, wl):
    """Training-time soft-gated attention forward on the workload's shape,
    with G = Sinkhorn soft assignments of its hidden states (computed once,
    outside the timed region); one JSON line, dense causal beside it."""
    import torch
    from group_gated_sparse_amd import focus, metrics, synth
    log(f"workload {wl.name}: generating seeded inputs")
    x = synth.make_inputs(wl)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    S = focus.focus_assign_scores(dev(x["hidden"]), dev(x["P"]), dev(x["C"]),
                                  None if x["bias"] is None else dev(x["bias"]))
    G = focus.focus_sinkhorn(S, args.tau, args.iters)
    del S
    q, k, v = dev16(x["q"]), dev16(x["k"]), dev16(x["v"])
    B, n, d, Hq, K, w = wl.B, wl.n, wl.d, wl.Hq, wl.K, wl.w
    out = torch.empty((B, Hq, n, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(focus.focus_soft_gate_attn_workspace_bytes(B, n, K), dtype=torch.uint8,
                     device="cuda")

    def call():
        focus.focus_soft_gate_attn_fwd(q, k, v, G, w, wl.softmax_scale, args.lam, out=out,
                                       workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    ms = max(wall_ms, ev_ms)
    pairs = B * (n * (n + 1) // 2)
    flops = metrics.attn_flops(pairs, Hq, d)
    ww = min(w, n - 1)
    far = pairs - B * (n * (ww + 1) - ww * (ww + 1) // 2)
    KG = 16 if K <= 16 else (32 if K <= 32 else 64)
    log(f"soft gate {ms:.3f} ms ({flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s on causal pairs)")
    res = {
        "metric": "Soft-gated attention forward TFLOP/s (causal pairs), 1 GPU",
        "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "op": "soft_gate", "B": B, "Hq": Hq, "Hkv": wl.Hkv,
                   "n": n, "d_head": d, "K": K, "window": w, "lambda": args.lam,
                   "sinkhorn_iters": args.iters, "tau": args.tau, "out_dtype": "bf16"},
        "causal_pairs_per_head": pairs, "far_pairs_per_head": far,
        "affinity_flops": 3 * 2 * KG * far * Hq,
        "roofline": {"kernel": f"attn_kernel<{d},{4 + (KG // 32)}> (soft-gated pass)",
                     "bound": "mfma", "achieved": flops / (ms * 1e-3) / 1e12,
                     "peak": metrics.MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / (ms * 1e-3) / 1e12 / metrics.MI355X_BF16_DENSE_TFLOPS,
                     "traffic": measured_traffic(f"soft_gate_{wl.name}",
                                                 f"attn_kernel<{d},{4 + (KG // 32)}>"),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "flops_per_launch": flops, "avg_launch_ms": ev_ms},
    }
    if not args.skip_dense:
        focus.dense_causal_attn_fwd(q, k, v, wl.softmax_scale, out=out)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.dense_iters):
            focus.dense_causal_attn_fwd(q, k, v, wl.softmax_scale, out=out)
        e1.record()
        torch.cuda.synchronize()
        res["dense_ms"] = e0.elapsed_time(e1) / args.dense_iters
        res["gate_overhead_vs_dense"] = ms / res["dense_ms"]
        log(f"dense {res['dense_ms']:.3f} ms")
    if args.copy_probe:
        copy_probe(torch, res)
    if not args.skip_cpu_baseline:
        import oracle
        rng = np.random.default_rng(7)
        rows = rng.integers(0, B * Hq * n, size=4096)
        g_host = G.cpu().numpy()
        t0 = time.perf_counter()
        oracle.soft_gate_attn(x["q"], x["k"], x["v"], g_host, w, wl.softmax_scale, args.lam,
                              rows=rows)
        t = time.perf_counter() - t0
        i = rows % n
        done = int((i + 1).sum())
        res["cpu_baseline"] = {"value": metrics.attn_flops(done, 1, d) / t / 1e12,
                               "unit": "TFLOP/s", "cores": oracle.max_threads(), "host_cpu": host_cpu(),
                               "kind": "oracle",
                               "sample": f"fp64 oracle on 4096 random query rows ({done} causal "
                                         f"pairs, {t:.1f} s)"}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs on one GPU "
              "(the design notes describe how the work would shard). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from group_gated_sparse_amd import focus, metrics, synth, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = workloads.BY_NAME[args.workload]
    if args.op == "sinkhorn":
        return bench_sinkhorn(args, wl)
    if args.op == "soft_gate":
        return bench_soft_gate(args, wl)
    log(f"workload {wl.name}: generating seeded inputs")
    t0 = time.perf_counter()
    x = synth.make_inputs(wl)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; uploading")

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    hidden, P, C = dev(x["hidden"]), dev(x["P"]), dev(x["C"])
    bias = None if x["bias"] is None else dev(x["bias"])
    q, k, v = dev16(x["q"]), dev16(x["k"]), dev16(x["v"])
    B, n, K, w, d, Hq, Hkv, m = wl.B, wl.n, wl.K, wl.w, wl.d, wl.Hq, wl.Hkv, wl.m
    scale = wl.softmax_scale
    dv = q.device
    ids = torch.empty((B, n) if m == 1 else (B, n, m), dtype=torch.int32, device=dv)
    perm = torch.empty((B, n * m), dtype=torch.int32, device=dv)
    offs = torch.empty((B, K + 1), dtype=torch.int32, device=dv)
    out = torch.empty((B, Hq, n, d), dtype=torch.bfloat16, device=dv)
    ws_a = torch.empty(focus.focus_assign_workspace_bytes(wl.d_model, K), dtype=torch.uint8,
                       device=dv)
    ws_s = torch.empty(max(focus.focus_group_sort_workspace_bytes(B, n * m, K), 1),
                       dtype=torch.uint8, device=dv)
    if m == 1:
        ws_n = focus.focus_attn_workspace_bytes(B, Hq, Hkv, n, d, K, w)
    else:
        ws_n = focus.focus_attn_topk_workspace_bytes(B, Hq, Hkv, n, d, K, m, w)
    ws_t = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dv)
    stream = torch.cuda.current_stream()

    side = torch.cuda.Stream()   # default priority
    overlap = not args.no_overlap
    # events: 0 step start, 1 assign end, 2 sort end, 7 prepare end, 3 apply start, 4 step
    # end (main stream); 5 window start, 6 window end (the stream the window pass runs on)
    NEV = 8

    def assign():
        if m == 1:
            focus.focus_assign(hidden, P, C, bias, group_ids=ids, want_margin=False,
                               workspace=ws_a)
        else:
            focus.focus_assign_topk(hidden, P, C, m, bias, group_ids=ids, want_margin=False,
                                    workspace=ws_a)

    def prepare():
        if m == 1:
            focus.focus_attn_long_range_prepare(q, k, v, ids, perm, offs, K, w, scale,
                                                workspace=ws_t, out=out)
        else:
            focus.focus_attn_topk_long_range_prepare(q, k, v, ids, perm, offs, K, m, w, scale,
                                                     workspace=ws_t, out=out)

    def long_range():
        if m == 1:
            focus.focus_attn_long_range_apply(q, k, v, ids, perm, offs, K, w, scale,
                                              workspace=ws_t, out=out)
        else:
            focus.focus_attn_topk_long_range_apply(q, k, v, ids, perm, offs, K, m, w, scale,
                                                   workspace=ws_t, out=out)

    schedule = "beside" if args.schedule == "auto" else args.schedule

    def step(evs=None):
        stream = torch.cuda.current_stream()   # the capture stream under --graph
        def mark(i, st):
            if evs is not None:
                evs[i].record(st)
        ws_stream = side if overlap else stream
        mark(0, stream)
        if overlap:
            side.wait_stream(stream)   # the previous apply has consumed the workspace
            # the assignment is enqueued ahead of the window pass, so its short
            # workgroups are dispatched first instead of waiting for the window
            # pass's to retire one by one
            assign()
            mark(1, stream)
            if schedule == "after_assign":
                side.wait_stream(stream)
        else:
            assign()
            mark(1, stream)
            focus.focus_group_sort(ids, K, perm=perm, group_offsets=offs, workspace=ws_s)
            mark(2, stream)
            prepare()
            mark(7, stream)
        mark(5, ws_stream)
        focus.focus_attn_window(q, k, v, K, w, scale, workspace=ws_t, out=out, stream=ws_stream)
        mark(6, ws_stream)
        if overlap:
            focus.focus_group_sort(ids, K, perm=perm, group_offsets=offs, workspace=ws_s)
            mark(2, stream)
            prepare()
            mark(7, stream)
            stream.wait_stream(side)
        mark(3, stream)
        long_range()
        mark(4, stream)

    log(f"warm-up {args.warmup} steps ({'overlapped' if overlap else 'one stream'})")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    probe = None
    if overlap and args.schedule == "auto":
        # part of the warm-up: a few steps of each schedule, the faster is kept
        probe = {}
        for sc in ("beside", "after_assign", "beside", "after_assign"):
            schedule = sc
            ts = []
            for _ in range(5):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                step()
                torch.cuda.synchronize()
                ts.append((time.perf_counter() - t0) * 1e3)
            probe.setdefault(sc, []).extend(ts)
        probe = {sc: float(np.median(ts)) for sc, ts in probe.items()}
        schedule = min(probe, key=probe.get)
        log(f"schedule {schedule} (median ms of 10 steps each: {probe})")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(NEV)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    flush = torch.empty(1 << 27, dtype=torch.float32, device=dv) if args.cold_mall else None
    for s in range(args.steps):
        if flush is not None:
            flush.fill_(float(s))
        step(evs[s])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    del flush

    def span(i, j):
        return float(np.mean([evs[s][i].elapsed_time(evs[s][j]) for s in range(args.steps)]))
    phase = {"assign": span(0, 1), "sort": span(1, 2), "long_range_prepare": span(2, 7),
             "window": span(5, 6), "long_range_apply": span(3, 4)}
    ev_step = span(0, 4)
    ms_step = ev_step if args.cold_mall else max(wall_ms, ev_step)
    per_step = sorted(evs[s][0].elapsed_time(evs[s][4]) for s in range(args.steps))
    eager_ms = ms_step
    if args.graph:
        # The whole step captured once (window on the second stream, the rest on
        # the capture stream) and replayed; the replay must equal the eager result.
        if args.cold_mall:
            raise SystemExit("--graph and --cold-mall are exclusive")
        ref_out = out.clone()
        eager_schedule = schedule

        def capture():
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step()
            for _ in range(max(args.warmup, 1)):
                gr.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, ref_out):
                raise RuntimeError("the replayed step differs from the eager step")
            return gr

        graph_probe = None
        if overlap and args.schedule == "auto":
            # the replayed graph may favour another schedule than eager launches:
            # time a few replays of each and keep the faster
            graph_probe = {}
            for sc in ("beside", "after_assign"):
                schedule = sc
                gr = capture()
                pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                pe0.record(stream)
                for _ in range(10):
                    gr.replay()
                pe1.record(stream)
                torch.cuda.synchronize()
                graph_probe[sc] = pe0.elapsed_time(pe1) / 10
                del gr
            schedule = min(graph_probe, key=graph_probe.get)
            log(f"graph schedule {schedule} (ms per replay: {graph_probe})")
        g = capture()
        ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ge0.record(stream)
        for _ in range(args.steps):
            g.replay()
        ge1.record(stream)
        torch.cuda.synchronize()
        g_wall = (time.perf_counter() - t0) * 1e3 / args.steps
        ms_step = max(g_wall, ge0.elapsed_time(ge1) / args.steps)
        log(f"graph replay: {ms_step:.4f} ms per step (eager {eager_ms:.4f})")
        del g, ref_out
        graph_schedule = schedule
        schedule = eager_schedule
    log(f"step {ms_step:.3f} ms (events {ev_step:.3f}, wall {wall_ms:.3f}); phases {phase}")

    gids = ids.cpu().numpy()
    if m == 1:
        win, lr = metrics.pair_counts(gids, w)
        lr_visited = lr
    else:
        win, lr, lr_visited = metrics.pair_counts_multi(gids, w)
        if metrics.uses_set_pass(K, m):
            lr_visited = lr   # the set pass meets each kept pair once
    pairs = win + lr
    flops = metrics.attn_flops(pairs, Hq, d)
    # the two attention passes; the tile plan (prepare) runs beside the window
    # pass in the step and is reported apart as plan_ms
    attn_ms = phase["window"] + phase["long_range_apply"]
    plan_ms = phase["long_range_prepare"]
    # pairs the kernels' MFMAs form, masked ones included (their tiling)
    tt = 128 // metrics.heads_per_workgroup(Hq, Hkv)
    bn = metrics.tile_keys(d)
    cwin = B * metrics.window_computed_pairs(n, w, tt, bn)
    if metrics.uses_set_pass(K, m):
        clr = metrics.set_long_range_computed_pairs(gids, K, w, tt, bn)
    elif m == 2:
        clr = metrics.entry_long_range_computed_pairs(gids.reshape(B, n * m), perm.cpu().numpy(),
                                                      offs.cpu().numpy(), w, tt, bn)
    else:
        clr = metrics.long_range_computed_pairs(gids.reshape(B, n), perm.cpu().numpy(),
                                                offs.cpu().numpy(), w, tt, bn)
    res = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "Hq": Hq, "Hkv": Hkv, "n": n, "d_head": d,
                   "d_model": wl.d_model, "d_proj": wl.d_proj, "K": K, "window": w,
                   "groups_per_token": m, "out_dtype": "bf16",
                   "mall": "cold (512 MiB written before each step)" if args.cold_mall
                   else "warm",
                   "launch": "HIP graph of the whole step, replayed" if args.graph else "eager",
                   "streams": "window pass overlapped with assign+sort" if overlap
                   else "one stream",
                   "schedule": schedule if overlap else None,
                   "graph_schedule": graph_schedule if (overlap and args.graph) else None},
        "visited_pairs_per_head": pairs,
        "window_pairs_per_head": win,
        "long_range_pairs_per_head": lr,
        "long_range_pairs_visited_per_head": lr_visited,
        "phase_ms": phase,
        "schedule_probe_ms": probe,
        "graph_schedule_probe_ms": graph_probe if args.graph else None,
        "eager_ms_per_step": eager_ms,
        "step_ms_stats": {"median": float(np.median(per_step)), "min": per_step[0],
                          "max": per_step[-1]},
        "device": device_info(torch),
        "attn_ms": attn_ms,
        "plan_ms": plan_ms,
        "attn_tflops": flops / (attn_ms * 1e-3) / 1e12,
        "attn_frac_of_bf16_peak": flops / (attn_ms * 1e-3) / 1e12 / metrics.MI355X_BF16_DENSE_TFLOPS,
        "assign_GBps": (B * n * wl.d_model * 4) / (phase["assign"] * 1e-3) / 1e9,
        "computed_pairs_per_head": {"window": cwin, "long_range": clr},
        "tile_utilization": {"window": win / cwin, "long_range": lr_visited / max(clr, 1)},
        "computed_tile_tflops": {
            "window": metrics.attn_flops(cwin, Hq, d) / (phase["window"] * 1e-3) / 1e12,
            "long_range": metrics.attn_flops(clr, Hq, d) / (phase["long_range_apply"] * 1e-3) / 1e12,
            "attention": metrics.attn_flops(cwin + clr, Hq, d) / (attn_ms * 1e-3) / 1e12},
    }

    # The dominant kernel of the step and its roofline (bf16 MFMA bound).
    kern = max(("long_range_apply", "window"), key=lambda nm: phase[nm])
    kflops = metrics.attn_flops(lr if kern == "long_range_apply" else win, Hq, d)
    ach = kflops / (phase[kern] * 1e-3) / 1e12
    lr_phase = 1 if m == 1 else (7 if metrics.uses_set_pass(K, m) else 3)
    kname = (f"attn_kernel<{d},{lr_phase}>" if kern == "long_range_apply"
             else f"attn_kernel<{d},0>")
    # the entry passes (two groups per token, K >= 5) launch their kernel
    # twice per step, once per membership index
    launches = 2 if kern == "long_range_apply" and lr_phase == 3 else 1
    what = {0: " (window pass)", 1: " (long-range pass + merge)", 7: " (set pass + merge)",
            3: " (two entry passes, merged in place)"}
    res["roofline"] = {"kernel": kname + what[lr_phase if kern == "long_range_apply" else 0],
                       "bound": "mfma", "achieved": ach,
                       "peak": metrics.MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                       "frac": ach / metrics.MI355X_BF16_DENSE_TFLOPS,
                       "traffic": measured_traffic(wl.name, kname),
                       "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                       "copy-calibrated)",
                       "launches_per_step": launches,
                       "flops_per_launch": kflops / launches,
                       "avg_launch_ms": phase[kern] / launches}

    if not args.skip_dense:
        log(f"dense causal baseline x{args.dense_iters}")
        focus.dense_causal_attn_fwd(q, k, v, scale, out=out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.dense_iters):
            focus.dense_causal_attn_fwd(q, k, v, scale, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.dense_iters
        dflops = metrics.attn_flops(B * (n * (n + 1) // 2), Hq, d)
        res["dense_ms"] = dense_ms
        res["dense_tflops"] = dflops / (dense_ms * 1e-3) / 1e12
        res["speedup_attn_vs_dense"] = dense_ms / attn_ms
        res["speedup_step_vs_dense"] = dense_ms / ms_step
        log(f"dense {dense_ms:.3f} ms ({res['dense_tflops']:.1f} TFLOP/s)")

    if args.copy_probe:
        copy_probe(torch, res)

    del hidden, q, k, v, out, ws_t
    torch.cuda.empty_cache()
    if not args.skip_cpu_baseline:
        log("CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(x, wl, args.cpu_seconds)
        log(f"cpu baseline {res['cpu_baseline']['value']:.3e} TFLOP/s")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
