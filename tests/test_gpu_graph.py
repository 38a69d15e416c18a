"""The hot path under HIP graph capture: every entry point only enqueues
kernels on the caller's stream (no allocation, no memset, no host
synchronisation), so a captured step replays to the eager result. The
graph is replayed several times with other eager work and synchronisation
in between, and every replay is compared with the eager run bit for bit."""
import numpy as np
import pytest
import torch

from group_gated_sparse_amd import focus, synth, workloads
from gpu_common import dev, dev_bf16, say

pytestmark = pytest.mark.gpu


def test_captured_step_replays_bitwise():
    wl = workloads.GPT2.with_(name="gpt2_graph", B=2)
    say(f"[graph] {wl.name}: B={wl.B} n={wl.n} K={wl.K} w={wl.w}")
    x = synth.make_inputs(wl)
    hidden, P, C = dev(x["hidden"]), dev(x["P"]), dev(x["C"])
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    B, n, K, d, Hq, Hkv = wl.B, wl.n, wl.K, wl.d, wl.Hq, wl.Hkv
    ids = torch.empty((B, n), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
    offs = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, n, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
    ws_a = torch.empty(focus.focus_assign_workspace_bytes(wl.d_model, K), dtype=torch.uint8,
                       device="cuda")
    ws_s = torch.empty(focus.focus_group_sort_workspace_bytes(B, n, K), dtype=torch.uint8,
                       device="cuda")
    ws_t = torch.empty(focus.focus_attn_workspace_bytes(B, Hq, Hkv, n, d, K, wl.w),
                       dtype=torch.uint8, device="cuda")

    def step():
        focus.focus_assign(hidden, P, C, None, group_ids=ids, want_margin=False, workspace=ws_a)
        focus.focus_group_sort(ids, K, perm=perm, group_offsets=offs, workspace=ws_s)
        focus.focus_attn_fwd(q, k, v, ids, perm, offs, K, wl.w, wl.softmax_scale, out=out,
                             lse=lse, workspace=ws_t)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (ids, perm, offs, out, lse)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (ids, perm, offs, lse):
            t.fill_(-7)
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        # some eager work between the replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        for a_, b_ in zip((ids, perm, offs, out, lse), ref):
            assert torch.equal(a_, b_), f"replay {rep} differs from the eager step"
        del junk
