"""focus_group_sort_noalloc, the sort that runs on the library's static
device scratch instead of a caller's workspace, called through the C ABI and
checked bit for bit against focus_group_sort with a workspace: two calls in a
row on one GPU (the second smaller, so it runs on what the first left in the
scratch), the largest request the scratch holds, and the host-side rejection
of one that needs more."""
import ctypes

import numpy as np
import pytest
import torch

from group_gated_sparse_amd import focus
from gpu_common import dev, host, say

pytestmark = pytest.mark.gpu

UNSUPPORTED = 2
SCRATCH_BYTES = 1 << 20


def _ids(rng, B, n, K):
    # skewed group sizes, so segments and per-block counts differ widely
    p = rng.dirichlet(np.full(K, 0.5))
    return rng.choice(K, size=(B, n), p=p).astype(np.int32)


def _both(ids_np, K):
    B, n = ids_np.shape
    ids = dev(ids_np)
    perm_ws, offs_ws = focus.focus_group_sort(ids, K)
    perm = torch.full((B, n), -1, dtype=torch.int32, device=ids.device)
    offs = torch.full((B, K + 1), -1, dtype=torch.int32, device=ids.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = focus.lib().focus_group_sort_noalloc(ctypes.c_void_p(ids.data_ptr()), B, n, K,
                                              ctypes.c_void_p(perm.data_ptr()),
                                              ctypes.c_void_p(offs.data_ptr()), stream)
    assert rc == 0, focus.lib().focus_last_error().decode()
    torch.cuda.synchronize()
    return host(perm), host(offs), host(perm_ws), host(offs_ws)


def test_noalloc_sort_equals_workspace_sort_two_calls():
    rng = np.random.default_rng(7301)
    for B, n, K in [(3, 50001, 64), (1, 777, 5)]:
        say(f"[sort noalloc] B={B} n={n} K={K}")
        ids = _ids(rng, B, n, K)
        perm, offs, perm_ws, offs_ws = _both(ids, K)
        assert np.array_equal(perm, perm_ws) and np.array_equal(offs, offs_ws)
        # and it is the stable sort
        for b in range(B):
            assert np.array_equal(perm[b], np.argsort(ids[b], kind="stable"))


def test_noalloc_sort_largest_request_and_rejection():
    # B * ceil(n / 2048) * K * 4 bytes of per-block counts: exactly the scratch
    B, K = 2, 64
    n = 2048 * (SCRATCH_BYTES // (4 * B * K))
    assert focus.focus_group_sort_workspace_bytes(B, n, K) == SCRATCH_BYTES
    say(f"[sort noalloc] largest: B={B} n={n} K={K}")
    rng = np.random.default_rng(7302)
    ids = _ids(rng, B, n, K)
    perm, offs, perm_ws, offs_ws = _both(ids, K)
    assert np.array_equal(perm, perm_ws) and np.array_equal(offs, offs_ws)
    # one more block needs more than the scratch: rejected on the host,
    # nothing enqueued (the outputs keep their fill)
    n2 = n + 1
    ids2 = dev(np.zeros((B, n2), dtype=np.int32))
    perm2 = torch.full((B, n2), -1, dtype=torch.int32, device=ids2.device)
    offs2 = torch.full((B, K + 1), -1, dtype=torch.int32, device=ids2.device)
    rc = focus.lib().focus_group_sort_noalloc(ctypes.c_void_p(ids2.data_ptr()), B, n2, K,
                                              ctypes.c_void_p(perm2.data_ptr()),
                                              ctypes.c_void_p(offs2.data_ptr()), None)
    assert rc == UNSUPPORTED
    assert "static scratch" in focus.lib().focus_last_error().decode()
    torch.cuda.synchronize()
    assert (host(perm2) == -1).all() and (host(offs2) == -1).all()
