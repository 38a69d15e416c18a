"""GPU parity on seeded random layer shapes: focus_attn_fwd through the C ABI
against the fp64 oracle, over the combinations the kernels specialise on —
head packing (query heads per kv head 1 .. 16, so 1, 2, 4 or 8 heads per
workgroup and 128 .. 16 tokens per tile), d = 32 / 64 / 128, ragged n,
windows from 0 to beyond n, K from 1 to 64, uniform and skewed group sizes,
batches, fp32 and bf16 output. Bars as in the other parity tests: max-abs
1e-2 and mean-abs 1e-3 on fp32 output (bf16 output adds its rounding), lse
within 1e-3, perm and offsets bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle
from group_gated_sparse_amd import focus, synth
from gpu_common import check_attn, dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu

N_CASES = 32


def _case(seed):
    rng = np.random.default_rng(90000 + seed)
    d = int(rng.choice([32, 64, 128]))
    Hkv = int(rng.integers(1, 5))
    hpk = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    while Hkv * hpk > 32:
        hpk //= 2
    Hq = Hkv * max(hpk, 1)
    B = int(rng.integers(1, 4))
    n = int(rng.integers(1, 901))
    K = int(rng.integers(1, 65))
    wkind = rng.integers(0, 4)
    w = 0 if wkind == 0 else (n + int(rng.integers(0, 5)) if wkind == 1 else int(rng.integers(0, n + 1)))
    skew = bool(rng.integers(0, 2))
    bf16_out = bool(rng.integers(0, 4) == 0)
    return rng, B, Hq, Hkv, n, d, K, w, skew, bf16_out


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape_matches_oracle(seed):
    rng, B, Hq, Hkv, n, d, K, w, skew, bf16_out = _case(seed)
    say(f"[random {seed}] B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} K={K} w={w} "
        f"skew={skew} out={'bf16' if bf16_out else 'fp32'}")
    q = synth.bf16_bits(rng.standard_normal((B, Hq, n, d), dtype=np.float32))
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    if skew:
        p = 1.0 / np.arange(1, K + 1) ** 1.1
        ids = synth.random_group_ids(rng, B, n, K, probs=p / p.sum())
    else:
        ids = synth.random_group_ids(rng, B, n, K)
    scale = 1.0 / math.sqrt(d)

    tid = dev(ids)
    perm, offs = focus.focus_group_sort(tid, K)
    out, lse = focus.focus_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), tid, perm, offs, K, w,
                                    scale, out_dtype=torch.bfloat16 if bf16_out else torch.float32,
                                    want_lse=True)
    torch.cuda.synchronize()

    rperm, roffs = oracle.group_sort(ids, K)
    assert np.array_equal(host(perm), rperm) and np.array_equal(host(offs), roffs)
    ref, rlse, _ = oracle.attn(q, k, v, ids, w, scale)
    check_attn(host(out.float()).reshape(-1, d), ref.reshape(-1, d), f"random {seed}",
               bf16_out=bf16_out)
    assert np.max(np.abs(host(lse) - rlse)) < 1e-3
