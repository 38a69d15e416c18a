"""Hand-derived fixture of the attention pattern (tests/golden/focus_pattern_n8_w1.txt)."""
import math
import os
from fractions import Fraction

import numpy as np

import oracle
from group_gated_sparse_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "focus_pattern_n8_w1.txt")


def _parse():
    ids, w, A, means, pairs = None, None, {}, {}, None
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, _, val = line.partition(":")
        if key == "ids":
            ids = [int(x) for x in val.split()]
        elif key == "w":
            w = int(val)
        elif key == "pairs":
            pairs = int(val)
        elif key.startswith("A "):
            A[int(key[2:])] = [int(x) for x in val.split()]
        elif key.startswith("mean "):
            means[int(key[5:])] = Fraction(val.strip())
    return ids, w, A, means, pairs


def test_hand_worked_pattern_and_uniform_score_outputs():
    ids, w, A, means, pairs = _parse()
    n = len(ids)
    q = np.zeros((1, 1, n, 2), np.uint16)                      # bf16 +0.0
    k = synth.bf16_bits(np.random.default_rng(0).standard_normal((1, 1, n, 2)).astype(np.float32))
    v = synth.bf16_bits(np.array([[j, 1.0] for j in range(n)], np.float32)).reshape(1, 1, n, 2)
    g = np.array([ids], np.int32)
    out, lse, vis = oracle.attn(q, k, v, g, w, 1.0)
    assert int(vis.sum()) == pairs
    for i in range(n):
        wt = oracle.attn_weights(q, k, g, w, 1.0, 0, 0, i)
        assert list(np.nonzero(wt)[0]) == A[i]
        assert vis[0, 0, i] == len(A[i])
        assert abs(out[0, 0, i, 0] - float(means[i])) < 1e-15
        assert out[0, 0, i, 1] == 1.0
        assert abs(lse[0, 0, i] - math.log(len(A[i]))) < 1e-15
