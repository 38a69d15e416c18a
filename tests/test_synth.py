"""The seeded input generator: determinism, rounding and the group-size targets."""
import numpy as np
import torch

from group_gated_sparse_amd import synth, workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_bits(x), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(synth.bf16_to_f32(ref), back)


def test_inputs_are_deterministic_and_shaped():
    wl = workloads.TINY
    a = synth.make_inputs(wl)
    b = synth.make_inputs(wl)
    assert synth.digest(a) == synth.digest(b)
    assert a["hidden"].shape == (wl.B, wl.n, wl.d_model) and a["hidden"].dtype == np.float32
    assert a["q"].shape == (wl.B, wl.Hq, wl.n, wl.d) and a["q"].dtype == np.uint16
    assert a["k"].shape == (wl.B, wl.Hkv, wl.n, wl.d)
    assert np.allclose(np.linalg.norm(a["C"], axis=1), 1.0, atol=1e-6)
    c = synth.make_inputs(wl.with_(seed=wl.seed + 1))
    assert synth.digest(a) != synth.digest(c)
    # attention-only draws reproduce the same q, k, v
    d = synth.make_inputs(wl, with_hidden=False)
    assert np.array_equal(d["q"], a["q"]) and np.array_equal(d["v"], a["v"])


def test_orthonormal_centroid_space():
    wl = workloads.ZIPF7B.with_(d_model=256, n=16)
    x = synth.make_inputs(wl, with_qkv=False)
    P, C = x["P"].astype(np.float64), x["C"].astype(np.float64)
    assert np.allclose(P.T @ P, np.eye(wl.d_proj), atol=1e-5)
    assert np.allclose(C @ C.T, np.eye(wl.K), atol=1e-5)


def test_gauss_max_win_probability_against_sampling():
    rng = np.random.default_rng(3)
    b = np.array([0.8, 0.1, -0.2, -0.7, 0.0])
    p = synth.gauss_max_win_prob(b)
    assert abs(p.sum() - 1.0) < 1e-6
    x = rng.standard_normal((400000, 5)) + b
    emp = np.bincount(np.argmax(x, axis=1), minlength=5) / 400000
    assert np.max(np.abs(emp - p)) < 4 * np.sqrt(p * (1 - p) / 400000).max()


def test_zipf_bias_sets_expected_group_sizes():
    K = 32
    target = synth.zipf_target(K, 1.1)
    b = synth.gauss_max_bias(target)
    assert np.max(np.abs(synth.gauss_max_win_prob(b) / target - 1)) < 1e-6
    assert abs(target[0] / target[-1] - 32 ** 1.1) < 1e-9
