"""The seeded input generator: determinism, shapes, ranges and the bf16 cast."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name", ["tiny_gdn_f32", "small_rankL_f32", "rec16k_bf16"])
def test_manifest_matches_stored(name):
    with open(os.path.join(GOLDEN, "manifest.json")) as f:
        man = json.load(f)
    assert workloads.manifest(workloads.generate(workloads.workload(name))) == man[name]


def test_oracle_regression_fixture():
    with open(os.path.join(GOLDEN, "tiny_gdn_f32.json")) as f:
        ref = json.load(f)
    w = workloads.workload("tiny_gdn_f32")
    x = workloads.generate(w)
    o, S = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, None, x["conv_w"], w.L)
    assert np.array_equal(np.asarray(ref["o"]), o.ravel())
    assert np.array_equal(np.asarray(ref["S_final"]), S.ravel())


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_shapes_and_ranges(idx):
    w = workloads.workload(idx)
    w = w.replace(T=min(w.T, 256))
    x = workloads.generate(w)
    B, H, T, dk, dv, L = w.B, w.H, w.T, w.dk, w.dv, w.L
    assert x["q"].shape == (B, H, T, dk) and x["k"].shape == (B, H, T, dk)
    assert x["v"].shape == (B, H, T, dv)
    assert x["g"].shape == (B, H, T) and x["beta"].shape == (B, H, T)
    assert x["conv_w"].shape == (H, 4, dv)
    assert np.all(x["g"] <= 1.0) and np.all(x["g"] >= np.exp(-w.x_hi) - 1e-6)
    assert np.all((x["beta"] > 0) & (x["beta"] < 1))
    nq = np.linalg.norm(x["q"].astype(np.float64), axis=-1)
    tol = 1e-6 if w.dtype == "f32" else 1e-2
    assert np.all(np.abs(nq - 1) < tol)
    if L > 1:
        assert x["u"].shape == (B, H, T, L - 1, dk)
        assert x["alpha"].shape == (B, H, T, L) and np.all((x["alpha"] > 0) & (x["alpha"] < 0.5))
        assert x["gamma"].shape == (B, H, T, L - 1, dv)
        assert np.all((x["gamma"] > -0.1701) & (x["gamma"] < 1.1701))
    else:
        assert x["u"] is None and x["alpha"] is None and x["gamma"] is None
    if w.dtype == "bf16":
        for key in ["q", "k", "v"] + (["u", "gamma"] if L > 1 else []):
            bits = x[key].view(np.uint32)
            assert np.all((bits & 0xFFFF) == 0), key


def test_bf16_rounding_is_rne():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: round to even (1.0)
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 1.0 + 2.0 ** -8 + 2.0 ** -20],
                    dtype=np.float32)
    got = workloads.to_bf16_values(vals)
    assert got.tolist() == [1.0, 1.0 + 2.0 ** -6, -1.0, 1.0 + 2.0 ** -7]


def test_correlated_keys_only_change_k():
    w = workloads.workload(1).replace(T=64)
    a = workloads.generate(w)
    b = workloads.generate(w, keys="correlated")
    for key in ["q", "v", "g", "beta", "u", "alpha", "gamma", "conv_w"]:
        assert np.array_equal(a[key], b[key]), key
    assert not np.array_equal(a["k"], b["k"])
