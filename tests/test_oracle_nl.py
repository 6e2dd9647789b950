"""Pins of the nonlinear-refinement oracle (oracle/prism_nl.py).

What fixes it besides itself:
* GELU: the standard normal CDF at +-1 (textbook constants), GELU(x) - GELU(-x) = x,
  and its limits.
* L = 1 never reads p: the output is the plain forward's.
* p = 0 switches the correction off: the linear forward with gamma = 0.
* Small gains: GELU(z) = z / 2 + O(z^2), so with p = eps p0 the nonlinear forward
  meets the linear forward with gamma = eps p0 / 2 up to O(eps^2).  A wrong sign,
  slope or step-size index leaves an O(eps) gap and fails the ratio check.
* Greedy subtraction with 0 < alpha p <= 1 never grows the residual and never
  flips its sign (the next layer sees what is left).
* The preconditioner (GELU absorbed into per-channel factors) run through the
  linear forward reproduces the nonlinear forward; where the residual is exactly
  zero its factor is the limit p / 2.
"""
import numpy as np
import pytest

import workloads
from oracle import prism as orc
from oracle import prism_nl as onl

PHI_1 = 0.8413447460685429   # standard normal CDF at 1
PHI_M1 = 0.15865525393145707  # at -1


def _inputs(L=3, T=24, d=8, B=1, H=2, seed=7):
    w = workloads.Workload("nl_pin", "f32", B=B, H=H, T=T, dk=d, dv=d, L=L, chunk=16, seed=seed)
    x = workloads.generate(w)
    x["p"] = workloads.generate_gain(w)
    return w, x


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def test_gelu_constants_and_symmetry():
    assert onl.gelu(np.array(1.0)) == pytest.approx(PHI_1, abs=1e-15)
    assert onl.gelu(np.array(-1.0)) == pytest.approx(-PHI_M1, abs=1e-15)
    assert onl.gelu(np.array(0.0)) == 0.0
    x = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(onl.gelu(x) - onl.gelu(-x), x, atol=1e-14)
    assert abs(onl.gelu(np.array(-12.0))) < 1e-30
    assert onl.gelu(np.array(12.0)) == pytest.approx(12.0, abs=1e-14)


def test_l1_ignores_gain():
    w, x = _inputs(L=1)
    o, S = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, None, x["conv_w"], 1)
    o_ref, S_ref = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, None, x["conv_w"], 1)
    assert _rel(o, o_ref) < 1e-13 and _rel(S, S_ref) < 1e-13


def test_zero_gain_is_linear_chain_with_zero_factor():
    w, x = _inputs(L=4)
    p0 = np.zeros_like(x["p"])
    o, S = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], p0, x["conv_w"], 4)
    o_ref, S_ref = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], p0,
                               x["conv_w"], 4)
    assert _rel(o, o_ref) < 1e-13 and _rel(S, S_ref) < 1e-13


def test_small_gain_linearisation_is_second_order():
    w, x = _inputs(L=4, T=16)
    errs = []
    for eps in (2e-3, 1e-3):
        p = eps * np.asarray(x["p"], np.float64)
        o, _ = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], p,
                              x["conv_w"], 4)
        o_lin, _ = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], 0.5 * p,
                               x["conv_w"], 4)
        errs.append(float(np.max(np.abs(o - o_lin))))
    assert errs[1] < 1e-5
    assert 3.5 < errs[0] / errs[1] < 4.5, errs


def test_greedy_subtraction_shrinks_residual():
    rng = np.random.default_rng(3)
    L, n = 6, 4000
    r0 = rng.standard_normal((n, 16)) * 3
    alpha = rng.uniform(0.05, 1.0, (n, L))
    p = rng.uniform(0.0, 1.0, (n, L - 1, 16)) / alpha[:, :L - 1, None]
    p = np.minimum(p, 1.0 / alpha[:, :L - 1, None])
    res, written = onl.nonlinear_chain(r0, alpha, p, L)
    prev = r0
    for l, r in enumerate(res, start=1):
        assert np.all(np.abs(r) <= np.abs(prev) + 1e-15)
        assert np.all(r * prev >= 0)
        np.testing.assert_allclose(written[l - 1], alpha[:, l, None] * r, rtol=0, atol=0)
        prev = r
    # strictly smaller somewhere: the correction is not a no-op
    assert np.mean(np.abs(res[-1])) < 0.9 * np.mean(np.abs(r0))


@pytest.mark.parametrize("hist", [False, True])
def test_preconditioner_reproduces_nonlinear_forward(hist):
    w, x = _inputs(L=4, T=20, B=2)
    ci = workloads.generate_state(w)["conv_in"] if hist else None
    gam = onl.preconditioner(x["v"], x["alpha"], x["p"], x["conv_w"], 4, conv_in=ci)
    o, S = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["p"],
                          x["conv_w"], 4, conv_in=ci)
    o_lin, S_lin = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], gam,
                               x["conv_w"], 4, conv_in=ci)
    assert _rel(o_lin, o) < 1e-12 and _rel(S_lin, S) < 1e-12
    # the factors are those of a GELU of the gain-modulated residual: between
    # p * Phi_min and p (GELU(z) / z lies in (0, 1) up to the dip below zero)
    assert np.all(np.abs(gam) <= np.abs(np.asarray(x["p"], np.float64)) + 1e-15)


def test_preconditioner_zero_residual_limit():
    w, x = _inputs(L=3, T=8)
    cw = np.zeros_like(x["conv_w"])
    cw[:, 3, :] = 1.0      # the anchor is the value itself: r_0 = 0
    gam = onl.preconditioner(x["v"], x["alpha"], x["p"], cw, 3)
    np.testing.assert_array_equal(gam, 0.5 * np.asarray(x["p"], np.float64))


def test_predictor_gains_brute_force():
    """p_{t,l}[o] = sum_i W[h, l, o, i] sum_j w[h, j, i] v[t - 3 + j, i], by plain loops."""
    rng = np.random.default_rng(11)
    B, H, T, dv, L = 1, 2, 6, 3, 3
    v = rng.standard_normal((B, H, T, dv))
    cw = rng.standard_normal((H, 4, dv))
    W = rng.standard_normal((H, L - 1, dv, dv))
    ci = rng.standard_normal((B, H, 3, dv))
    p = onl.predictor_gains(v, cw, W, L, conv_in=ci)
    for h in range(H):
        for t in range(T):
            for l in range(L - 1):
                for o in range(dv):
                    acc = 0.0
                    for i in range(dv):
                        a = 0.0
                        for j in range(4):
                            s = t - 3 + j
                            x = v[0, h, s, i] if s >= 0 else ci[0, h, s + 3, i]
                            a += cw[h, j, i] * x
                        acc += W[h, l, o, i] * a
                    assert abs(p[0, h, t, l, o] - acc) < 1e-12
    # identity weights give the anchor itself; zero weights give zero gains
    eye = np.broadcast_to(np.eye(dv), (H, L - 1, dv, dv))
    pa = onl.predictor_gains(v, cw, eye, L)
    pz = onl.predictor_gains(v, cw, np.zeros_like(W), L)
    assert np.all(pz == 0)
    np.testing.assert_allclose(pa[:, :, :, 0], pa[:, :, :, 1], rtol=0, atol=0)
    for t in range(T):
        np.testing.assert_allclose(pa[0, :, t, 0], orc.shortconv_anchor(
            np.concatenate([np.zeros((H, 3, dv)), v[0]], axis=1), cw, t + 3), atol=1e-14)
