"""Pins of the written-correction oracle and its predictor front end (oracle/prism_delta.py).

What fixes them besides themselves:
* L = 1 never reads the gains, keys or gates: the plain (GDN) forward of oracle/prism.py.
* p = 0 and p r << 0 (GELU(z) -> 0) write nothing beyond the GDN write.
* Small gains: GELU(z) = z / 2 + O(z^2), so with p = eps c (c the same on every channel)
  each written correction is alpha_l eps c_{l-1} r_0 / 2 + O(eps^2): the linear oracle with
  zero factors and step sizes alpha_l eps c_{l-1} / 2 matches to O(eps^2) (error ratio 4
  when eps halves).  A wrong gain or gate index, a sign, or writing r instead of the
  correction leaves an O(eps) gap.
* Saturated gains (p r >= 50 everywhere: GELU(z) = z to double precision): the chain is
  r_l = (1 - c_{l-1}) r_{l-1} with written c_{l-1} r_{l-1}, which the linear oracle
  reproduces exactly with step sizes and factors mapped per level.  This fixes the
  subtraction without a step size and the written correction at full size.
* The factor form (r <- r - f r, written alpha f r) with channel-constant factors maps
  onto the linear oracle exactly; with the oracle's own factors it reproduces the GELU
  forward, and a zero residual takes the limit p / 2.
* Greedy subtraction with 0 < p <= 1 never grows the residual and never flips its sign.
* Front end: the anchor from numpy.convolve and the three projections by explicit loops;
  identity key weights give the normalised anchor; zero gate weights give gates 1/2.
"""
import numpy as np
import pytest

import workloads
from oracle import prism as orc
from oracle import prism_delta as odl
from oracle import prism_nl as onl


def _inputs(L=3, T=20, d=8, B=1, H=2, seed=17):
    w = workloads.Workload("dl_pin", "f32", B=B, H=H, T=T, dk=d, dv=d, L=L, chunk=16, seed=seed)
    x = workloads.generate(w)
    x["p"] = workloads.generate_gain(w)
    return w, x


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _fwd(x, L, p=None, **kw):
    return odl.forward_delta(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"],
                             x["p"] if p is None else p, x["conv_w"], L, **kw)


def test_l1_is_the_gdn_forward_and_ignores_rank_inputs():
    w, x = _inputs(L=1)
    o, S = odl.forward_delta(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, None, x["conv_w"], 1)
    o_ref, S_ref = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, None, x["conv_w"], 1)
    assert _rel(o, o_ref) < 1e-13 and _rel(S, S_ref) < 1e-13


def test_zero_gain_writes_only_the_gdn_term():
    w, x = _inputs(L=4)
    o, S = _fwd(x, 4, p=np.zeros_like(x["p"]))
    o_ref, S_ref = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, None, x["conv_w"], 1)
    assert _rel(o, o_ref) < 1e-13 and _rel(S, S_ref) < 1e-13


def _channel_constant(w, rng, lo, hi):
    c = rng.uniform(lo, hi, size=(w.B, w.H, w.T, w.L - 1, 1))
    return np.broadcast_to(c, (w.B, w.H, w.T, w.L - 1, w.dv)).copy(), c[..., 0]


def test_small_gain_limit_against_the_linear_oracle():
    w, x = _inputs(L=4, T=16)
    rng = np.random.default_rng(5)
    cfull, c = _channel_constant(w, rng, 0.5, 1.5)
    alpha = np.asarray(x["alpha"], np.float64)
    errs = []
    for eps in (2e-3, 1e-3):
        o, _ = _fwd(x, 4, p=eps * cfull)
        a_lin = np.zeros_like(alpha)
        a_lin[..., 1:] = alpha[..., 1:] * eps * c / 2.0
        o_lin, _ = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], a_lin,
                               np.zeros_like(x["p"]), x["conv_w"], 4)
        errs.append(float(np.max(np.abs(o - o_lin))))
    assert errs[1] < 1e-5
    assert 3.5 < errs[0] / errs[1] < 4.5, errs


def _linear_map(alpha, c):
    """Step sizes and factors of the linear chain that reproduce r_l = (1 - c_{l-1}) r_{l-1}
    with written values alpha_l c_{l-1} r_{l-1} (c constant over channels)."""
    a_lin = np.ones_like(alpha)
    a_lin[..., 1:] = alpha[..., 1:] * c / (1.0 - c)
    gam = c / a_lin[..., :-1]
    return a_lin, gam


def test_saturated_gains_map_exactly_onto_the_linear_oracle():
    w, x = _inputs(L=4, T=12)
    rng = np.random.default_rng(6)
    x = dict(x)
    x["v"] = (1000.0 + 100.0 * np.abs(rng.standard_normal(x["v"].shape))).astype(np.float64)
    x["conv_w"] = np.zeros_like(x["conv_w"])                   # anchor 0: r_0 = v >= 1000
    cfull, c = _channel_constant(w, rng, 0.1, 0.2)              # p r >= 0.1 * 1000 * 0.8^3 = 51
    o, S = _fwd(x, 4, p=cfull)
    a_lin, gam = _linear_map(np.asarray(x["alpha"], np.float64), c)
    gam_full = np.broadcast_to(gam[..., None], cfull.shape)
    o_ref, S_ref = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], a_lin, gam_full,
                               x["conv_w"], 4)
    assert _rel(o, o_ref) < 1e-12 and _rel(S, S_ref) < 1e-12


def test_negative_saturation_writes_nothing():
    w, x = _inputs(L=3, T=12)
    rng = np.random.default_rng(8)
    x = dict(x)
    x["v"] = (1000.0 + np.abs(rng.standard_normal(x["v"].shape))).astype(np.float64)
    x["conv_w"] = np.zeros_like(x["conv_w"])
    o, S = _fwd(x, 3, p=-np.ones_like(x["p"]))                   # p r <= -1000: GELU = 0
    o_ref, S_ref = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, None, x["conv_w"], 1)
    assert _rel(o, o_ref) < 1e-13 and _rel(S, S_ref) < 1e-13


def test_factor_form_with_constant_factors_maps_onto_the_linear_oracle():
    w, x = _inputs(L=5, T=14)
    rng = np.random.default_rng(9)
    ffull, f = _channel_constant(w, rng, 0.05, 0.9)
    o, S = odl.forward_delta_factors(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], ffull,
                                     x["conv_w"], 5)
    a_lin, gam = _linear_map(np.asarray(x["alpha"], np.float64), f)
    o_ref, S_ref = orc.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], a_lin,
                               np.broadcast_to(gam[..., None], ffull.shape), x["conv_w"], 5)
    assert _rel(o, o_ref) < 1e-12 and _rel(S, S_ref) < 1e-12


@pytest.mark.parametrize("L", [2, 3, 5])
def test_factors_reproduce_the_gelu_forward(L):
    w, x = _inputs(L=L, T=18)
    fac = odl.delta_factors(x["v"], x["p"], x["conv_w"], L)
    o, S = odl.forward_delta_factors(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], fac,
                                     x["conv_w"], L)
    o_ref, S_ref = _fwd(x, L)
    assert _rel(o, o_ref) < 1e-12 and _rel(S, S_ref) < 1e-12


def test_factor_limit_at_zero_residual():
    w, x = _inputs(L=3, T=6)
    v = np.zeros_like(x["v"])                                   # r = 0 everywhere
    fac = odl.delta_factors(v, x["p"], x["conv_w"], 3)
    np.testing.assert_allclose(fac, 0.5 * np.asarray(x["p"], np.float64), atol=0, rtol=0)


def test_factor_rounding_is_the_chain_the_forward_sees():
    """With each factor rounded before the chain continues, the factor form run with those
    factors is still exact: the rounding only moves the residuals the next levels see."""
    w, x = _inputs(L=5, T=10)
    rnd = lambda f: np.round(f * 64.0) / 64.0  # noqa: E731  (a coarse grid: visible effect)
    fr = odl.delta_factors(x["v"], x["p"], x["conv_w"], 5, rounding=rnd)
    assert np.all(fr * 64.0 == np.round(fr * 64.0))
    assert np.max(np.abs(fr - odl.delta_factors(x["v"], x["p"], x["conv_w"], 5))) > 1e-3
    # level 0 sees the exact residual r_0 either way
    f0 = odl.delta_factors(x["v"], x["p"], x["conv_w"], 5)[..., 0, :]
    np.testing.assert_array_equal(fr[..., 0, :], rnd(f0))


def test_greedy_subtraction_shrinks_residual():
    rng = np.random.default_rng(3)
    r0 = rng.standard_normal((50, 16))
    p = rng.uniform(0.01, 1.0, size=(50, 6, 16))
    alpha = rng.uniform(0.0, 1.0, size=(50, 7))
    deltas, written = odl.delta_chain(r0, alpha, p, 7)
    r = r0
    for l, d in enumerate(deltas):
        r_new = r - d
        assert np.all(np.abs(r_new) <= np.abs(r) + 1e-15)
        assert np.all(r_new * r >= 0.0)
        np.testing.assert_allclose(written[l], alpha[:, l + 1, None] * d)
        r = r_new


def _anchor_loops(v, conv_w, conv_in=None):
    B, H, T, dv = v.shape
    hist = np.zeros((B, H, 3, dv)) if conv_in is None else np.asarray(conv_in, np.float64)
    ext = np.concatenate([hist, np.asarray(v, np.float64)], axis=2)
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            for c in range(dv):
                full = np.convolve(ext[b, h, :, c], np.asarray(conv_w, np.float64)[h, ::-1, c])
                out[b, h, :, c] = full[3:3 + T]
    return out


@pytest.mark.parametrize("hist", [False, True])
def test_front_end_by_loops(hist):
    rng = np.random.default_rng(11)
    B, H, T, dk, dv, L = 1, 2, 7, 4, 6, 3
    v = rng.standard_normal((B, H, T, dv))
    cw = rng.standard_normal((H, 4, dv))
    Wp = rng.standard_normal((H, L - 1, dv, dv))
    Wk = rng.standard_normal((H, L - 1, dk, dv))
    Wb = rng.standard_normal((H, L, dv))
    ci = rng.standard_normal((B, H, 3, dv)) if hist else None
    p, u, alpha = odl.anchor_predict(v, cw, Wp, Wk, Wb, L, conv_in=ci)
    anc = _anchor_loops(v, cw, ci)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                a = anc[b, h, t]
                for l in range(L - 1):
                    for o in range(dv):
                        assert p[b, h, t, l, o] == pytest.approx(sum(Wp[h, l, o, i] * a[i] for i in range(dv)),
                                                                 abs=1e-12)
                    key = [sum(Wk[h, l, o, i] * a[i] for i in range(dv)) for o in range(dk)]
                    nrm = sum(z * z for z in key) ** 0.5
                    for o in range(dk):
                        assert u[b, h, t, l, o] == pytest.approx(key[o] / nrm, abs=1e-12)
                for l in range(L):
                    z = sum(Wb[h, l, i] * a[i] for i in range(dv))
                    assert alpha[b, h, t, l] == pytest.approx(1.0 / (1.0 + np.exp(-z)), abs=1e-14)


def test_front_end_identity_and_zero_weights():
    rng = np.random.default_rng(12)
    B, H, T, d, L = 2, 1, 9, 5, 4
    v = rng.standard_normal((B, H, T, d))
    cw = rng.standard_normal((H, 4, d))
    Wk = np.broadcast_to(np.eye(d), (H, L - 1, d, d))
    p, u, alpha = odl.anchor_predict(v, cw, np.zeros((H, L - 1, d, d)), Wk, np.zeros((H, L, d)), L)
    anc = _anchor_loops(v, cw)
    ref = anc / np.linalg.norm(anc, axis=-1, keepdims=True)
    for l in range(L - 1):
        np.testing.assert_allclose(u[:, :, :, l], ref, atol=1e-14)
    assert np.all(p == 0.0)
    assert np.all(alpha == 0.5)


def test_gelu_shared_with_the_nonlinear_oracle():
    # the correction is the same exact-erf GELU whose constants tests/test_oracle_nl.py pins
    assert odl.gelu is onl.gelu


# ---- planted mistakes in the written-correction chain must fail a pin -----------------------
def _writes_residual(r0, alpha_t, p_t, L):           # writes r_l instead of the correction
    r, ds, wr = r0, [], []
    for l in range(1, L):
        d = onl.gelu(p_t[..., l - 1, :] * r)
        r = r - d
        ds.append(d)
        wr.append(alpha_t[..., l, None] * r)
    return ds, wr


def _step_size_on_subtraction(r0, alpha_t, p_t, L):  # r <- r - alpha_{l-1} delta
    r, ds, wr = r0, [], []
    for l in range(1, L):
        d = onl.gelu(p_t[..., l - 1, :] * r)
        r = r - alpha_t[..., l - 1, None] * d
        ds.append(d)
        wr.append(alpha_t[..., l, None] * d)
    return ds, wr


def _gain_index_shift(r0, alpha_t, p_t, L):          # layer l reads gain slot l (wraps)
    r, ds, wr = r0, [], []
    for l in range(1, L):
        d = onl.gelu(p_t[..., l % (L - 1), :] * r)
        r = r - d
        ds.append(d)
        wr.append(alpha_t[..., l, None] * d)
    return ds, wr


def _gate_index_shift(r0, alpha_t, p_t, L):          # written with the previous layer's gate
    r, ds, wr = r0, [], []
    for l in range(1, L):
        d = onl.gelu(p_t[..., l - 1, :] * r)
        r = r - d
        ds.append(d)
        wr.append(alpha_t[..., l - 1, None] * d)
    return ds, wr


def _no_subtraction(r0, alpha_t, p_t, L):            # every layer sees r_0
    ds, wr = [], []
    for l in range(1, L):
        d = onl.gelu(p_t[..., l - 1, :] * r0)
        ds.append(d)
        wr.append(alpha_t[..., l, None] * d)
    return ds, wr


DELTA_PINS = [
    test_small_gain_limit_against_the_linear_oracle,
    test_saturated_gains_map_exactly_onto_the_linear_oracle,
    test_negative_saturation_writes_nothing,
    test_zero_gain_writes_only_the_gdn_term,
]


@pytest.mark.parametrize("mutant", [_writes_residual, _step_size_on_subtraction, _gain_index_shift,
                                    _gate_index_shift, _no_subtraction])
def test_planted_chain_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(odl, "delta_chain", mutant)
    caught = 0
    for pin in DELTA_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, mutant.__name__
