"""Pins of the float64 gradient oracle (oracle/prism_grad.py).

The gradients come from autograd through a torch re-statement of the
recurrence; they are checked against central finite differences of the numpy
oracle's forward (an independent implementation), one random direction per
input tensor, so a wrong derivative of any input (a dropped term of the
chain, a wrong sign in the erase, a transposed state) fails its own case.
"""
import numpy as np
import pytest

from oracle import prism_grad
from tests.test_oracle_pins import _inputs

NAMES = ["q", "k", "v", "g", "beta", "u", "alpha", "gamma", "conv_w"]


def _setup(seed, L, T=7, dk=4, dv=3, B=1, H=2, with_dS=True):
    rng = np.random.default_rng(seed)
    x = _inputs(rng, B=B, H=H, T=T, dk=dk, dv=dv, L=L)
    d_o = rng.standard_normal((B, H, T, dv))
    dS = rng.standard_normal((B, H, dk, dv)) if with_dS else None
    return rng, x, d_o, dS


def _loss(x, L, d_o, dS):
    return prism_grad.loss(x["q"], x["k"], x["v"], x["g"], x["beta"],
                           x["u"] if L > 1 else None, x["alpha"] if L > 1 else None,
                           x["gamma"] if L > 1 else None, x["conv_w"], L, d_o, dS)


def _grads(x, L, d_o, dS):
    return prism_grad.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"],
                               x["gamma"], x["conv_w"], L, d_o, dS)


@pytest.mark.parametrize("L", [1, 2, 4])
@pytest.mark.parametrize("name", NAMES)
def test_directional_derivative_matches_finite_differences(L, name):
    """<grad, e> equals (f(x + h e) - f(x - h e)) / 2h for a random direction e (the
    numpy forward; O(h^2) error)."""
    if L == 1 and name in ("u", "alpha", "gamma", "conv_w"):
        pytest.skip("the rank-L inputs do not enter at L = 1")
    rng, x, d_o, dS = _setup(11 + L, L)
    gr = _grads(x, L, d_o, dS)["d" + name]
    e = rng.standard_normal(np.shape(x[name]))
    h = 1e-5
    xp = dict(x); xp[name] = x[name] + h * e
    xm = dict(x); xm[name] = x[name] - h * e
    fd = (_loss(xp, L, d_o, dS) - _loss(xm, L, d_o, dS)) / (2 * h)
    an = float(np.sum(gr * e))
    assert abs(an - fd) <= 1e-7 * max(1.0, abs(fd)), (name, an, fd)


def test_gdn_gradients_ignore_rank_inputs():
    """At L = 1 the rank-L inputs do not enter, so the gradients of q, k, v, g, beta
    are those of the plain gated delta rule whatever u, alpha, gamma, conv_w hold."""
    rng, x, d_o, dS = _setup(5, 1)
    a = _grads(x, 1, d_o, dS)
    y = dict(x)
    for n in ("u", "alpha", "gamma", "conv_w"):
        y[n] = rng.standard_normal(np.shape(x[n]))
    b = _grads(y, 1, d_o, dS)
    for n in ("q", "k", "v", "g", "beta"):
        np.testing.assert_array_equal(a["d" + n], b["d" + n])
    assert a["du"] is None and a["dconv_w"] is None


def test_value_gradient_independent_of_values():
    """o and S_final are linear in v (A_t does not depend on v, B_t is linear in v),
    so the gradient with respect to v does not depend on v."""
    rng, x, d_o, dS = _setup(9, 3)
    a = _grads(x, 3, d_o, dS)["dv"]
    y = dict(x); y["v"] = rng.standard_normal(np.shape(x["v"]))
    b = _grads(y, 3, d_o, dS)["dv"]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_query_gradient_is_state_readout():
    """do_t only reaches q_t through o_t = S_t q_t, so dq_t = S_t^T do_t; with d_o
    zero except at the last token, dq at that token is S_final do_T (S_final = S_T^T)."""
    rng, x, d_o, _ = _setup(21, 3, with_dS=False)
    d_o[:] = 0
    d_o[:, :, -1] = rng.standard_normal(d_o[:, :, -1].shape)
    import oracle
    _, S_final = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"],
                                x["gamma"], x["conv_w"], 3)
    dq = _grads(x, 3, d_o, None)["dq"]
    want = np.einsum("bhkv,bhv->bhk", S_final, d_o[:, :, -1])
    np.testing.assert_allclose(dq[:, :, -1], want, rtol=1e-12, atol=1e-12)
    assert np.all(dq[:, :, :-1] == 0)
