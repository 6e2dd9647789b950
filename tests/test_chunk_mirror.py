"""The chunked / segmented algebra (numpy mirror) against the oracle, in float64."""
import numpy as np
import pytest

import oracle
from tests import chunk_mirror as cm
from tests.test_oracle_pins import _inputs


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("L", [1, 3, 4])
@pytest.mark.parametrize("T,seg", [(150, None), (150, 1), (200, 2), (64, 1), (5, None)])
def test_mirror_matches_oracle(chunk, L, T, seg):
    rng = np.random.default_rng(1000 + chunk + 10 * L + T)
    x = _inputs(rng, B=1, H=1, T=T, dk=16, dv=16, L=L, g_range=(0.9, 1.0))
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                  x["u"] if L > 1 else None, x["alpha"] if L > 1 else None,
                                  x["gamma"] if L > 1 else None, x["conv_w"], L)
    o, H = cm.forward_chunked(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], x["g"][0, 0], x["beta"][0, 0],
                              x["u"][0, 0] if L > 1 else None, x["alpha"][0, 0] if L > 1 else None,
                              x["gamma"][0, 0] if L > 1 else None, x["conv_w"][0], L, chunk, seg)
    assert _rel(o, o_ref[0, 0]) < 1e-11
    assert _rel(H, S_ref[0, 0]) < 1e-11


def test_blocked_inverse():
    rng = np.random.default_rng(5)
    for C in [16, 32, 48, 64]:
        M = np.eye(C) + np.tril(rng.standard_normal((C, C)) * 0.1, -1)
        T = cm.unit_lower_inverse_blocked(M)
        assert np.max(np.abs(T @ M - np.eye(C))) < 1e-12


@pytest.mark.parametrize("T,chunk,L,d,with_dS", [(150, 32, 3, 16, True), (64, 16, 1, 8, False),
                                                 (100, 64, 4, 16, True), (37, 16, 2, 8, True),
                                                 (70, 16, 8, 8, False)])
def test_backward_mirror_matches_gradient_oracle(T, chunk, L, d, with_dS):
    """The chunked adjoint (per chunk: the readout, end-state, UT-transform and decay
    terms; across chunks: dH = Qt^T dO + Acc^T dH') against autograd through the token
    recurrence, every gradient at 1e-11."""
    from oracle import prism_grad
    rng = np.random.default_rng(7 + T + L)
    x = _inputs(rng, B=1, H=1, T=T, dk=d, dv=d, L=L, g_range=(0.9, 1.0))
    d_o = rng.standard_normal((1, 1, T, d))
    dS = rng.standard_normal((1, 1, d, d)) if with_dS else None
    ref = prism_grad.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["gamma"],
                              x["conv_w"], L, d_o, dS)
    got = cm.backward_chunked(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], x["g"][0, 0], x["beta"][0, 0],
                              x["u"][0, 0] if L > 1 else None, x["alpha"][0, 0] if L > 1 else None,
                              x["gamma"][0, 0] if L > 1 else None, x["conv_w"][0], L, chunk, d_o[0, 0],
                              None if dS is None else dS[0, 0])
    names = ["dq", "dk", "dv", "dg", "dbeta"] + (["du", "dalpha", "dgamma", "dconv_w"] if L > 1 else [])
    for n in names:
        r = ref[n][0] if n == "dconv_w" else ref[n][0, 0]
        assert _rel(got[n], r) < 1e-11, n
