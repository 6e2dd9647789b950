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
