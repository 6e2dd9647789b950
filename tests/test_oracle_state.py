"""Pins of the oracle's starting-state, value-history and one-token paths.

A sequence continued from its previous state and last three values must give
exactly what the uninterrupted sequence gives: the state is all the linear
recurrence carries, and the ShortConv anchor only looks three tokens back
("PRISM" reading notes, section 2.3; Tencent Ads article, section 01-二).  These
tests tie the new inputs to the plain forward (itself pinned in
test_oracle_pins.py) and, for the starting state, to dense transition matrices.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import _dense_AB, _inputs, _rel


def _slice(x, a, b):
    return {k: (v[:, :, a:b] if k != "conv_w" else v) for k, v in x.items()}


def _fwd(x, L, S0=None, conv_in=None):
    return oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"],
                          x["u"] if L > 1 else None, x["alpha"] if L > 1 else None,
                          x["gamma"] if L > 1 else None, x["conv_w"], L, S0=S0, conv_in=conv_in)


@pytest.mark.parametrize("L,T1", [(1, 5), (3, 1), (3, 2), (3, 7), (4, 3)])
def test_split_and_resume_equals_whole(L, T1):
    # run [0, T1) then [T1, T) from (S_final, last three values): same o and S_T as one run.
    # T1 < 3 checks that the carried window keeps the rows of the first part only.
    rng = np.random.default_rng(100 + 10 * L + T1)
    x = _inputs(rng, B=2, H=2, T=11, dk=6, dv=5, L=L)
    o, S = _fwd(x, L)
    a = _slice(x, 0, T1)
    o1, S1 = _fwd(a, L)
    tail = oracle.conv_tail(a["v"])
    o2, S2 = _fwd(_slice(x, T1, 11), L, S0=S1, conv_in=tail)
    assert _rel(np.concatenate([o1, o2], axis=2), o) < 1e-12
    assert _rel(S2, S) < 1e-12


def test_three_way_split_carries_history_across_a_short_middle():
    # the middle part (1 token) is shorter than the window: its tail mixes the
    # first part's values with its own
    L = 3
    rng = np.random.default_rng(7)
    x = _inputs(rng, B=1, H=2, T=9, dk=5, dv=4, L=L)
    o, S = _fwd(x, L)
    parts, S_, tail, outs = [(0, 4), (4, 5), (5, 9)], None, None, []
    for a, b in parts:
        xa = _slice(x, a, b)
        oa, S_ = _fwd(xa, L, S0=S_, conv_in=tail)
        tail = oracle.conv_tail(xa["v"], tail)
        outs.append(oa)
    assert _rel(np.concatenate(outs, axis=2), o) < 1e-12
    assert _rel(S_, S) < 1e-12


def test_conv_tail_rows():
    # the window after T tokens is rows T-3 .. T-1 of [history; v]
    rng = np.random.default_rng(3)
    hist = rng.standard_normal((1, 2, 3, 4))
    v = rng.standard_normal((1, 2, 5, 4))
    assert np.array_equal(oracle.conv_tail(v, hist), v[:, :, 2:5])
    v2 = rng.standard_normal((1, 2, 2, 4))
    assert np.array_equal(oracle.conv_tail(v2, hist), np.concatenate([hist[:, :, 2:], v2], axis=2))
    assert np.array_equal(oracle.conv_tail(v2), np.concatenate([np.zeros((1, 2, 1, 4)), v2], axis=2))


@pytest.mark.parametrize("L", [1, 3])
def test_start_state_adds_the_free_response(L):
    # S_t = S_0 A_1 ... A_t + sum_{s<=t} B_s A_{s+1} ... A_t: the starting state enters
    # only through the product of the dense transitions (catches a transposed S_0,
    # which is passed in the S_final layout, i.e. as S_0^T)
    rng = np.random.default_rng(40 + L)
    T, dk, dv = 7, 5, 4
    x = _inputs(rng, B=1, H=2, T=T, dk=dk, dv=dv, L=L)
    S0t = rng.standard_normal((1, 2, dk, dv))          # the S_final layout: S_0^T
    o0, S_0 = _fwd(x, L)
    o1, S_1 = _fwd(x, L, S0=S0t)
    for h in range(2):
        A, _ = _dense_AB(x, 0, h, L)
        M = S0t[0, h].T                                   # S_0, dv x dk
        for t in range(T):
            M = M @ A[t]
            assert _rel(o1[0, h, t] - o0[0, h, t], M @ x["q"][0, h, t]) < 1e-11
        assert _rel(S_1[0, h] - S_0[0, h], M.T) < 1e-11


@pytest.mark.parametrize("L", [1, 2, 4])
def test_decode_steps_equal_forward(L):
    # token-at-a-time from a starting state and value history = one forward call
    rng = np.random.default_rng(60 + L)
    B, H, T, dk, dv = 2, 3, 6, 5, 4
    x = _inputs(rng, B=B, H=H, T=T, dk=dk, dv=dv, L=L)
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.3
    hist = rng.standard_normal((B, H, 3, dv))
    o, S = _fwd(x, L, S0=S0, conv_in=hist)
    St, conv = S0, hist
    for t in range(T):
        ot, St, conv = oracle.decode_step(
            St, conv, x["q"][:, :, t], x["k"][:, :, t], x["v"][:, :, t], x["g"][:, :, t],
            x["beta"][:, :, t], x["u"][:, :, t] if L > 1 else None, x["alpha"][:, :, t] if L > 1 else None,
            x["gamma"][:, :, t] if L > 1 else None, x["conv_w"], L)
        assert _rel(ot, o[:, :, t]) < 1e-12
    assert _rel(St, S) < 1e-12
    assert np.array_equal(conv, x["v"][:, :, T - 3:])
