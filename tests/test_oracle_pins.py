"""Pins of the float64 oracle to facts that do not come from the oracle itself.

Each test checks the oracle against a library routine, a closed form, an
invariant of the method, or a brute-force evaluation written differently
(dense transition matrices, a tree-ordered scan).  Together they are meant to
catch a dropped term, a wrong sign, a wrong index and a transposed operand
anywhere in the oracle; the comment on each test says which.
"""
import numpy as np
import pytest

import oracle

RTOL = 1e-12


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(rng, B=1, H=1, T=12, dk=6, dv=5, L=3, g_range=(0.85, 1.0), beta=None):
    q = _unit(rng.standard_normal((B, H, T, dk)))
    k = _unit(rng.standard_normal((B, H, T, dk)))
    v = rng.standard_normal((B, H, T, dv))
    g = rng.uniform(*g_range, size=(B, H, T))
    b = rng.uniform(0.05, 0.95, size=(B, H, T)) if beta is None else np.full((B, H, T), float(beta))
    w = rng.normal(0, 0.5, size=(H, 4, dv))
    u = _unit(rng.standard_normal((B, H, T, max(L - 1, 1), dk)))[:, :, :, :L - 1]
    alpha = rng.uniform(0.05, 0.5, size=(B, H, T, L))
    gamma = rng.uniform(-0.12, 1.12, size=(B, H, T, max(L - 1, 1), dv))[:, :, :, :L - 1]
    return dict(q=q, k=k, v=v, g=g, beta=b, u=u, alpha=alpha, gamma=gamma, conv_w=w)


def _run(x, L):
    return oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"],
                          x["u"] if L > 1 else None, x["alpha"] if L > 1 else None,
                          x["gamma"] if L > 1 else None, x["conv_w"], L)


def _anchor_np(v, w):
    """ShortConv via numpy.convolve, per channel: tap j multiplies v_{t-3+j}."""
    T, dv = v.shape
    return np.stack([np.convolve(v[:, c], w[::-1, c])[:T] for c in range(dv)], axis=1)


def _written_closed_form(v, w, alpha, gamma, L):
    """R_{t,l} = alpha_{t,l} * prod_{m<l}(1 - alpha_{t,m} gamma_{t,m}) * (v_t - anchor_t)."""
    r0 = v - _anchor_np(v, w)
    out = []
    for l in range(1, L):
        fac = np.prod(1.0 - alpha[:, :l, None] * gamma[:, :l, :], axis=1)
        out.append(alpha[:, l, None] * fac * r0)
    return out  # list of [T, dv]


# --- the pieces --------------------------------------------------------------

def test_anchor_is_numpy_convolve():
    # catches a reversed tap order, a window that skips token t, or padding errors
    rng = np.random.default_rng(11)
    T, dv = 19, 7
    v = rng.standard_normal((T, dv))
    w = rng.standard_normal((4, dv))
    ref = _anchor_np(v, w)
    got = np.stack([oracle.shortconv_anchor(v, w, t) for t in range(T)])
    assert _rel(got, ref) < RTOL


@pytest.mark.parametrize("L", [2, 3, 5, 8])
def test_chain_iterated_equals_closed_form(L):
    # the pages: the linearised chain collapses to one closed-form step.
    # catches an off-by-one in the alpha / gamma slot used at step l
    rng = np.random.default_rng(L)
    dv = 9
    r0 = rng.standard_normal((4, dv))
    alpha = rng.uniform(0, 0.5, (4, L))
    gamma = rng.uniform(-0.13, 1.13, (4, L - 1, dv))
    res, wr = oracle.residual_chain(r0, alpha, gamma, L)
    for l in range(1, L):
        closed = np.prod(1.0 - alpha[:, :l, None] * gamma[:, :l, :], axis=1) * r0
        assert _rel(res[l - 1], closed) < 1e-14
        assert _rel(wr[l - 1], alpha[:, l, None] * closed) < 1e-14


# --- the whole map -------------------------------------------------------------

def test_L1_reduces_to_gdn_delta_form():
    # at L = 1 the method is exactly Gated DeltaNet:  S = g S + beta (v - g S k) k^T.
    # catches a missing beta on the write and a decay applied to the write
    rng = np.random.default_rng(3)
    x = _inputs(rng, B=2, H=2, T=40, dk=8, dv=6, L=1)
    o, S = _run(x, 1)
    for b in range(2):
        for h in range(2):
            St = np.zeros((6, 8))
            ref = np.empty((40, 6))
            for t in range(40):
                k, v, g, be = x["k"][b, h, t], x["v"][b, h, t], x["g"][b, h, t], x["beta"][b, h, t]
                St = g * St + be * np.outer(v - g * St @ k, k)
                ref[t] = St @ x["q"][b, h, t]
            assert _rel(o[b, h], ref) < RTOL
            assert _rel(S[b, h], St.T) < RTOL


def test_L1_ignores_rank_inputs():
    # at L = 1 the anchor, directions, step sizes and preconditioners do not matter
    rng = np.random.default_rng(4)
    x = _inputs(rng, T=30, L=3)
    base = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, None, x["conv_w"], 1)
    other = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"] * 3, x["alpha"] + 1,
                           x["gamma"] - 2, x["conv_w"] * 7, 1)
    assert np.array_equal(base[0], other[0]) and np.array_equal(base[1], other[1])


def test_delta_rule_writes_value_at_key_L1():
    # delta rule with beta = 1 and unit keys: the state maps k_t exactly to v_t.
    # Read out with q = k:  o_t = S_t k_t = v_t.  Catches a wrong erase sign,
    # a transposed state and a readout taken before the write.
    rng = np.random.default_rng(5)
    x = _inputs(rng, B=1, H=3, T=50, dk=8, dv=8, L=1, beta=1.0, g_range=(0.5, 1.0))
    x["q"] = x["k"]
    o, _ = _run(x, 1)
    assert _rel(o, x["v"]) < 1e-12


def test_delta_rule_with_rank_terms():
    # beta = 1, L > 1:  S_t k_t = v_t + sum_l R_{t,l} (u_{t,l} . k_t)
    rng = np.random.default_rng(6)
    L = 4
    x = _inputs(rng, B=1, H=2, T=33, dk=7, dv=5, L=L, beta=1.0)
    x["q"] = x["k"]
    o, _ = _run(x, L)
    for h in range(2):
        R = _written_closed_form(x["v"][0, h], x["conv_w"][h], x["alpha"][0, h], x["gamma"][0, h], L)
        ref = x["v"][0, h].copy()
        for l in range(1, L):
            dots = np.sum(x["u"][0, h, :, l - 1] * x["k"][0, h], axis=-1)
            ref += R[l - 1] * dots[:, None]
        assert _rel(o[0, h], ref) < 1e-12


@pytest.mark.parametrize("gated", [False, True])
def test_beta0_is_causal_linear_attention(gated):
    # beta = 0 leaves only the rank-(L-1) injection.  With g = 1 the map is
    # plain causal linear attention over (u, R) pairs:  O = sum_l tril(Q U_l^T) R_l.
    # With g < 1 each term is decayed by prod_{s<j<=t} g_j (gated linear
    # attention).  Catches wrong u / R orientation, a decayed write, a missing
    # diagonal (readout before the write) and anchor / chain errors.
    rng = np.random.default_rng(7 + gated)
    L, T = 4, 37
    x = _inputs(rng, B=2, H=2, T=T, dk=6, dv=5, L=L, beta=0.0,
                g_range=(0.7, 1.0) if gated else (1.0, 1.0))
    o, _ = _run(x, L)
    for b in range(2):
        for h in range(2):
            lg = np.cumsum(np.log(x["g"][b, h]))
            decay = np.tril(np.exp(lg[:, None] - lg[None, :]))
            R = _written_closed_form(x["v"][b, h], x["conv_w"][h], x["alpha"][b, h], x["gamma"][b, h], L)
            ref = sum((decay * (x["q"][b, h] @ x["u"][b, h, :, l - 1].T)) @ R[l - 1] for l in range(1, L))
            assert _rel(o[b, h], ref) < 1e-12


def _dense_AB(x, b, h, L):
    """Dense A_t (dk x dk) and B_t (dv x dk) written out from the definitions."""
    T, dk = x["k"].shape[2:]
    dv = x["v"].shape[-1]
    R = _written_closed_form(x["v"][b, h], x["conv_w"][h], x["alpha"][b, h], x["gamma"][b, h], L) if L > 1 else []
    A, Bm = [], []
    for t in range(T):
        k = x["k"][b, h, t]
        A.append(x["g"][b, h, t] * (np.eye(dk) - x["beta"][b, h, t] * np.outer(k, k)))
        Bt = x["beta"][b, h, t] * np.outer(x["v"][b, h, t], k)
        for l in range(1, L):
            Bt = Bt + np.outer(R[l - 1][t], x["u"][b, h, t, l - 1])
        Bm.append(Bt)
    return A, Bm


@pytest.mark.parametrize("L", [1, 3])
def test_brute_force_dense_sum(L):
    # S_t = sum_{s<=t} B_s A_{s+1} ... A_t, evaluated with dense matrices (T <= 8)
    rng = np.random.default_rng(20 + L)
    T = 8
    x = _inputs(rng, B=1, H=2, T=T, dk=5, dv=4, L=L)
    o, S = _run(x, L)
    for h in range(2):
        A, Bm = _dense_AB(x, 0, h, L)
        for t in range(T):
            St = np.zeros_like(Bm[0])
            for s in range(t + 1):
                M = Bm[s]
                for j in range(s + 1, t + 1):
                    M = M @ A[j]
                St = St + M
            assert _rel(o[0, h, t], St @ x["q"][0, h, t]) < 1e-12
        assert _rel(S[0, h], St.T) < 1e-12


def test_tree_order_scan_matches():
    # associativity: a Hillis-Steele inclusive scan of (A_t, B_t) pairs under
    # (A1, B1) then (A2, B2)  ->  (A1 A2, B1 A2 + B2) reproduces every S_t.
    rng = np.random.default_rng(31)
    T, L = 8, 3
    x = _inputs(rng, B=1, H=1, T=T, dk=5, dv=5, L=L)
    o, _ = _run(x, L)
    A, Bm = _dense_AB(x, 0, 0, L)
    pairs = list(zip(A, Bm))
    step = 1
    while step < T:
        new = list(pairs)
        for t in range(step, T):
            A1, B1 = pairs[t - step]
            A2, B2 = pairs[t]
            new[t] = (A1 @ A2, B1 @ A2 + B2)
        pairs = new
        step *= 2
    for t in range(T):
        assert _rel(o[0, 0, t], pairs[t][1] @ x["q"][0, 0, t]) < 1e-12


@pytest.mark.parametrize("L", [1, 2, 4, 6])
def test_write_has_rank_L(L):
    # rank accumulation: each token's injection B_t has rank min(L, dk, dv)
    rng = np.random.default_rng(40 + L)
    x = _inputs(rng, T=10, dk=8, dv=7, L=L)
    _, Bm = _dense_AB(x, 0, 0, L)
    # the oracle's own B_t: one step from a zero state
    P = 1
    S0 = np.zeros((P, 7, 8))
    for t in range(3, 10):
        anchor = oracle.shortconv_anchor(x["v"][0], x["conv_w"], t)
        Bt, _ = oracle.token_step(S0, x["q"][0, :, t], x["k"][0, :, t], x["v"][0, :, t],
                                  x["g"][0, :, t], x["beta"][0, :, t], anchor,
                                  x["u"][0, :, t] if L > 1 else None, x["alpha"][0, :, t] if L > 1 else None,
                                  x["gamma"][0, :, t] if L > 1 else None, L)
        assert np.linalg.matrix_rank(Bt[0], tol=1e-10) == min(L, 7, 8)
        assert _rel(Bt[0], Bm[t]) < 1e-12


def test_linear_in_v():
    # A_t does not depend on v and B_t is linear in v, with S_0 = 0
    rng = np.random.default_rng(50)
    L = 4
    x1 = _inputs(rng, B=1, H=2, T=25, dk=6, dv=6, L=L)
    v2 = rng.standard_normal(x1["v"].shape)
    a, b = 0.7, -1.9
    o1, S1 = _run(x1, L)
    x2 = dict(x1, v=v2)
    o2, S2 = _run(x2, L)
    x3 = dict(x1, v=a * x1["v"] + b * v2)
    o3, S3 = _run(x3, L)
    assert _rel(o3, a * o1 + b * o2) < 1e-12
    assert _rel(S3, a * S1 + b * S2) < 1e-12


def test_state_bounded_for_contractive_transitions():
    # with beta in [0, 1], unit keys and g <= 1, ||A_t|| <= 1, so
    # ||S_T|| <= sum_t ||B_t||
    rng = np.random.default_rng(60)
    L, T = 3, 60
    x = _inputs(rng, T=T, dk=6, dv=6, L=L)
    _, S = _run(x, L)
    _, Bm = _dense_AB(x, 0, 0, L)
    assert np.linalg.norm(S[0, 0], 2) <= sum(np.linalg.norm(Bt, 2) for Bt in Bm) + 1e-12


def test_heads_subset_matches_full():
    rng = np.random.default_rng(70)
    x = _inputs(rng, B=2, H=3, T=20, L=3)
    o, S = _run(x, 3)
    o1, S1 = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["gamma"],
                            x["conv_w"], 3, heads=[2, 0])
    assert np.array_equal(o1[:, 0], o[:, 2]) and np.array_equal(o1[:, 1], o[:, 0])
    assert np.array_equal(S1[:, 0], S[:, 2])
