"""The fused prologue on its own: the rank-L factors R_{t,l} = alpha_{t,l} r_{t,l} that each
sweep forms from the ShortConv anchor and the residual chain, against the oracle's own
intermediates (oracle.shortconv_anchor, oracle.residual_chain).

The sweeps never write R out, so the test reads it through the forward with inputs that
switch the rest of the recurrence off.  With beta = 0 and g = 1 every token's operator is
the identity and the state is S_t = sum_{s <= t} sum_l R_{s,l} u_{s,l}^T (PRISM reading
notes, section 2.2: the rank writes add up; with the GDN write gated off nothing else
enters).  Each direction u_{s,l} is a one-hot key e_{c(s,l)} with c(s,l) = ((L-1) s + l - 1)
mod dk, so:

* for T (L-1) <= dk every factor owns one key column, and row c(s,l) of S_final (the
  S^T layout) is exactly R_{s,l};
* with a one-hot query q_t = e_{c(t,l_t)}, o_t is the sum of the R_{s,l} with s <= t that
  share that key column: R_{t,l_t} plus those of tokens a multiple of dk / gcd apart, over
  several chunks (so the anchor window crosses chunk and segment boundaries).

One-hot keys and queries make the state products exact, so what is left is the factors'
own arithmetic and their rounding to the MFMA operand type: a factor taken from the
wrong tap, residual or step shows up at its own token, at O(1).  Tolerance (max-abs error
relative to max |reference|): 1e-2 in bfloat16 (each factor rounded once to bfloat16,
2^-9, then summed and rounded to the output type), 1e-5 in float32.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def prism():
    if not gpu_available():
        pytest.skip("no GPU")
    import delta_rule_sequence_amd as m
    m.load_library()
    return m


def key_col(s, l, L, dk):
    return ((L - 1) * s + l - 1) % dk


def isolating_inputs(w, x):
    """beta = 0, g = 1, one-hot directions u_{s,l} = e_{c(s,l)} and queries q_t = e_{c(t,l_t)}."""
    B, H, T, dk, L = w.B, w.H, w.T, w.dk, w.L
    y = dict(x)
    y["beta"] = np.zeros_like(x["beta"])
    y["g"] = np.ones_like(x["g"])
    u = np.zeros((B, H, T, L - 1, dk), np.float32)
    q = np.zeros((B, H, T, dk), np.float32)
    for t in range(T):
        for l in range(1, L):
            u[:, :, t, l - 1, key_col(t, l, L, dk)] = 1.0
        q[:, :, t, key_col(t, 1 + t % (L - 1), L, dk)] = 1.0
    y["u"], y["q"] = u, q
    return y


def oracle_factors(w, x):
    """R[t, l - 1] = alpha_{t,l} r_{t,l}, [B, H, T, L-1, dv] in float64, from the oracle's anchor
    and chain functions (not its forward)."""
    v = x["v"].astype(np.float64)
    cw = x["conv_w"].astype(np.float64)[None]  # per head, shared by the batch
    R = np.zeros(v.shape[:3] + (w.L - 1, v.shape[-1]))
    for t in range(w.T):
        r0 = v[:, :, t] - oracle.shortconv_anchor(v, cw, t)
        _, written = oracle.residual_chain(r0, x["alpha"][:, :, t].astype(np.float64),
                                           x["gamma"][:, :, t].astype(np.float64), w.L)
        for l in range(1, w.L):
            R[:, :, t, l - 1] = written[l - 1]
    return R


def run(prism, w, y):
    import torch
    d = workloads.to_torch(y, w.dtype)
    o, S = prism.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["gamma"], d["conv_w"],
                     L=w.L, chunk=w.chunk)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-30, float(np.max(np.abs(b)))))


CASES = [
    # (dtype, d, chunk, L, T): the bf16 d = 64 sweep, the d = 128 half-split sweep, the
    # generic sweep in float32 and in bfloat16
    ("bf16", 64, 64, 4, 200),
    ("bf16", 64, 64, 8, 150),
    ("bf16", 128, 64, 5, 170),
    ("f32", 32, 32, 3, 110),
    ("bf16", 32, 16, 4, 90),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_d{c[1]}_c{c[2]}_L{c[3]}")
def test_rank_factors_through_the_output(prism, case):
    dt, d, chunk, L, T = case
    w = workloads.Workload("prologue", dt, B=1, H=2, T=T, dk=d, dv=d, L=L, chunk=chunk, seed=300 + d + L)
    x = workloads.generate(w)
    y = isolating_inputs(w, x)
    R = oracle_factors(w, y)
    o, _ = run(prism, w, y)
    ref = np.zeros_like(o)
    cols = np.array([[key_col(s, l, L, d) for l in range(1, L)] for s in range(T)])  # [T, L-1]
    for t in range(T):
        hit = cols[: t + 1] == key_col(t, 1 + t % (L - 1), L, d)  # [t+1, L-1]
        ref[:, :, t] = np.einsum("sl,bhslv->bhv", hit.astype(np.float64), R[:, :, : t + 1])
    err = rel(o, ref)
    log(f"[prologue] {case}: o rel err {err:.3e} (tol {TOL[dt]:.0e})")
    assert err <= TOL[dt]


@pytest.mark.parametrize("case", [("bf16", 64, 64, 4, 21), ("bf16", 128, 64, 8, 18), ("f32", 32, 32, 3, 16)],
                         ids=lambda c: f"{c[0]}_d{c[1]}_L{c[3]}")
def test_rank_factors_one_per_key_column(prism, case):
    dt, d, chunk, L, T = case
    assert T * (L - 1) <= d
    w = workloads.Workload("prologue1", dt, B=1, H=2, T=T, dk=d, dv=d, L=L, chunk=chunk, seed=320 + d + L)
    x = workloads.generate(w)
    y = isolating_inputs(w, x)
    R = oracle_factors(w, y)
    _, S = run(prism, w, y)  # [B, H, dk, dv]
    got = np.stack([S[:, :, [key_col(t, l, L, d) for l in range(1, L)]] for t in range(T)], axis=2)
    err = rel(got, R)
    log(f"[prologue] {case}: S_final rows vs factors rel err {err:.3e} (tol {TOL[dt]:.0e})")
    assert err <= TOL[dt]
    used = {key_col(t, l, L, d) for t in range(T) for l in range(1, L)}
    free = [c for c in range(d) if c not in used]
    if free:  # key columns no factor was written along stay exactly zero
        assert np.all(S[:, :, free] == 0.0)
