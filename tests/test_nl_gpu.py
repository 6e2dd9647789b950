"""Nonlinear residual refinement on the GPU (through the C ABI) against the float64 oracle.

* prism_nl_gain: the per-channel chain factors, element by element against
  oracle.prism_nl.preconditioner (GELU(p r) / r along the nonlinear chain).
* prism_fwd_nl: o and S_final against oracle.prism_nl.forward_nl, the token recurrence
  with the GELU chain written out (it never forms the factors).
* Streaming: factors from a carried ShortConv window, then prism_fwd_state, resumed in
  two pieces, against one oracle pass.
* At the 16K workload (T = 16384, H = 4, d = 64, L = 4, bf16) the factors of sampled
  token windows against the oracle, and the one-call forward against the two-call one.
* Gains predicted from the anchor (prism_nl_gain_pred, prism_fwd_nl_pred): factors and
  forward against the oracle fed oracle.prism_nl.predictor_gains.

Tolerances (max-abs error relative to max |reference|): forward as the linear forward's
parity tests, 1e-4 for float32 I/O and 2e-2 for bfloat16 I/O.  Factors: 1e-5 in float32
(erfc to a few ulp, and the chain's float32 residuals); in bfloat16 each factor is rounded
to 8 bits (relative 2^-9) and the residuals carry earlier levels' roundings, so 1e-2.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import prism_nl as onl
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
GTOL = {"f32": 1e-5, "bf16": 1e-2}

CASES = {
    "f32_d16_L2": workloads.Workload("nl_f32_d16", "f32", B=1, H=2, T=77, dk=16, dv=16, L=2, chunk=16, seed=80),
    "f32_d32_L3": workloads.Workload("nl_f32_d32", "f32", B=2, H=2, T=100, dk=32, dv=32, L=3, chunk=32, seed=81),
    # bf16 d = 64, chunk 64, L <= 4: the two-wave sweep path, with a ragged tail
    "bf16_d64_L4": workloads.Workload("nl_bf16_d64", "bf16", B=1, H=2, T=209, dk=64, dv=64, L=4, chunk=64, seed=82),
    "bf16_d128_L8": workloads.Workload("nl_bf16_d128", "bf16", B=1, H=2, T=130, dk=128, dv=128, L=8, chunk=64,
                                       seed=83),
    "bf16_d64_L1": workloads.Workload("nl_bf16_L1", "bf16", B=1, H=1, T=70, dk=64, dv=64, L=1, chunk=64, seed=84),
    # the nonlinear d = 64 sweep's other instantiations: L = 2 and 8 unrolled, L = 3 through
    # the run-time step loop
    "bf16_d64_L2": workloads.Workload("nl_bf16_d64_L2", "bf16", B=2, H=1, T=130, dk=64, dv=64, L=2, chunk=64,
                                      seed=86),
    "bf16_d64_L3": workloads.Workload("nl_bf16_d64_L3", "bf16", B=1, H=2, T=100, dk=64, dv=64, L=3, chunk=64,
                                      seed=87),
    "bf16_d64_L8": workloads.Workload("nl_bf16_d64_L8", "bf16", B=1, H=2, T=150, dk=64, dv=64, L=8, chunk=64,
                                      seed=88),
}


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


def rel_err(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - b)) / max(1e-30, float(np.max(np.abs(b)))))


def _inputs(w):
    x = workloads.generate(w)
    x["p"] = workloads.generate_gain(w)
    return x


def _dev(x, w):
    return workloads.to_torch({k: v for k, v in x.items() if k != "gamma"}, w.dtype)


@pytest.mark.parametrize("hist", [False, True])
@pytest.mark.parametrize("key", [k for k in CASES if CASES[k].L > 1])
def test_gain_factors(prism, key, hist):
    import torch
    w = CASES[key]
    x = _inputs(w)
    ci = workloads.generate_state(w)["conv_in"] if hist else None
    log(f"[nl gain] {key} hist={hist}")
    d = _dev(x, w)
    cid = workloads.to_torch({"conv_in": ci}, w.dtype)["conv_in"] if hist else None
    gam = prism.nl_gain(d["v"], d["alpha"], d["p"], d["conv_w"], w.L, conv_in=cid)
    torch.cuda.synchronize()
    ref = onl.preconditioner(x["v"], x["alpha"], x["p"], x["conv_w"], w.L, conv_in=ci)
    err = rel_err(gam.float().cpu().numpy(), ref)
    log(f"  factors rel err {err:.3e} (tol {GTOL[w.dtype]:.0e})")
    assert err <= GTOL[w.dtype]


@pytest.mark.parametrize("key", list(CASES))
def test_fwd_nl_parity(prism, key):
    import torch
    w = CASES[key]
    x = _inputs(w)
    log(f"[nl fwd] {key}")
    d = _dev(x, w)
    o, S = prism.fwd_nl(d["q"], d["k"], d["v"], d["g"], d["beta"], d.get("u"), d.get("alpha"), d.get("p"),
                        d["conv_w"], L=w.L, chunk=w.chunk)
    torch.cuda.synchronize()
    ref_o, ref_S = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["p"],
                                  x["conv_w"], w.L)
    o = o.float().cpu().numpy()
    S = S.cpu().numpy()
    eo, es = rel_err(o, ref_o), rel_err(S, ref_S)
    log(f"  rel err o {eo:.3e}  S_final {es:.3e} (tol {TOL[w.dtype]:.0e})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


@pytest.mark.parametrize("key", ["f32_d32_L3", "bf16_d64_L4"])
def test_nl_streaming_resume(prism, key):
    import torch
    w = CASES[key]
    x = _inputs(w)
    T1 = 67
    log(f"[nl stream] {key} split at {T1}")
    d = _dev(x, w)

    def part(a, b):
        return {k: (v if k == "conv_w" else v[:, :, a:b].contiguous()) for k, v in d.items()}

    p1, p2 = part(0, T1), part(T1, w.T)
    g1 = prism.nl_gain(p1["v"], p1["alpha"], p1["p"], p1["conv_w"], w.L)
    o1, S1, c1 = prism.fwd_state(p1["q"], p1["k"], p1["v"], p1["g"], p1["beta"], p1["u"], p1["alpha"], g1,
                                 p1["conv_w"], L=w.L, chunk=w.chunk)
    g2 = prism.nl_gain(p2["v"], p2["alpha"], p2["p"], p2["conv_w"], w.L, conv_in=c1)
    o2, S2, _ = prism.fwd_state(p2["q"], p2["k"], p2["v"], p2["g"], p2["beta"], p2["u"], p2["alpha"], g2,
                                p2["conv_w"], L=w.L, chunk=w.chunk, S0=S1, conv_in=c1)
    torch.cuda.synchronize()
    o = torch.cat([o1, o2], dim=2).float().cpu().numpy()
    ref_o, ref_S = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["p"],
                                  x["conv_w"], w.L)
    eo, es = rel_err(o, ref_o), rel_err(S2.cpu().numpy(), ref_S)
    log(f"  rel err o {eo:.3e}  S_final {es:.3e}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_nl_full_size_16k(prism):
    """The 16K workload: factors of sampled token windows against the oracle (each
    window's three earlier values as its history), and the one-call forward (whose d = 64
    sweep evaluates the factors in its own chain) against factors + prism_fwd: the same
    rounded factors up to float32 contraction order, so within a few bfloat16 steps."""
    import torch
    w = workloads.workload("rec16k_bf16")
    x = _inputs(w)
    log("[nl 16k] gain + forward at T=16384 H=4 d=64 L=4")
    d = _dev(x, w)
    gam = prism.nl_gain(d["v"], d["alpha"], d["p"], d["conv_w"], w.L)
    o, S = prism.fwd_nl(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["p"], d["conv_w"],
                        L=w.L, chunk=w.chunk)
    o2, S2 = prism.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], gam, d["conv_w"],
                       L=w.L, chunk=w.chunk)
    torch.cuda.synchronize()
    eo = rel_err(o.float().cpu().numpy(), o2.float().cpu().numpy().astype(np.float64))
    es = rel_err(S.cpu().numpy(), S2.cpu().numpy().astype(np.float64))
    log(f"  fused vs two-pass forward: rel diff o {eo:.3e}  S_final {es:.3e}")
    assert eo <= 1e-2 and es <= 1e-2
    gam = gam.float().cpu().numpy()
    rng = np.random.default_rng(5)
    for t0 in [0, 1, 2, 3, 4095, 8191] + list(rng.integers(3, w.T - 64, 6)):
        t0 = int(t0)
        t1 = min(w.T, t0 + 64)
        h0 = max(0, t0 - 3)
        ci = np.zeros((w.B, w.H, 3, w.dv), np.float32)
        if t0 > 0:
            ci[:, :, 3 - (t0 - h0):] = x["v"][:, :, h0:t0]
        ref = onl.preconditioner(x["v"][:, :, t0:t1], x["alpha"][:, :, t0:t1], x["p"][:, :, t0:t1],
                                 x["conv_w"], w.L, conv_in=ci)
        err = rel_err(gam[:, :, t0:t1], ref)
        assert err <= GTOL["bf16"], (t0, err)
    log("  sampled factors within tolerance")


# ---- gains predicted from the anchor (prism_nl_gain_pred, prism_fwd_nl_pred) -------------
PRED_CASES = {
    "bf16_d32_L3": workloads.Workload("nlp_bf16_d32", "bf16", B=2, H=2, T=75, dk=32, dv=32, L=3, chunk=32, seed=85),
    "bf16_d64_L4": CASES["bf16_d64_L4"],
    "bf16_d128_L8": CASES["bf16_d128_L8"],
}


def _pred_inputs(w, conv_in=None):
    x = workloads.generate(w)
    x["W_p"] = workloads.generate_predictor(w)
    x["p"] = onl.predictor_gains(x["v"], x["conv_w"], x["W_p"], w.L, conv_in=conv_in)
    return x


@pytest.mark.parametrize("hist", [False, True])
@pytest.mark.parametrize("key", list(PRED_CASES))
def test_pred_gain_factors(prism, key, hist):
    """Factors from predicted gains against the oracle's (gains in float64 from the float64
    anchor; the kernel rounds the anchor to bfloat16 for its MFMA operand)."""
    import torch
    w = PRED_CASES[key]
    ci = workloads.generate_state(w)["conv_in"] if hist else None
    x = _pred_inputs(w, ci)
    log(f"[nl pred gain] {key} hist={hist}")
    d = workloads.to_torch({k: x[k] for k in ("v", "alpha", "W_p", "conv_w")}, w.dtype)
    cid = workloads.to_torch({"conv_in": ci}, w.dtype)["conv_in"] if hist else None
    gam = prism.nl_gain_pred(d["v"], d["alpha"], d["W_p"], d["conv_w"], w.L, conv_in=cid)
    torch.cuda.synchronize()
    ref = onl.preconditioner(x["v"], x["alpha"], x["p"], x["conv_w"], w.L, conv_in=ci)
    err = rel_err(gam.float().cpu().numpy(), ref)
    log(f"  factors rel err {err:.3e} (tol {GTOL[w.dtype]:.0e})")
    assert err <= GTOL[w.dtype]


@pytest.mark.parametrize("key", list(PRED_CASES))
def test_fwd_nl_pred_parity(prism, key):
    import torch
    w = PRED_CASES[key]
    x = _pred_inputs(w)
    log(f"[nl pred fwd] {key}")
    d = workloads.to_torch({k: v for k, v in x.items() if k not in ("gamma", "p")}, w.dtype)
    o, S = prism.fwd_nl_pred(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["W_p"],
                             d["conv_w"], L=w.L, chunk=w.chunk)
    torch.cuda.synchronize()
    ref_o, ref_S = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["p"],
                                  x["conv_w"], w.L)
    o = o.float().cpu().numpy()
    S = S.cpu().numpy()
    eo, es = rel_err(o, ref_o), rel_err(S, ref_S)
    log(f"  rel err o {eo:.3e}  S_final {es:.3e} (tol {TOL[w.dtype]:.0e})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


@pytest.mark.parametrize("key", ["f32_d32_L3", "bf16_d64_L4"])
def test_nl_decode_steps(prism, key):
    """Token-by-token generation of the nonlinear variant: each token's factors from the
    carried ShortConv window (prism_nl_gain with T = 1, conv_in = the decode window), then
    prism_decode_step; against the oracle over the same tokens from the same start."""
    import torch
    w = CASES[key].replace(T=12)
    x = _inputs(w)
    st = workloads.generate_state(w)
    log(f"[nl decode] {key} {w.T} steps")
    d = _dev(x, w)
    s = workloads.to_torch(st, w.dtype)
    S, conv = s["S0"].clone(), s["conv_in"].clone()
    outs = []
    for t in range(w.T):
        one = {k: (None if v is None else v[:, :, t:t + 1].contiguous()) for k, v in d.items() if k != "conv_w"}
        gam = prism.nl_gain(one["v"], one["alpha"], one["p"], d["conv_w"], w.L, conv_in=conv)
        sq = lambda t_: t_[:, :, 0].contiguous()  # noqa: E731
        o = prism.decode_step(S, conv, sq(one["q"]), sq(one["k"]), sq(one["v"]), sq(one["g"]), sq(one["beta"]),
                              sq(one["u"]), sq(one["alpha"]), sq(gam), d["conv_w"], L=w.L)
        outs.append(o.float().cpu().numpy().astype(np.float64))
    torch.cuda.synchronize()
    ref_o, ref_S = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["p"],
                                  x["conv_w"], w.L, S0=st["S0"], conv_in=st["conv_in"])
    o = np.stack(outs, axis=2)
    eo, es = rel_err(o, ref_o), rel_err(S.cpu().numpy(), ref_S)
    log(f"  rel err o {eo:.3e}  S_final {es:.3e}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


@pytest.mark.parametrize("seg", [2, 3])
@pytest.mark.parametrize("L", [2, 3, 4, 8])
def test_nl_sweep_multichunk_segments(prism, L, seg):
    """The nonlinear d = 64 sweep with segments of several chunks (state, segment operator
    and rank-input slots carried from chunk to chunk) against the token-by-token oracle."""
    import torch
    w = workloads.Workload("nl_seg", "bf16", B=1, H=2, T=450, dk=64, dv=64, L=L, chunk=64, seed=150 + L)
    x = _inputs(w)
    log(f"[nl fwd] L={L} seg={seg} T={w.T}")
    d = _dev(x, w)
    o, S = prism.fwd_nl(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["p"], d["conv_w"],
                        L=w.L, chunk=w.chunk, seg_chunks=seg)
    torch.cuda.synchronize()
    ref_o, ref_S = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["p"],
                                  x["conv_w"], w.L)
    eo, es = rel_err(o.float().cpu().numpy(), ref_o), rel_err(S.cpu().numpy(), ref_S)
    log(f"  rel err o {eo:.3e}  S_final {es:.3e} (tol {TOL[w.dtype]:.0e})")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


@pytest.mark.parametrize("L", [2, 5, 8])
def test_nl_half_split_sweep_segments(prism, L):
    """The nonlinear d = 128 half-split sweep (factors formed in its chain) with segments of
    three chunks and a ragged tail, against the token-by-token oracle."""
    import torch
    w = workloads.Workload("nl_seg128", "bf16", B=2, H=1, T=5 * 64 + 29, dk=128, dv=128, L=L, chunk=64,
                           seed=160 + L)
    x = _inputs(w)
    log(f"[nl fwd] d=128 L={L} seg=3 T={w.T}")
    d = _dev(x, w)
    o, S = prism.fwd_nl(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["p"], d["conv_w"],
                        L=w.L, chunk=w.chunk, seg_chunks=3)
    torch.cuda.synchronize()
    ref_o, ref_S = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["p"],
                                  x["conv_w"], w.L)
    eo, es = rel_err(o.float().cpu().numpy(), ref_o), rel_err(S.cpu().numpy(), ref_S)
    log(f"  rel err o {eo:.3e}  S_final {es:.3e} (tol {TOL[w.dtype]:.0e})")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_nl_full_size_16k_against_oracle(prism):
    """The fused nonlinear forward at the 16K workload (B2 H4 T16384 d64 L4, planner's
    segments of 8 chunks) against the token-by-token oracle on head 1 (both batches)."""
    import torch
    w = workloads.workload("rec16k_bf16")
    x = _inputs(w)
    log("[nl 16k] fused forward vs oracle, head 1")
    d = _dev(x, w)
    o, S = prism.fwd_nl(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["p"], d["conv_w"],
                        L=w.L, chunk=w.chunk)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    S = S.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    ref_o, ref_S = onl.forward_nl(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["p"],
                                  x["conv_w"], w.L, heads=[1])
    eo, es = rel_err(o[:, [1]], ref_o), rel_err(S[:, [1]], ref_S)
    log(f"  rel err o {eo:.3e}  S_final {es:.3e} (tol {TOL[w.dtype]:.0e})")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]
