"""The written-correction form on the GPU (through the C ABI) against the float64 oracle.

* prism_delta_gain: the correction factors element by element against
  oracle.prism_delta.delta_factors (GELU(p r) / r along the chain r <- r - GELU(p r)).
* prism_fwd_delta (and _seg): o and S_final against oracle.prism_delta.forward_delta, the
  token recurrence with the GELU corrections written out (it never forms the factors), on
  the generic kernels and the bf16 d = 64 sweep (every instantiation: L = 2, 4, 8 unrolled,
  L = 3 through the run-time step loop), with one- and multi-chunk segments.
* prism_anchor_predict: factors, unit keys and gates against oracle.prism_delta.anchor_predict
  (gains, keys and gates from the float64 anchor) and delta_factors on those gains.
* prism_fwd_delta_pred: the whole front end + forward against the oracle fed its own
  predictions, at small sizes and at the 16K workload (one head).

Tolerances (max-abs error relative to max |reference|): forward 1e-4 (float32 I/O) and
2e-2 (bfloat16 I/O), as the linear forward's parity tests.  Factors: the ABI defines each
factor on the residual left by the previous levels' factors as stored (rounded to the I/O
type), so the reference is the oracle's factor chain with that rounding
(delta_factors(..., rounding=)); 1e-5 in float32 and 1e-2 in bfloat16, where a factor that
rounds to the other neighbour moves the later levels' residuals.  The gap between those
rounded factors and the exact ones is the storage type's own (measured 1e-2 at L = 8 in
bfloat16) and is reported, not bounded.  Front end, bfloat16 MFMA operands (the anchor
rounded to 8 bits, float32 sums): keys 1e-2 relative, gates 1e-2 absolute, factors 1e-2
against the oracle with the same anchor and factor roundings.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import prism_delta as odl
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
GTOL = {"f32": 1e-5, "bf16": 1e-2}


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


W = workloads.Workload
CASES = {
    "f32_d16_L2": W("dl_f32_d16", "f32", B=1, H=2, T=77, dk=16, dv=16, L=2, chunk=16, seed=170),
    "f32_d32_L3": W("dl_f32_d32", "f32", B=2, H=2, T=100, dk=32, dv=32, L=3, chunk=32, seed=171),
    "f32_d64_L5": W("dl_f32_d64", "f32", B=1, H=1, T=140, dk=64, dv=64, L=5, chunk=32, seed=172),
    "bf16_d32_L4": W("dl_bf16_d32", "bf16", B=1, H=2, T=90, dk=32, dv=32, L=4, chunk=32, seed=173),
    "bf16_d64_L2": W("dl_bf16_d64_L2", "bf16", B=2, H=1, T=130, dk=64, dv=64, L=2, chunk=64, seed=174),
    "bf16_d64_L3": W("dl_bf16_d64_L3", "bf16", B=1, H=2, T=100, dk=64, dv=64, L=3, chunk=64, seed=175),
    "bf16_d64_L4": W("dl_bf16_d64_L4", "bf16", B=1, H=2, T=209, dk=64, dv=64, L=4, chunk=64, seed=176),
    "bf16_d64_L8": W("dl_bf16_d64_L8", "bf16", B=1, H=2, T=150, dk=64, dv=64, L=8, chunk=64, seed=177),
    "bf16_d128_L8": W("dl_bf16_d128", "bf16", B=1, H=2, T=130, dk=128, dv=128, L=8, chunk=64, seed=178),
    "bf16_dk64_dv128_L3": W("dl_bf16_unequal", "bf16", B=1, H=2, T=70, dk=64, dv=128, L=3, chunk=64, seed=179),
}


def _store(w):
    """The I/O type's rounding of a stored factor."""
    if w.dtype == "bf16":
        return lambda f: workloads.to_bf16_values(np.asarray(f, np.float32))
    return lambda f: np.asarray(f, np.float32)


def _inputs(w):
    x = workloads.generate(w)
    x["p"] = workloads.generate_gain(w)
    return x


def _dev(x, w):
    return workloads.to_torch({k: v for k, v in x.items() if k != "gamma"}, w.dtype)


@pytest.mark.parametrize("hist", [False, True])
@pytest.mark.parametrize("key", ["f32_d16_L2", "f32_d32_L3", "bf16_d64_L4", "bf16_d128_L8"])
def test_delta_factors(prism, key, hist):
    import torch
    w = CASES[key]
    x = _inputs(w)
    ci = workloads.generate_state(w)["conv_in"] if hist else None
    log(f"[delta gain] {key} hist={hist}")
    d = _dev(x, w)
    cid = workloads.to_torch({"conv_in": ci}, w.dtype)["conv_in"] if hist else None
    fac = prism.delta_gain(d["v"], d["p"], d["conv_w"], w.L, conv_in=cid)
    torch.cuda.synchronize()
    got = fac.float().cpu().numpy()
    ref = odl.delta_factors(x["v"], x["p"], x["conv_w"], w.L, conv_in=ci, rounding=_store(w))
    exact = odl.delta_factors(x["v"], x["p"], x["conv_w"], w.L, conv_in=ci)
    err = rel_err(got, ref)
    log(f"  factors rel err {err:.3e} (tol {GTOL[w.dtype]:.0e}); against unrounded chain {rel_err(got, exact):.3e}")
    assert err <= GTOL[w.dtype]


def _check_fwd(w, o, S, ref, tag):
    o = o.float().cpu().numpy()
    S = S.cpu().numpy()
    eo, es = rel_err(o, ref[0]), rel_err(S, ref[1])
    log(f"  {tag}: rel err o {eo:.3e}  S_final {es:.3e} (tol {TOL[w.dtype]:.0e})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def _oracle(w, x, heads=None):
    return odl.forward_delta(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["p"],
                             x["conv_w"], w.L, heads=heads)


@pytest.mark.parametrize("key", list(CASES))
def test_fwd_delta_parity(prism, key):
    import torch
    w = CASES[key]
    x = _inputs(w)
    log(f"[delta fwd] {key}")
    d = _dev(x, w)
    o, S = prism.fwd_delta(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["p"], d["conv_w"],
                           L=w.L, chunk=w.chunk)
    torch.cuda.synchronize()
    _check_fwd(w, o, S, _oracle(w, x), key)


@pytest.mark.parametrize("seg", [2, 3])
@pytest.mark.parametrize("L", [2, 3, 4, 8])
def test_fwd_delta_multichunk_segments(prism, L, seg):
    """The d = 64 written-correction sweep with segments of several chunks."""
    import torch
    w = W("dl_seg", "bf16", B=1, H=2, T=450, dk=64, dv=64, L=L, chunk=64, seed=180 + L)
    x = _inputs(w)
    log(f"[delta fwd] L={L} seg={seg} T={w.T}")
    d = _dev(x, w)
    o, S = prism.fwd_delta(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["p"], d["conv_w"],
                           L=w.L, chunk=w.chunk, seg_chunks=seg)
    torch.cuda.synchronize()
    _check_fwd(w, o, S, _oracle(w, x), f"L={L} seg={seg}")


@pytest.mark.parametrize("L", [2, 3, 5, 8])
def test_fwd_delta_half_split_segments(prism, L):
    """The d = 128 written-correction half-split sweep with segments of three chunks."""
    import torch
    w = W("dl_seg128", "bf16", B=2, H=1, T=5 * 64 + 21, dk=128, dv=128, L=L, chunk=64, seed=200 + L)
    x = _inputs(w)
    log(f"[delta fwd] d=128 L={L} seg=3 T={w.T}")
    d = _dev(x, w)
    o, S = prism.fwd_delta(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["p"], d["conv_w"],
                           L=w.L, chunk=w.chunk, seg_chunks=3)
    torch.cuda.synchronize()
    _check_fwd(w, o, S, _oracle(w, x), f"d128 L={L} seg=3")


def test_fwd_delta_generic_multichunk_segments(prism):
    import torch
    w = W("dl_gseg", "f32", B=1, H=2, T=7 * 32 + 5, dk=32, dv=32, L=4, chunk=32, seed=189)
    x = _inputs(w)
    d = _dev(x, w)
    o, S = prism.fwd_delta(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["p"], d["conv_w"],
                           L=w.L, chunk=w.chunk, seg_chunks=3)
    torch.cuda.synchronize()
    _check_fwd(w, o, S, _oracle(w, x), "generic f32 d32 seg=3")


PRED = {
    "d32_L3": W("dlp_d32", "bf16", B=2, H=2, T=75, dk=32, dv=32, L=3, chunk=32, seed=190),
    "d64_L4": W("dlp_d64", "bf16", B=1, H=2, T=209, dk=64, dv=64, L=4, chunk=64, seed=191),
    "d64_L8": W("dlp_d64_L8", "bf16", B=1, H=2, T=300, dk=64, dv=64, L=8, chunk=64, seed=192),
    "d128_L8": W("dlp_d128", "bf16", B=1, H=2, T=130, dk=128, dv=128, L=8, chunk=64, seed=193),
}


def _front(w, conv_in=None, anchor_rounding=None):
    x = workloads.generate(w)
    x.update(workloads.generate_front(w))
    p, u, alpha = odl.anchor_predict(x["v"], x["conv_w"], x["W_p"], x["W_k"], x["W_b"], w.L, conv_in=conv_in,
                                     anchor_rounding=anchor_rounding)
    return x, p, u, alpha


@pytest.mark.parametrize("hist", [False, True])
@pytest.mark.parametrize("key", list(PRED))
def test_anchor_predict(prism, key, hist):
    import torch
    w = PRED[key]
    ci = workloads.generate_state(w)["conv_in"] if hist else None
    x, p, u, alpha = _front(w, ci)
    # the kernel's gains: the anchor rounded to bfloat16 as the MFMA operand
    _, p_b, _, _ = _front(w, ci, anchor_rounding=_store(w))
    log(f"[front] {key} hist={hist}")
    d = workloads.to_torch({k: x[k] for k in ("v", "conv_w", "W_p", "W_k", "W_b")}, w.dtype)
    cid = workloads.to_torch({"conv_in": ci}, w.dtype)["conv_in"] if hist else None
    fac, uk, al = prism.anchor_predict(d["v"], d["conv_w"], d["W_p"], d["W_k"], d["W_b"], w.L, conv_in=cid)
    torch.cuda.synchronize()
    got_f = fac.float().cpu().numpy()
    ref_f = odl.delta_factors(x["v"], p_b, x["conv_w"], w.L, conv_in=ci, rounding=_store(w))
    ef = rel_err(got_f, ref_f)
    ex = rel_err(got_f, odl.delta_factors(x["v"], p, x["conv_w"], w.L, conv_in=ci))
    eu = rel_err(uk.float().cpu().numpy(), u)
    ea = float(np.max(np.abs(al.cpu().numpy() - alpha)))
    log(f"  factors {ef:.3e} (unrounded operands and chain {ex:.3e})  keys {eu:.3e}  gates (abs) {ea:.3e}")
    assert ef <= 1e-2 and eu <= 1e-2 and ea <= 1e-2
    norms = np.linalg.norm(uk.float().cpu().numpy(), axis=-1)
    assert np.max(np.abs(norms - 1.0)) < 2e-2


@pytest.mark.parametrize("key", list(PRED))
def test_fwd_delta_pred_parity(prism, key):
    import torch
    w = PRED[key]
    x, p, u, alpha = _front(w)
    log(f"[front fwd] {key}")
    d = workloads.to_torch({k: x[k] for k in ("q", "k", "v", "g", "beta", "conv_w", "W_p", "W_k", "W_b")},
                           w.dtype)
    o, S = prism.fwd_delta_pred(d["q"], d["k"], d["v"], d["g"], d["beta"], d["W_p"], d["W_k"], d["W_b"],
                                d["conv_w"], L=w.L, chunk=w.chunk)
    torch.cuda.synchronize()
    ref = odl.forward_delta(x["q"], x["k"], x["v"], x["g"], x["beta"], u, alpha, p, x["conv_w"], w.L)
    _check_fwd(w, o, S, ref, key)


def test_fwd_delta_pred_full_size_16k(prism):
    """The 16K workload's shape (B2 H4 T16384 d64 L4) through the front end and the
    written-correction sweep, head 2 of both batches against the oracle."""
    import torch
    w = workloads.workload("rec16k_bf16")
    x = workloads.generate(w)
    x.update(workloads.generate_front(w))
    log("[front fwd 16k] gpu")
    d = workloads.to_torch({k: x[k] for k in ("q", "k", "v", "g", "beta", "conv_w", "W_p", "W_k", "W_b")},
                           w.dtype)
    o, S = prism.fwd_delta_pred(d["q"], d["k"], d["v"], d["g"], d["beta"], d["W_p"], d["W_k"], d["W_b"],
                                d["conv_w"], L=w.L, chunk=w.chunk)
    torch.cuda.synchronize()
    o = o[:, 2:3].contiguous()
    S = S[:, 2:3].contiguous()
    log("[front fwd 16k] oracle head 2")
    hs = [2]
    p, u, alpha = odl.anchor_predict(x["v"][:, hs], x["conv_w"][hs], x["W_p"][hs], x["W_k"][hs], x["W_b"][hs], w.L)
    ref = odl.forward_delta(x["q"][:, hs], x["k"][:, hs], x["v"][:, hs], x["g"][:, hs], x["beta"][:, hs], u, alpha,
                            p, x["conv_w"][hs], w.L)
    _check_fwd(w, o, S, ref, "16k head 2")
