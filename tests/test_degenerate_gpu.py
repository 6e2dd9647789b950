"""Degenerate inputs of the method on every forward path (the bf16 d = 64 and d = 128 sweeps,
the generic sweep in float32 and bf16) and both backward forms,
against the float64 oracle (forward) and gradient oracle (backward):

* beta = 1 everywhere: each write fully replaces the value read along k (the delta rule's
  projection I - k k^T with unit keys);
* beta = 0 everywhere: no GDN write, the state is built from the rank-L writes alone;
* alpha = 0: the rank-L writes vanish (the GDN forward with the rank inputs present);
* one key for every token, with beta = 1: the intra-chunk triangular system is as
  ill-conditioned as unit keys allow (M_ij = Gam_ij for all j < i), and each token erases
  the previous one's write.

Tolerances as elsewhere: 2e-2 (bf16 forward and chunked backward), 1e-4 (float32 forward
and backward),
max-abs error relative to max |reference| per output or gradient; where a reference is
identically zero (du, dgamma and dconv_w at alpha = 0: nothing is written along u), the
largest entry over all gradients is the scale.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def prism():
    if not gpu_available():
        pytest.skip("no GPU")
    import delta_rule_sequence_amd as m
    m.load_library()
    return m


def degenerate(kind, x):
    y = dict(x)
    if kind == "beta1":
        y["beta"] = np.ones_like(x["beta"])
    elif kind == "beta0":
        y["beta"] = np.zeros_like(x["beta"])
    elif kind == "alpha0":
        y["alpha"] = np.zeros_like(x["alpha"])
    elif kind == "one_key":
        y["k"] = np.broadcast_to(x["k"][:, :, :1], x["k"].shape).copy()
        y["beta"] = np.ones_like(x["beta"])
    return y


KINDS = ["beta1", "beta0", "alpha0", "one_key"]


def rel(a, b, scale=None):
    s = float(np.max(np.abs(b))) if scale is None else scale
    return float(np.max(np.abs(np.asarray(a, np.float64) - b)) / max(1e-30, s))


# (dtype, d, chunk): the bf16 d = 64 and d = 128 sweeps and the generic sweep
FWD_PATHS = [("bf16", 64, 64), ("bf16", 128, 64), ("f32", 32, 32), ("bf16", 32, 16)]


@pytest.mark.parametrize("path", FWD_PATHS, ids=lambda p: f"{p[0]}_d{p[1]}_c{p[2]}")
@pytest.mark.parametrize("kind", KINDS)
def test_forward_degenerate(prism, kind, path):
    import torch
    dt, d, chunk = path
    w = workloads.Workload("degen", dt, B=1, H=2, T=300, dk=d, dv=d, L=4, chunk=chunk, seed=500)
    y = degenerate(kind, workloads.generate(w))
    ref = oracle.forward(y["q"], y["k"], y["v"], y["g"], y["beta"], y["u"], y["alpha"], y["gamma"], y["conv_w"], w.L)
    t = workloads.to_torch(y, dt)
    tol = 2e-2 if dt == "bf16" else 1e-4
    for sc in (None, 2):
        o, S = prism.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["u"], t["alpha"], t["gamma"], t["conv_w"],
                         L=w.L, chunk=chunk, seg_chunks=sc)
        torch.cuda.synchronize()
        eo, es = rel(o.float().cpu().numpy(), ref[0]), rel(S.cpu().numpy(), ref[1])
        print(f"[degenerate] fwd {kind} {path} seg={sc}: o {eo:.2e} S_final {es:.2e}", flush=True)
        assert eo <= tol and es <= tol


@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "float32"])
@pytest.mark.parametrize("kind", KINDS)
def test_backward_degenerate(prism, kind, chunked):
    import torch
    from oracle import prism_grad
    from tests.test_bwd_gpu import _setup
    dt = "bf16" if chunked else "f32"
    L = 4
    w, x, d_o, dS = _setup(dt, 1, 2, 200, 64, L, True, seed=510)
    y = degenerate(kind, x)
    d = workloads.to_torch(y, dt)
    vt = torch.bfloat16 if dt == "bf16" else torch.float32
    got = prism.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["gamma"], d["conv_w"], L=L,
                    d_o=torch.tensor(d_o, device="cuda").to(vt), dS_final=torch.tensor(dS, device="cuda"),
                    chunked=chunked)
    torch.cuda.synchronize()
    ref = prism_grad.backward(y["q"], y["k"], y["v"], y["g"], y["beta"], y["u"], y["alpha"], y["gamma"],
                              y["conv_w"], L, d_o, dS)
    names = ["dq", "dk", "dv", "dg", "dbeta", "du", "dalpha", "dgamma", "dconv_w"]
    scale = max(float(np.max(np.abs(ref[n]))) for n in names)
    errs = {}
    for n in names:
        g = got[n].cpu().numpy()
        assert np.all(np.isfinite(g)), n
        rmax = float(np.max(np.abs(ref[n])))
        errs[n] = rel(g, ref[n], rmax if rmax > 0 else scale)
    print(f"[degenerate] bwd {kind} chunked={chunked}: " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()),
          flush=True)
    tol = 2e-2 if chunked else 1e-4
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
