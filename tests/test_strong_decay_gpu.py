"""Near-total forgetting: gates g = exp(-x) with x up to 20 (g down to 2e-9), a run of
tokens with g = 1 exactly, and a few tokens at the smallest gate, on every forward path and
both backward forms, against the float64 oracle.

The workloads' own gates stay within exp(-0.1) .. 1, so the chunk decays (b = cumsum log g
over 64 tokens), the products exp(b_i - b_j) and the segment operators never come near
underflow there.  Here b reaches about -640 inside a chunk: G = exp(b) and the state's
carry across chunks underflow to zero (the exact limit), the masked differences b_i - b_j
must still be formed before the exponential, and the gate's gradient carries 1 / g up to
5e8.  Tolerances as elsewhere: 1e-4 (float32 I/O) and 2e-2 (bfloat16 I/O), max-abs error
relative to max |reference| per output or gradient.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def prism():
    if not gpu_available():
        pytest.skip("no GPU")
    import delta_rule_sequence_amd as m
    m.load_library()
    return m


def strong_gates(w, seed):
    rng = np.random.default_rng(seed)
    x = rng.uniform(0.0, 20.0, size=(w.B, w.H, w.T))
    x[..., 10:40] = 0.0           # a run without decay
    x[..., 5] = 20.0              # single tokens at the smallest gate
    x[..., w.T // 2] = 20.0
    return np.exp(-x).astype(np.float32)


def rel(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - b)) / max(1e-30, float(np.max(np.abs(b)))))


CASES = [
    # dtype, d, chunk, L, T: the bf16 d = 64 sweep (with segments of two chunks), the bf16
    # d = 128 half-split sweep, the generic sweep in float32
    ("bf16", 64, 64, 4, 300, 2),
    ("bf16", 128, 64, 3, 200, 2),
    ("f32", 32, 32, 3, 150, 2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_d{c[1]}_L{c[3]}")
def test_forward_strong_decay(prism, case):
    import torch
    dt, d, chunk, L, T, seg = case
    w = workloads.Workload("decay", dt, B=1, H=2, T=T, dk=d, dv=d, L=L, chunk=chunk, seed=400 + d)
    x = workloads.generate(w)
    x["g"] = strong_gates(w, 401 + d)
    ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["gamma"],
                         x["conv_w"], L)
    dv = workloads.to_torch(x, dt)
    for sc in (None, seg):
        o, S = prism.fwd(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["u"], dv["alpha"], dv["gamma"],
                         dv["conv_w"], L=L, chunk=chunk, seg_chunks=sc)
        torch.cuda.synchronize()
        o = o.float().cpu().numpy()
        S = S.cpu().numpy()
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
        eo, es = rel(o, ref[0]), rel(S, ref[1])
        print(f"[decay] fwd {case} seg={sc}: o {eo:.2e} S_final {es:.2e}", flush=True)
        assert eo <= TOL[dt] and es <= TOL[dt]


@pytest.mark.parametrize("L", [1, 4, 8])
@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "float32"])
def test_backward_strong_decay(prism, chunked, L):
    import torch
    from oracle import prism_grad
    from tests.test_bwd_gpu import _setup
    dt = "bf16" if chunked else "f32"
    T = 200
    w, x, d_o, dS = _setup(dt, 1, 2, T, 64, L, True, seed=410)
    x["g"] = strong_gates(w, 411)
    dv = workloads.to_torch(x, dt)
    vt = torch.bfloat16 if dt == "bf16" else torch.float32
    got = prism.bwd(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["u"], dv["alpha"], dv["gamma"],
                    dv["conv_w"], L=L, d_o=torch.tensor(d_o, device="cuda").to(vt),
                    dS_final=torch.tensor(dS, device="cuda"), chunked=chunked)
    torch.cuda.synchronize()
    ref = prism_grad.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["gamma"],
                              x["conv_w"], L, d_o, dS)
    errs = {}
    for n in ["dq", "dk", "dv", "dg", "dbeta"] + (["du", "dalpha", "dgamma", "dconv_w"] if L > 1 else []):
        g = got[n].cpu().numpy()
        assert np.all(np.isfinite(g)), n
        errs[n] = rel(g, ref[n])
    print(f"[decay] bwd chunked={chunked} L={L}: " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)
    tol = 2e-2 if chunked else 1e-4
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
