"""Starting state, ShortConv window and one-token decode on the GPU (through the C ABI)
against the float64 oracle.

Tolerances as the forward parity tests (max-abs error relative to max |reference|):
1e-4 for float32 I/O, 2e-2 for bfloat16 I/O.  The carried ShortConv window is a copy of
input values, so it is compared bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}

CASES = {
    # bf16, d = 64, chunk 64, L <= 4: the two-wave sweep path (4 segments of 1 chunk and a tail)
    "bf16_d64": workloads.Workload("state_bf16_d64", "bf16", B=1, H=2, T=209, dk=64, dv=64, L=4, chunk=64, seed=70),
    # float32 and bf16 d = 128 through the generic chunk kernel
    "f32_d32": workloads.Workload("state_f32_d32", "f32", B=2, H=1, T=100, dk=32, dv=32, L=3, chunk=32, seed=71),
    "bf16_d128": workloads.Workload("state_bf16_d128", "bf16", B=1, H=2, T=130, dk=128, dv=128, L=4, chunk=64,
                                    seed=72),
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


def _slice(x, a, b):
    return {k: (None if v is None else (v if k == "conv_w" else v[:, :, a:b])) for k, v in x.items()}


def _gpu_fwd_state(prism, w, x, S0=None, conv_in=None):
    import torch
    d = workloads.to_torch(x, w.dtype)
    st = workloads.to_torch({"S0": S0, "conv_in": conv_in}, w.dtype)
    o, S, conv = prism.fwd_state(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["gamma"],
                                 d["conv_w"], L=w.L, chunk=w.chunk, S0=st["S0"], conv_in=st["conv_in"])
    torch.cuda.synchronize()
    return (o.float().cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64),
            conv.float().cpu().numpy())


def _oracle(w, x, S0=None, conv_in=None):
    return oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["gamma"],
                          x["conv_w"], w.L, S0=S0, conv_in=conv_in)


def _check(tag, w, o, S, ref_o, ref_S):
    eo, es = rel_err(o, ref_o), rel_err(S, ref_S)
    log(f"  {tag}: rel err o {eo:.3e}  S_final {es:.3e}  (tol {TOL[w.dtype]:.0e})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


@pytest.mark.parametrize("key", list(CASES))
def test_start_state_and_history(prism, key):
    w = CASES[key]
    x = workloads.generate(w)
    st = workloads.generate_state(w)
    o, S, conv = _gpu_fwd_state(prism, w, x, st["S0"], st["conv_in"])
    ro, rS = _oracle(w, x, st["S0"], st["conv_in"])
    _check(f"{w.name} from (S0, history)", w, o, S, ro, rS)
    assert np.array_equal(conv, x["v"][:, :, w.T - 3:])


@pytest.mark.parametrize("key", list(CASES))
def test_split_and_resume(prism, key):
    # [0, T1) then [T1, T) from the first call's (S_final, window) = one call over [0, T)
    w = CASES[key]
    x = workloads.generate(w)
    T1 = w.T // 2 + 3  # not a chunk boundary
    o1, S1, c1 = _gpu_fwd_state(prism, w.replace(T=T1), _slice(x, 0, T1))
    o2, S2, _ = _gpu_fwd_state(prism, w.replace(T=w.T - T1), _slice(x, T1, w.T), S1.astype(np.float32), c1)
    ro, rS = _oracle(w, x)
    _check(f"{w.name} split at {T1}", w, np.concatenate([o1, o2], axis=2), S2, ro, rS)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_window_shorter_than_three(prism, dtype):
    # T = 2: the new window keeps the newest given row
    w = workloads.Workload("state_short", dtype, B=1, H=2, T=2, dk=32, dv=32, L=3, chunk=16, seed=73)
    x = workloads.generate(w)
    st = workloads.generate_state(w)
    o, S, conv = _gpu_fwd_state(prism, w, x, st["S0"], st["conv_in"])
    ro, rS = _oracle(w, x, st["S0"], st["conv_in"])
    _check("T=2 from (S0, history)", w, o, S, ro, rS)
    assert np.array_equal(conv, np.concatenate([st["conv_in"][:, :, 2:], x["v"]], axis=2))


DECODE = {
    "bf16_d64_L4": workloads.Workload("dec_bf16_d64", "bf16", B=2, H=4, T=6, dk=64, dv=64, L=4, chunk=64, seed=80),
    "f32_d32_L3": workloads.Workload("dec_f32_d32", "f32", B=1, H=3, T=6, dk=32, dv=32, L=3, chunk=32, seed=81),
    "bf16_d128_L8": workloads.Workload("dec_bf16_d128", "bf16", B=1, H=2, T=5, dk=128, dv=128, L=8, chunk=64,
                                       seed=82),
    "f32_d16_L1": workloads.Workload("dec_f32_d16", "f32", B=2, H=2, T=5, dk=16, dv=16, L=1, chunk=16, seed=83),
}


@pytest.mark.parametrize("key", list(DECODE))
def test_decode_steps(prism, key):
    # T decode steps from (S0, history) = the oracle over those T tokens from the same start
    import torch
    w = DECODE[key]
    x = workloads.generate(w)
    st = workloads.generate_state(w)
    d = workloads.to_torch(x, w.dtype)
    s = workloads.to_torch(st, w.dtype)
    S, conv = s["S0"].clone(), s["conv_in"].clone()
    outs = []
    for t in range(w.T):
        pick = lambda name: None if d[name] is None else d[name][:, :, t].contiguous()
        o = prism.decode_step(S, conv, pick("q"), pick("k"), pick("v"), pick("g"), pick("beta"),
                              pick("u"), pick("alpha"), pick("gamma"), d["conv_w"] if w.L > 1 else None, L=w.L)
        outs.append(o.float().cpu().numpy().astype(np.float64))
    torch.cuda.synchronize()
    ro, rS = _oracle(w, x, st["S0"], st["conv_in"])
    _check(f"{w.name} {w.T} decode steps", w, np.stack(outs, axis=2), S.cpu().numpy().astype(np.float64), ro, rS)
    assert np.array_equal(conv.float().cpu().numpy(), x["v"][:, :, w.T - 3:])
