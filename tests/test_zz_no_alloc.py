"""prism_fwd_noalloc (the forward whose workspace is the library's static device array)
against prism_fwd (caller workspace), both called through the C ABI.

Two calls in a row on one GPU, the second on a smaller input, so the second call runs
over the array the first one left filled: each result must equal prism_fwd's on the same
inputs bit for bit (the same kernels, the same segment plan, deterministic reductions).
"""
import ctypes
import sys

import numpy as np
import pytest

import workloads
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not gpu_available():
        pytest.skip("no GPU")
    import delta_rule_sequence_amd as m
    return m.load_library()


def _run(lib, w, x, noalloc):
    import torch
    import delta_rule_sequence_amd as m
    d = workloads.to_torch(x, w.dtype, "cuda")
    dt = m.PRISM_BF16 if w.dtype == "bf16" else m.PRISM_F32
    vt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    o = torch.full((w.B, w.H, w.T, w.dv), float("nan"), dtype=vt, device="cuda")
    S = torch.full((w.B, w.H, w.dk, w.dv), float("nan"), dtype=torch.float32, device="cuda")
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    args = [p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]), p(d["u"]), p(d["alpha"]), p(d["gamma"]),
            p(d["conv_w"]), w.B, w.H, w.T, w.dk, w.dv, w.L, w.chunk, dt, p(o), p(S)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        lib.prism_fwd_noalloc.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 8 + [ctypes.c_void_p] * 3
        lib.prism_fwd_noalloc.restype = ctypes.c_int
        st = lib.prism_fwd_noalloc(*args, stream)
    else:
        need = lib.prism_fwd_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.L, w.chunk, dt)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        st = lib.prism_fwd(*args, ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(need), stream)
    assert st == 0, m.status_string(st)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


CASES = [
    # the 16K workload (bf16 d = 64 fast path), then a smaller generic-path problem
    (workloads.workload("rec16k_bf16"), workloads.Workload("na_small", "f32", B=1, H=2, T=300, dk=32, dv=32,
                                                           L=3, chunk=32, seed=160)),
    # two fast-path calls, the second shorter (fewer segments in the shared array)
    (workloads.Workload("na_a", "bf16", B=1, H=2, T=2000, dk=64, dv=64, L=4, chunk=64, seed=161),
     workloads.Workload("na_b", "bf16", B=1, H=1, T=333, dk=64, dv=64, L=2, chunk=64, seed=162)),
]


@pytest.mark.parametrize("pair", CASES, ids=["16k_then_f32", "fast_then_shorter"])
def test_noalloc_matches_fwd_twice(lib, pair):
    for w in pair:
        log(f"[noalloc] {w.name} B={w.B} H={w.H} T={w.T} d={w.dk} L={w.L} {w.dtype}")
        x = workloads.generate(w)
        o1, S1 = _run(lib, w, x, noalloc=True)
        o2, S2 = _run(lib, w, x, noalloc=False)
        assert np.all(np.isfinite(o1)) and np.all(np.isfinite(S1))
        assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
