"""Parity of the HIP forward (through the C ABI) with the float64 oracle.

Tolerance (max-abs error relative to max |reference|, for o and for S_final):
1e-4 for float32 I/O, 2e-2 for bfloat16 I/O.  The bf16 path rounds MFMA operands
to bfloat16 (relative step 2^-8) while the state stays float32; the measured
errors sit one to two orders of magnitude under the bound.
"""
import sys
import time

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


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


def run_gpu(prism, w, x, chunk=None, seg=None):
    import torch
    d = workloads.to_torch(x, w.dtype)
    o, S = prism.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["gamma"], d["conv_w"],
                     L=w.L, chunk=chunk or w.chunk, seg_chunks=seg)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64)


def run_oracle(w, x, heads=None):
    return oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["gamma"],
                          x["conv_w"], w.L, heads=heads)


def check(w, got, ref, tag=""):
    eo, es = rel_err(got[0], ref[0]), rel_err(got[1], ref[1])
    log(f"  {w.name}{tag}: rel err o {eo:.3e}  S_final {es:.3e}  (tol {TOL[w.dtype]:.0e})")
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1]))
    assert eo <= TOL[w.dtype], f"o error {eo}"
    assert es <= TOL[w.dtype], f"S_final error {es}"


@pytest.mark.parametrize("name", workloads.ORDER)
def test_parity_full_size(prism, name):
    """Every workload at its full size; the 64K workload checks 2 of its 8 heads
    against the oracle (heads are independent) and all heads for finiteness."""
    w = workloads.workload(name)
    log(f"[parity] {name}: generating")
    x = workloads.generate(w)
    log(f"[parity] {name}: gpu")
    got = run_gpu(prism, w, x)
    heads = [0, 5] if name == "long64k_bf16" else None
    log(f"[parity] {name}: oracle heads={heads}")
    t = time.time()
    ref = run_oracle(w, x, heads)
    log(f"[parity] {name}: oracle took {time.time() - t:.1f}s")
    if heads is not None:
        assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1]))
        got = (got[0][:, heads], got[1][:, heads])
    check(w, got, ref)


SMALL = {
    "f32": workloads.Workload("small_f32", "f32", B=1, H=2, T=203, dk=32, dv=32, L=3, chunk=32, seed=11),
    "bf16": workloads.Workload("small_bf16", "bf16", B=2, H=1, T=331, dk=64, dv=64, L=4, chunk=64, seed=12),
    "bf16_128": workloads.Workload("small_bf16_128", "bf16", B=1, H=2, T=150, dk=128, dv=128, L=8, chunk=64, seed=13),
    "f32_64": workloads.Workload("small_f32_64", "f32", B=1, H=1, T=300, dk=64, dv=64, L=2, chunk=64, seed=14),
}


@pytest.mark.parametrize("key", list(SMALL))
def test_ragged_tail(prism, key):
    w = SMALL[key]
    x = workloads.generate(w)
    check(w, run_gpu(prism, w, x), run_oracle(w, x), " ragged")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 17])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_short_sequences(prism, T, dtype):
    w = workloads.Workload("short", dtype, B=2, H=1, T=T, dk=32, dv=32, L=3, chunk=16, seed=20 + T)
    x = workloads.generate(w)
    check(w, run_gpu(prism, w, x), run_oracle(w, x), f" T={T}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_size_independent(prism, chunk, dtype):
    w = workloads.Workload("chunks", dtype, B=1, H=2, T=256, dk=32, dv=32, L=4, chunk=chunk, seed=30)
    x = workloads.generate(w)
    check(w, run_gpu(prism, w, x), run_oracle(w, x), f" chunk={chunk}")


@pytest.mark.parametrize("seg", [1, 2, 3, 100])
def test_segment_size_independent(prism, seg):
    w = workloads.Workload("segs", "bf16", B=1, H=2, T=700, dk=64, dv=64, L=4, chunk=64, seed=40)
    x = workloads.generate(w)
    check(w, run_gpu(prism, w, x, seg=seg), run_oracle(w, x), f" seg={seg}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_L1_with_null_rank_pointers(prism, dtype):
    w = workloads.Workload("gdn", dtype, B=2, H=2, T=200, dk=64, dv=64, L=1, chunk=32, seed=50)
    x = workloads.generate(w)
    assert x["u"] is None and x["alpha"] is None and x["gamma"] is None
    check(w, run_gpu(prism, w, x), run_oracle(w, x), " L=1")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_correlated_keys(prism, dtype):
    w = workloads.Workload("corr", dtype, B=1, H=2, T=256, dk=64 if dtype == "bf16" else 32,
                           dv=64 if dtype == "bf16" else 32, L=3, chunk=64 if dtype == "bf16" else 32, seed=60)
    x = workloads.generate(w, keys="correlated")
    check(w, run_gpu(prism, w, x), run_oracle(w, x), " correlated keys")


def test_run_to_run_deterministic(prism):
    w = workloads.workload("rec16k_bf16").replace(T=2048)
    x = workloads.generate(w)
    a = run_gpu(prism, w, x)
    b = run_gpu(prism, w, x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_linear_in_v_on_device(prism):
    w = workloads.Workload("lin", "f32", B=1, H=2, T=300, dk=32, dv=32, L=3, chunk=32, seed=70)
    x1 = workloads.generate(w)
    x2 = dict(x1, v=workloads.generate(w, seed=71)["v"])
    x3 = dict(x1, v=(x1["v"] + 2.0 * x2["v"]).astype(np.float32))
    o1, _ = run_gpu(prism, w, x1)
    o2, _ = run_gpu(prism, w, x2)
    o3, _ = run_gpu(prism, w, x3)
    assert rel_err(o3, o1 + 2.0 * o2) < 1e-4


@pytest.mark.parametrize("L", [1, 2, 3, 5, 8])
def test_bf16_d64_c64_all_L(prism, L):
    """The specialised bf16 / d=64 / chunk=64 sweep streams the rank inputs one
    refinement step at a time; every L uses the two LDS slots differently."""
    w = workloads.Workload("fastL", "bf16", B=1, H=2, T=450, dk=64, dv=64, L=L, chunk=64, seed=80 + L)
    x = workloads.generate(w)
    check(w, run_gpu(prism, w, x), run_oracle(w, x), f" L={L}")


@pytest.mark.parametrize("T", [1, 3, 64, 65, 130])
def test_bf16_d64_c64_short(prism, T):
    w = workloads.Workload("fastT", "bf16", B=2, H=1, T=T, dk=64, dv=64, L=4, chunk=64, seed=90 + T)
    x = workloads.generate(w)
    check(w, run_gpu(prism, w, x), run_oracle(w, x), f" T={T}")


def test_bf16_d64_generic_chunk32_matches(prism):
    """chunk=32 at d=64 runs the generic sweep; both must meet the oracle."""
    w = workloads.Workload("gen32", "bf16", B=1, H=2, T=300, dk=64, dv=64, L=4, chunk=32, seed=95)
    x = workloads.generate(w)
    check(w, run_gpu(prism, w, x), run_oracle(w, x), " generic chunk=32")


# ---- segments spanning several chunks on every path -------------------------------------
# A segment of more than one chunk carries the state H and the segment operator A_acc from
# chunk to chunk inside one workgroup, and (on the bf16 d = 64 sweep) prefetches the next
# chunk at an L-dependent rank step and rotates the two rank-input slots across chunks.  The
# planner gives small problems one chunk per segment, so these cases force longer segments.

@pytest.mark.parametrize("seg", [2, 4])
@pytest.mark.parametrize("L", [1, 2, 3, 4, 5, 8])
def test_fast_sweep_multichunk_segments(prism, L, seg):
    w = workloads.Workload("fastseg", "bf16", B=1, H=2, T=600, dk=64, dv=64, L=L, chunk=64, seed=100 + L)
    x = workloads.generate(w)
    log(f"[parity] fast sweep L={L} seg={seg} T={w.T}")
    check(w, run_gpu(prism, w, x, seg=seg), run_oracle(w, x), f" L={L} seg={seg}")


# The bf16 d = 128 half-split sweep (two workgroups per segment, one per value half): every
# L it is instantiated for, with segments of several chunks and a ragged last chunk.
@pytest.mark.parametrize("seg", [2, 3])
@pytest.mark.parametrize("L", [1, 2, 3, 4, 5, 6, 7, 8])
def test_half_split_sweep_multichunk_segments(prism, L, seg):
    w = workloads.Workload("d128seg", "bf16", B=2, H=1, T=6 * 64 + 35, dk=128, dv=128, L=L, chunk=64,
                           seed=140 + L)
    x = workloads.generate(w)
    log(f"[parity] d=128 half-split sweep L={L} seg={seg} T={w.T}")
    check(w, run_gpu(prism, w, x, seg=seg), run_oracle(w, x), f" d128 L={L} seg={seg}")


# The d = 128 path in the planner's launch configuration at 48 pairs (the 130M layer's pair
# count, several segments per pair): every pair against the oracle, which covers the
# inter-segment scan's 32-column workgroups (more pairs than 256 / 8 of 16-column ones).
@pytest.mark.parametrize("L", [2, 4])
def test_half_split_planned_48_pairs(prism, L):
    w = workloads.Workload("d128plan", "bf16", B=8, H=6, T=7 * 64 + 20, dk=128, dv=128, L=L, chunk=64,
                           seed=170 + L)
    x = workloads.generate(w)
    log(f"[parity] d=128 planned launch L={L} T={w.T} pairs={w.B * w.H}")
    check(w, run_gpu(prism, w, x), run_oracle(w, x), f" d128 planned L={L}")


GENERIC_SEG = [
    # (dtype, d, chunk, L)
    ("f32", 16, 16, 3), ("f32", 32, 32, 4), ("f32", 64, 32, 2), ("f32", 64, 64, 5),
    ("bf16", 16, 16, 3), ("bf16", 32, 32, 8), ("bf16", 64, 32, 4), ("bf16", 128, 64, 4),
]


@pytest.mark.parametrize("seg", [2, 3])
@pytest.mark.parametrize("case", GENERIC_SEG, ids=lambda c: f"{c[0]}_d{c[1]}_c{c[2]}_L{c[3]}")
def test_generic_multichunk_segments(prism, case, seg):
    dt, d, chunk, L = case
    T = 6 * chunk + chunk // 2 + 3       # ragged last chunk
    w = workloads.Workload("genseg", dt, B=2, H=1, T=T, dk=d, dv=d, L=L, chunk=chunk, seed=110 + d + L)
    x = workloads.generate(w)
    log(f"[parity] generic {case} seg={seg} T={T}")
    check(w, run_gpu(prism, w, x, seg=seg), run_oracle(w, x), f" {case} seg={seg}")


# dk != dv (generic kernels): every key width meets every value width
UNEQUAL = [
    # (dtype, dk, dv, chunk, L)
    ("bf16", 64, 128, 64, 4), ("bf16", 128, 64, 64, 3), ("bf16", 32, 64, 32, 2), ("bf16", 16, 128, 16, 5),
    ("bf16", 128, 32, 32, 1), ("f32", 64, 32, 32, 3), ("f32", 32, 64, 64, 4), ("f32", 16, 32, 16, 2),
    ("f32", 128, 16, 16, 3),
]


@pytest.mark.parametrize("case", UNEQUAL, ids=lambda c: f"{c[0]}_dk{c[1]}_dv{c[2]}_c{c[3]}_L{c[4]}")
def test_unequal_key_value_widths(prism, case):
    dt, dk, dv, chunk, L = case
    T = 4 * chunk + 7
    w = workloads.Workload("unequal", dt, B=1, H=2, T=T, dk=dk, dv=dv, L=L, chunk=chunk, seed=130 + dk + dv + L)
    x = workloads.generate(w)
    log(f"[parity] dk={dk} dv={dv} {dt} chunk={chunk} L={L}")
    check(w, run_gpu(prism, w, x), run_oracle(w, x), f" dk={dk} dv={dv}")
    check(w, run_gpu(prism, w, x, seg=2), run_oracle(w, x), f" dk={dk} dv={dv} seg=2")


@pytest.mark.parametrize("L", [1, 2, 8])
def test_lsweep_shape_against_oracle(prism, L):
    """The L-sweep runs the 16K workload's shape (B2 H4 T16384 d64, chunk 64) at other L,
    in the planner's launch configuration (32 segments of 8 chunks per pair); heads 0 and 3
    are compared with the oracle, every head checked for finiteness."""
    w = workloads.workload("rec16k_bf16").replace(L=L, seed=140 + L)
    x = workloads.generate(w)
    log(f"[parity] L-sweep shape L={L}: gpu")
    got = run_gpu(prism, w, x)
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1]))
    heads = [0, 3]
    log(f"[parity] L-sweep shape L={L}: oracle heads={heads}")
    ref = run_oracle(w, x, heads)
    check(w, (got[0][:, heads], got[1][:, heads]), ref, f" L={L}")
