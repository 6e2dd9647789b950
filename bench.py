"""Benchmark of the PRISM rank-L gated delta-rule forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload rec16k_bf16] [--no-cpu-baseline]

One step = one prism_fwd call (segment sweep + segment scan + output
correction) over one batch of synthetic inputs already resident in HBM.  Input
sets are rotated so the working set exceeds the 256 MB Infinity Cache.  The K
timed steps run twice: plainly (the reported tokens/s) and with HIP events on
the launch stream around each kernel (the dominant kernel's duration, hence its
achieved HBM bandwidth against the 8 TB/s peak).  Prints one JSON line, with the
float64 oracle timed on the host cores on a bounded sample.

    python bench.py --bwd [--workload NAME] [--steps K] [--bwd-form auto|chunked|float32]
times the backward pass instead (the chunked MFMA form where it applies, else prism_bwd)
and prints its own JSON line.

    python bench.py --nl [--workload NAME] [--steps K]
times the forward with the nonlinear refinement (prism_fwd_nl) and its factor kernel.

    python bench.py --calibrate-copy MB
runs a plain device-to-device copy of MB megabytes (for scaling the
FETCH_SIZE / WRITE_SIZE counters of rocprofv3) and exits.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16
MALL_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic_bytes(w):
    """Bytes the method must move per token-head (inputs once, output once) and
    the share read by the segment-sweep kernel (all inputs)."""
    E = 2 if w.dtype == "bf16" else 4
    rank = (w.L - 1) * (w.dk + w.dv) * E + (4 * w.L if w.L > 1 else 0)
    inputs = (2 * w.dk + w.dv) * E + rank + 8
    return inputs, inputs + w.dv * E


# the sources the segment-sweep kernel is compiled from, and the build flags
SWEEP_SOURCES = ["delta_rule_sequence_amd/csrc/prism_sweep8.h", "delta_rule_sequence_amd/csrc/prism_fast.h",
                 "delta_rule_sequence_amd/csrc/prism_kernels.h", "delta_rule_sequence_amd/csrc/prism_tile.h",
                 "delta_rule_sequence_amd/csrc/prism_nl.h", "delta_rule_sequence_amd/csrc/prism_generic_launch.h",
                 "delta_rule_sequence_amd/csrc/fwd_fast_linear.hip", "delta_rule_sequence_amd/csrc/prism_sweep128.h",
                 "delta_rule_sequence_amd/csrc/fwd_fast128_linear.hip", "delta_rule_sequence_amd/build.py"]


def kernel_source_hash():
    """Hash of the sweep kernel's sources: counters taken with other sources are void."""
    h = hashlib.sha256()
    for f in SWEEP_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload_name):
    """HBM bytes per launch of the segment-sweep kernel from the committed
    rocprofv3 counter summary, or None if the kernels changed since."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(workload_name)
    if not ent or ent.get("kernel_source_sha") != kernel_source_hash():
        return None
    # FETCH_SIZE / WRITE_SIZE in KiB per dispatch, scaled by the copy-kernel calibration
    return int(1024 * (ent["fetch_kib"] * ent["fetch_scale"] + ent["write_kib"] * ent["write_scale"]))


class Hip:
    """Minimal ctypes access to HIP events (the library records them on the
    stream its kernels run on)."""

    def __init__(self):
        self.lib = None
        for name in ["libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"]:
            try:
                self.lib = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if self.lib is None:
            raise RuntimeError("libamdhip64.so not found")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def cpu_baseline(w, x, budget_s=10.0):
    """The float64 oracle on the host, single-threaded, on whole sequences of
    the workload's first input set (repeated until `budget_s` has elapsed)."""
    import numpy as np  # noqa: F401
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    tokens = 0
    runs = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["u"], x["alpha"], x["gamma"],
                       x["conv_w"], w.L)
        tokens += w.B * w.T
        runs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {"value": tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{runs} full pass(es) of {w.name} (B={w.B}, H={w.H}, T={w.T}), all heads, "
                      f"float64 numpy, one thread, {dt:.1f} s"}


_PAIR_DATA = None  # per-pair oracle inputs, inherited by the forked workers


def _oracle_pair(p):
    """Pair p through the oracle in a single-threaded worker process."""
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        oracle.forward_pairs(*_PAIR_DATA[p])
    return p


def cpu_baseline_parallel(w, x, budget_s=5.0):
    """The oracle with one single-threaded worker per (b, h) pair (P = min(pairs,
    usable cores, 16) processes), whole passes of the first input set until
    `budget_s` has elapsed.  Runs before the GPU is touched (workers are forked and
    inherit the inputs)."""
    import multiprocessing as mp
    import numpy as np
    global _PAIR_DATA
    usable = len(os.sched_getaffinity(0))
    procs = max(1, min(w.pairs, usable, 16))
    P = w.pairs

    def pick(a):
        return None if a is None else np.asarray(a).reshape((P,) + a.shape[2:])

    conv = np.broadcast_to(np.asarray(x["conv_w"])[None], (w.B, w.H, 4, w.dv)).reshape(P, 4, w.dv)
    cols = [pick(x["q"]), pick(x["k"]), pick(x["v"]), pick(x["g"]), pick(x["beta"]),
            pick(x["u"]), pick(x["alpha"]), pick(x["gamma"]), conv]
    _PAIR_DATA = [tuple(None if a is None else a[p_:p_ + 1] for a in cols) + (w.L,) for p_ in range(P)]
    tokens, runs = 0, 0
    with mp.get_context("fork").Pool(procs) as pool:
        t0 = time.perf_counter()
        while True:
            pool.map(_oracle_pair, range(P))
            tokens += w.B * w.T
            runs += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    _PAIR_DATA = None
    return {"value": tokens / dt, "unit": "tokens/s", "cores": procs, "kind": "oracle",
            "cpu_count": os.cpu_count(), "usable_cores": usable,
            "sample": f"{runs} full pass(es) of {w.name}, one single-threaded process per (b, h) "
                      f"pair over {procs} processes, {dt:.1f} s"}


def copy_bandwidth(torch, mb=1024, reps=10):
    """Measured device-to-device copy rate (read + write bytes per second)."""
    n = mb * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    del a, b
    return {"value": 2 * n * 4 * reps / dt / 1e9, "unit": "GB/s", "bytes_per_copy": 2 * n * 4}


def mfma_rate(torch, n=8192, reps=10):
    """Measured dense bf16 matrix rate: a vendor GEMM (torch.mm on contiguous n x n bfloat16
    operands, float32 accumulation inside) as the achievable MFMA ceiling beside the peak."""
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = torch.mm(a, b)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        c = torch.mm(a, b)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    del a, b, c
    return {"value": 2.0 * n ** 3 * reps / dt / 1e12, "unit": "TFLOP/s", "shape": [n, n, n], "dtype": "bf16",
            "via": "torch.mm"}


def calibrate_copy(mb):
    import torch
    n = mb * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": 3}))


def time_workload(w, steps, warmup, sets, x0=None):
    """Rotated input sets of workload w in HBM, warm-up, then the two timed regions
    (plain, and with per-kernel HIP events).  Returns the timings."""
    import numpy as np
    import torch

    import delta_rule_sequence_amd as prism
    import workloads

    lib = prism.load_library()
    dt = prism.PRISM_BF16 if w.dtype == "bf16" else prism.PRISM_F32
    in_bytes, _ = algorithmic_bytes(w)
    set_bytes = w.pairs * w.T * in_bytes
    nsets = sets or max(1, -(-2 * MALL_BYTES // set_bytes))
    print(f"[bench] {w.name}: {nsets} input set(s) of {set_bytes / 1e6:.1f} MB", file=sys.stderr, flush=True)
    dev_sets = []
    for i in range(nsets):
        x = x0 if (i == 0 and x0 is not None) else workloads.generate(w, seed=w.seed + 1000 * i)
        dev_sets.append(workloads.to_torch(x, w.dtype, "cuda"))
    vt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    o = torch.empty((w.B, w.H, w.T, w.dv), dtype=vt, device="cuda")
    S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    need = lib.prism_fwd_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.L, w.chunk, dt)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)

    def argv(d):
        p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
        return [p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]), p(d["u"]), p(d["alpha"]),
                p(d["gamma"]), p(d["conv_w"]), w.B, w.H, w.T, w.dk, w.dv, w.L, w.chunk, dt,
                ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(S.data_ptr()),
                ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(need)]

    calls = [argv(d) for d in dev_sets]
    for i in range(warmup):
        st = lib.prism_fwd(*calls[i % nsets], sh)
        if st != 0:
            raise RuntimeError(prism.status_string(st))
    torch.cuda.synchronize()

    # timed region 1 (the reported throughput): K forwards back to back, no instrumentation
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        st = lib.prism_fwd(*calls[i % nsets], sh)
        if st != 0:
            raise RuntimeError(prism.status_string(st))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # timed region 2: the same K forwards with HIP events recorded on the launch stream
    # around each of the three kernels (the per-kernel durations of the roofline)
    hip = Hip()
    evs = hip.events(4 * steps)
    ev_arrays = [(ctypes.c_void_p * 4)(*evs[4 * i:4 * i + 4]) for i in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        st = lib.prism_fwd_timed(*calls[i % nsets], ev_arrays[i], sh)
        if st != 0:
            raise RuntimeError(prism.status_string(st))
    torch.cuda.synchronize()
    per = np.array([[hip.elapsed_ms(evs[4 * i + j], evs[4 * i + j + 1]) for j in range(3)]
                    for i in range(steps)])
    # each call's own duration, first event to last (the three kernels and the gaps between)
    call_ms = np.array([hip.elapsed_ms(evs[4 * i], evs[4 * i + 3]) for i in range(steps)])
    span_ms = hip.elapsed_ms(evs[0], evs[4 * steps - 1])
    hip.destroy(evs)
    del dev_sets, o, S, ws
    return {"ms_per_step": 1e3 * wall / steps, "per": per, "span_ms": span_ms, "nsets": nsets,
            "call_ms": call_ms}


def l_sweep(steps, warmup):
    """The 16K bf16 shape at L = 1 (the plain gated delta rule), 2, 4 and 8: one JSON
    line per L with whole-forward tokens/s and the sweep's HBM roofline fraction, and for
    L > 1 the nonlinear-refinement forward (prism_fwd_nl) on the same shape."""
    import workloads
    base = workloads.workload("rec16k_bf16")
    for L in (1, 2, 4, 8):
        w = base.replace(L=L, name=f"rec16k_bf16_L{L}")
        nl = time_nl(w, max(10, steps // 2), warmup) if L > 1 else None
        t = time_workload(w, steps, warmup, 0)
        in_bytes, path_bytes = algorithmic_bytes(w)
        sweep_ms = float(t["per"][:, 0].mean())
        sweep_bytes = w.pairs * w.T * in_bytes
        print(json.dumps({"workload": w.name, "L": L, "tokens_per_s": w.B * w.T / (t["ms_per_step"] * 1e-3),
                          "ms_per_step": t["ms_per_step"],
                          "kernel_ms": {"sweep": sweep_ms, "scan": float(t["per"][:, 1].mean()),
                                        "fixup": float(t["per"][:, 2].mean())},
                          "input_bytes_per_token_head": in_bytes,
                          "sweep_hbm_frac": sweep_bytes / (sweep_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "path_hbm_roofline_tokens_per_s":
                              w.B * w.T * HBM_PEAK_GBS * 1e9 / (w.pairs * w.T * path_bytes),
                          "nl_ms_per_step": None if nl is None else nl["ms_per_step"],
                          "nl_tokens_per_s": None if nl is None else nl["tokens_per_s"]}), flush=True)


def decode_bench(steps, warmup, batch):
    """One-token decode steps (prism_decode_step) at the 16K workload's head shape (H = 4,
    d = 64, L = 4, bf16) for `batch` sequences: the float32 state (batch x 4 x 16 KB) is
    read and written once per step, so the step is HBM-bound once the state exceeds the
    256 MB Infinity Cache.  One JSON line: tokens/s (one token per sequence per step) and
    the step's algorithmic bytes against the HBM peak."""
    import torch
    import workloads
    import delta_rule_sequence_amd as prism
    base = workloads.workload("rec16k_bf16")
    w = base.replace(B=batch, T=steps + warmup, name=f"decode_b{batch}")
    x = workloads.to_torch(workloads.generate(w, seed=w.seed), w.dtype)
    st = workloads.to_torch(workloads.generate_state(w), w.dtype)
    S, conv = st["S0"], st["conv_in"]
    per_step = []
    for t in range(w.T):
        per_step.append({k: (x[k][:, :, t].contiguous() if x[k] is not None and k != "conv_w" else x[k])
                         for k in ("q", "k", "v", "g", "beta", "u", "alpha", "gamma")})
    del x["q"], x["k"], x["v"], x["u"], x["gamma"]

    def step(t):
        d = per_step[t]
        prism.decode_step(S, conv, d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["gamma"],
                          x["conv_w"], L=w.L)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(warmup, warmup + steps):
        step(t)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    P, d, L, E = w.B * w.H, w.dk, w.L, 2
    step_bytes = P * (2 * d * d * 4                          # state read + write
                      + 2 * 3 * d * E                        # window read + write
                      + (3 * d + 2 * (L - 1) * d) * E        # q, k, v, u, gamma
                      + (2 + L) * 4                          # g, beta, alpha
                      + d * E)                               # o
    print(json.dumps({"metric": "decode tokens/sec (prism_decode_step), H=4, d=64, L=4, bf16",
                      "batch": w.B, "steps": steps, "warmup": warmup, "ms_per_step": dt * 1e3,
                      "tokens_per_s": w.B / dt, "state_bytes": P * d * d * 4,
                      "achieved_GBs": step_bytes / dt / 1e9, "peak_GBs": HBM_PEAK_GBS,
                      "frac": step_bytes / dt / 1e9 / HBM_PEAK_GBS}), flush=True)


def bwd_bench(steps, warmup, workload_name, cpu=True, form="auto"):
    """The backward on one workload (form: "chunked" prism_bwd_chunked, "float32" prism_bwd,
    "auto" the chunked form where it applies): whole calls timed with HIP events on the
    launch stream.  One JSON line: tokens/s and the call's algorithmic bytes (inputs and
    d_o read once, every gradient written once in float32) against the HBM peak, beside
    the float64 gradient oracle timed on a bounded sample (one pair, 512 tokens)."""
    import numpy as np
    import torch
    import delta_rule_sequence_amd as prism
    import workloads
    w = workloads.workload(workload_name)
    x = workloads.generate(w, seed=w.seed)
    rng = np.random.default_rng(w.seed + 7)
    d_o = rng.standard_normal((w.B, w.H, w.T, w.dv)).astype(np.float32)
    if w.dtype == "bf16":
        d_o = workloads.to_bf16_values(d_o)
    cpu_out = None
    if cpu:
        from oracle import prism_grad
        Ts = min(w.T, 512)
        sl = lambda a: None if a is None else np.ascontiguousarray(a[:1, :1, :Ts])  # noqa: E731
        t0 = time.perf_counter()
        prism_grad.backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), sl(x["u"]),
                            sl(x["alpha"]), sl(x["gamma"]), x["conv_w"][:1], w.L, sl(d_o))
        dt_cpu = time.perf_counter() - t0
        cpu_out = {"value": Ts / dt_cpu, "unit": "tokens/s (per head)", "cores": torch.get_num_threads(),
                   "kind": "oracle", "sample": f"one (b, h) pair, {Ts} tokens, float64 autograd, {dt_cpu:.1f} s"}
    chunked = form == "chunked" or (form == "auto" and bwd_chunked_supported(w))
    res = time_bwd(w, x, d_o, steps, warmup, chunked=chunked)
    name = "prism_bwd_chunked" if chunked else "prism_bwd"
    print(json.dumps({"metric": f"bwd tokens/sec ({name})", "workload": w.name, "dtype": w.dtype,
                      "config": {"B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv, "L": w.L},
                      "steps": steps, "warmup": warmup, "ms_per_step": res["ms_per_step"],
                      "tokens_per_s": res["tokens_per_s"], "roofline": res["roofline"],
                      "cpu_baseline": cpu_out}), flush=True)


def bwd_chunked_supported(w):
    """prism_bwd_chunked covers bfloat16 inputs at dk = dv = 64."""
    return w.dtype == "bf16" and w.dk == 64 and w.dv == 64


def time_bwd(w, x, d_o, steps, warmup, chunked=False):
    """prism_bwd (or, chunked, prism_bwd_chunked) on workload w (inputs x, output gradient
    d_o): whole calls timed with HIP events on the launch stream; returns ms per call,
    tokens/s and the HBM roofline of the call's algorithmic bytes."""
    import torch
    import delta_rule_sequence_amd as prism
    import workloads
    dev = workloads.to_torch(x, w.dtype, "cuda")
    vt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    do_t = torch.tensor(d_o, device="cuda").to(vt)
    args = (dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["u"], dev["alpha"], dev["gamma"],
            dev["conv_w"])
    lib = prism.load_library()
    sizer = lib.prism_bwd_chunked_workspace_bytes if chunked else lib.prism_bwd_workspace_bytes
    need = sizer(w.B, w.H, w.T, w.dk, w.dv, w.L, prism.PRISM_BF16 if w.dtype == "bf16" else prism.PRISM_F32)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        prism.bwd(*args, L=w.L, d_o=do_t, workspace=ws, chunked=chunked)
    torch.cuda.synchronize()
    hip = Hip()
    ev = hip.events(2)
    stream = torch.cuda.current_stream()
    rec = hip.lib.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    rec(ev[0], ctypes.c_void_p(stream.cuda_stream))
    for _ in range(steps):
        prism.bwd(*args, L=w.L, d_o=do_t, workspace=ws, chunked=chunked)
    rec(ev[1], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(ev[0], ev[1]) / steps
    hip.destroy(ev)
    in_bytes, _ = algorithmic_bytes(w)
    E = 2 if w.dtype == "bf16" else 4
    grad_bytes = 4 * (2 * w.dk + w.dv + 2 + ((w.L - 1) * (w.dk + w.dv) + w.L if w.L > 1 else 0))
    per_th = in_bytes + w.dv * E + grad_bytes
    total = w.pairs * w.T * per_th
    del dev, do_t, ws
    return {"ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
            "roofline": {"bound": "hbm", "bytes_per_token_head": per_th, "bytes_per_call": total,
                         "achieved": total / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "scope": ("whole prism_bwd_chunked call (chunk operators, compose, group scans, "
                                   "expand, chunk gradients, sums)" if chunked else
                                   "whole prism_bwd call (segment-parallel: local pass, scans, token steps, sums)")},
            "form": "prism_bwd_chunked (bf16 MFMA)" if chunked else "prism_bwd (float32)"}


def time_nl(w, steps, warmup, x0=None):
    """The nonlinear-refinement forward (prism_fwd_nl: the chain-factor kernel, then the
    forward) on workload w, gains drawn by workloads.generate_gain.  Two input sets are
    rotated (with the gains they exceed the 256 MB Infinity Cache at the 16K shape).  Whole
    calls, and the factor kernel alone (prism_nl_gain), timed with HIP events on the launch
    stream; the factor kernel's roofline counts v, the gains and the step sizes read once
    and the factors written once."""
    import torch
    import delta_rule_sequence_amd as prism
    import workloads
    sets = []
    for s in range(2):
        x = dict(x0) if (s == 0 and x0 is not None) else workloads.generate(w, seed=w.seed + 100 * s)
        x.pop("gamma", None)
        x["p"] = workloads.generate_gain(w, seed=w.seed + 100 * s)
        x["W_p"] = workloads.generate_predictor(w, seed=w.seed + 100 * s)
        sets.append(workloads.to_torch(x, w.dtype, "cuda"))
    lib = prism.load_library()
    dt = prism.PRISM_BF16 if w.dtype == "bf16" else prism.PRISM_F32
    ws = torch.empty(lib.prism_fwd_nl_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.L, w.chunk, dt),
                     dtype=torch.uint8, device="cuda")
    vt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    o = torch.empty((w.B, w.H, w.T, w.dv), dtype=vt, device="cuda")
    S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")

    def fwd(d):
        prism.fwd_nl(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["p"], d["conv_w"],
                     L=w.L, chunk=w.chunk, out=(o, S), workspace=ws)

    def gain(d):
        prism.nl_gain(d["v"], d["alpha"], d["p"], d["conv_w"], w.L)

    def fwd_pred(d):
        prism.fwd_nl_pred(d["q"], d["k"], d["v"], d["g"], d["beta"], d["u"], d["alpha"], d["W_p"], d["conv_w"],
                          L=w.L, chunk=w.chunk, out=(o, S), workspace=ws)

    def gain_pred(d):
        prism.nl_gain_pred(d["v"], d["alpha"], d["W_p"], d["conv_w"], w.L)

    hip = Hip()
    stream = torch.cuda.current_stream()
    rec = hip.lib.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    res = {}
    pred = w.dtype == "bf16" and w.dv in (32, 64, 128) and w.L > 1
    fns = [("fwd_nl", fwd), ("nl_gain", gain)] + ([("fwd_nl_pred", fwd_pred), ("nl_gain_pred", gain_pred)]
                                                  if pred else [])
    for name, fn in fns:
        for i in range(warmup):
            fn(sets[i % 2])
        torch.cuda.synchronize()
        ev = hip.events(2)
        rec(ev[0], ctypes.c_void_p(stream.cuda_stream))
        for i in range(steps):
            fn(sets[i % 2])
        rec(ev[1], ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        res[name] = hip.elapsed_ms(ev[0], ev[1]) / steps
        hip.destroy(ev)
    E = 2 if w.dtype == "bf16" else 4
    per_th = E * w.dv + 2 * E * (w.L - 1) * w.dv + 4 * w.L if w.L > 1 else 0
    total = w.pairs * w.T * per_th
    gb = total / (res["nl_gain"] * 1e-3) / 1e9 if w.L > 1 else None
    # predicted gains: v and the step sizes read, the factors written (the weights stay cached)
    per_pred = E * w.dv + E * (w.L - 1) * w.dv + 4 * w.L
    total_pred = w.pairs * w.T * per_pred
    del sets, ws
    if pred:
        gp = total_pred / (res["nl_gain_pred"] * 1e-3) / 1e9
        pred_out = {"ms_per_step": res["fwd_nl_pred"], "tokens_per_s": w.B * w.T / (res["fwd_nl_pred"] * 1e-3),
                    "gain_kernel_ms": res["nl_gain_pred"],
                    "gain_roofline": {"bound": "hbm", "bytes_per_token_head": per_pred,
                                      "bytes_per_launch": total_pred, "achieved": gp, "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": gp / HBM_PEAK_GBS, "kernel": "nl_pred_gain_kernel"}}
    else:
        pred_out = None
    return {"ms_per_step": res["fwd_nl"], "tokens_per_s": w.B * w.T / (res["fwd_nl"] * 1e-3),
            "gain_kernel_ms": res["nl_gain"],
            "gain_roofline": {"bound": "hbm", "bytes_per_token_head": per_th, "bytes_per_launch": total,
                              "achieved": gb, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": None if gb is None else gb / HBM_PEAK_GBS, "kernel": "nl_gain_kernel"},
            "predicted_gains": pred_out, "steps": steps, "warmup": warmup, "input_sets": 2}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="rec16k_bf16")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0: enough to exceed the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB")
    ap.add_argument("--l-sweep", action="store_true",
                    help="time the 16K shape at L = 1, 2, 4, 8 (one JSON line each) instead")
    ap.add_argument("--decode", type=int, default=0, metavar="BATCH",
                    help="time one-token decode steps for BATCH sequences instead")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward on --workload instead")
    ap.add_argument("--bwd-form", default="auto", choices=["auto", "chunked", "float32"],
                    help="--bwd: prism_bwd_chunked (bf16 MFMA, dk = dv = 64), prism_bwd (float32), or "
                         "auto (the chunked form where it applies)")
    ap.add_argument("--nl", action="store_true",
                    help="time the nonlinear-refinement forward (prism_fwd_nl) on --workload instead")
    ap.add_argument("--forward-only", action="store_true",
                    help="the forward's line only: skip the backward, nonlinear, copy and GEMM legs "
                         "(for profiler runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the forward has no multi-GPU path "
              "(pairs and sequence segments would shard with no exchange but a small operator "
              "all-gather of the segment operators). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.l_sweep:
        l_sweep(args.steps, args.warmup)
        return
    if args.decode:
        decode_bench(args.steps, args.warmup, args.decode)
        return
    if args.bwd:
        bwd_bench(args.steps, args.warmup, args.workload, cpu=not args.no_cpu_baseline, form=args.bwd_form)
        return
    if args.nl:
        import workloads
        w = workloads.workload(args.workload)
        res = time_nl(w, args.steps, args.warmup)
        print(json.dumps({"metric": "fwd tokens/sec, nonlinear refinement (prism_fwd_nl)", "workload": w.name,
                          "dtype": w.dtype, "config": {"B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                                                       "L": w.L, "chunk": w.chunk}, **res}), flush=True)
        return

    import workloads

    w = workloads.workload(args.workload)
    x0 = workloads.generate(w, seed=w.seed)
    cpu_par = None
    if not args.no_cpu_baseline:  # forked workers: before anything touches the GPU
        print("[bench] timing the oracle on the host (one process per pair)", file=sys.stderr, flush=True)
        cpu_par = cpu_baseline_parallel(w, x0)
    t = time_workload(w, args.steps, args.warmup, args.sets, x0)
    import torch

    import numpy as np
    in_bytes, path_bytes = algorithmic_bytes(w)
    ms_per_step, per, span_ms, nsets = t["ms_per_step"], t["per"], t["span_ms"], t["nsets"]
    tokens = w.B * w.T
    sweep_ms = float(per[:, 0].mean())
    sweep_bytes = w.pairs * w.T * in_bytes + w.H * 4 * w.dv * 4
    achieved = sweep_bytes / (sweep_ms * 1e-3) / 1e9
    traffic = load_traffic(w.name)
    fast = w.dtype == "bf16" and w.dk == 64 and w.dv == 64 and w.chunk == 64
    fast128 = w.dtype == "bf16" and w.dk == 128 and w.dv == 128 and w.chunk == 64
    sweep_name = "seg_sweep8_kernel" if fast else "seg_sweep128_kernel" if fast128 else "seg_local_kernel"

    out = {
        "metric": "fwd tokens/sec at T=16K,H=4,d=64,L=4 bf16; % of HBM/MFMA roofline",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded generator; random inputs of the workload's shapes and distributions)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv, "L": w.L,
                   "chunk": w.chunk, "input_sets": nsets},
        # the dominant kernel alone (the segment sweep): its input bytes over its own event time
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "scope": "dominant kernel (segment sweep), input bytes over its event-timed duration",
                     # the counters' HBM bytes over the same duration (null with traffic)
                     "traffic_GBs": None if traffic is None else traffic / (sweep_ms * 1e-3) / 1e9,
                     "kernel": sweep_name, "algorithmic_bytes_per_launch": sweep_bytes},
        "path": {"algorithmic_bytes_per_step": w.pairs * w.T * path_bytes,
                 "hbm_roofline_tokens_per_s": tokens * HBM_PEAK_GBS * 1e9 / (w.pairs * w.T * path_bytes),
                 # the whole forward (all three kernels) against the same HBM roofline
                 "hbm_frac": (tokens / (ms_per_step * 1e-3)) / (tokens * HBM_PEAK_GBS * 1e9 /
                                                               (w.pairs * w.T * path_bytes)),
                 # per-call durations from HIP events on the launch stream (second timed region)
                 "event_ms_per_call": {"median": float(np.median(t["call_ms"])), "mean": float(t["call_ms"].mean()),
                                       "min": float(t["call_ms"].min()), "calls": int(len(t["call_ms"]))},
                 "event_median_tokens_per_s": tokens / (float(np.median(t["call_ms"])) * 1e-3),
                 "kernel_ms": {"sweep": sweep_ms, "scan": float(per[:, 1].mean()),
                               "fixup": float(per[:, 2].mean())},
                 "instrumented_ms_per_step": span_ms / args.steps},
        "cpu_baseline": None,
    }
    # secondary figure: the chunked form's MFMA work in the sweep against the dense bf16 peak
    C = w.chunk
    chunk_flop = 2 * (2 * w.L * C * w.dk + (w.L - 1) * C * w.dv + C * w.dv + C * w.dk + 2 * w.dk * w.dv
                      + w.L * C * w.dv + w.L * w.dk * w.dv)
    mfma_achieved = w.pairs * w.T * chunk_flop / (sweep_ms * 1e-3) / 1e12
    out["roofline"]["mfma_secondary"] = {"achieved": mfma_achieved, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                         "frac": mfma_achieved / MFMA_PEAK_TFLOPS,
                                         "flop_per_token_head": chunk_flop}
    if args.forward_only:
        print(json.dumps(out))
        return
    # the backward on the same workload (one warm-up, two timed calls): reported beside the
    # forward metric, not part of it
    d_o = np.random.default_rng(w.seed + 7).standard_normal((w.B, w.H, w.T, w.dv)).astype(np.float32)
    if w.dtype == "bf16":
        d_o = workloads.to_bf16_values(d_o)
    if bwd_chunked_supported(w):
        out["bwd"] = dict(time_bwd(w, x0, d_o, 5, 2, chunked=True), steps=5, warmup=2)
        out["bwd_float32"] = dict(time_bwd(w, x0, d_o, 2, 1), steps=2, warmup=1)
    else:
        out["bwd"] = dict(time_bwd(w, x0, d_o, 2, 1), steps=2, warmup=1)
    # the nonlinear-refinement forward on the same shape (its own gains), reported beside it
    out["nl"] = time_nl(w, 10, 2, x0)
    out["roofline"]["measured_copy"] = copy_bandwidth(torch)
    out["roofline"]["measured_mfma"] = mfma_rate(torch)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, x0)
        out["cpu_baseline_parallel"] = cpu_par
    print(json.dumps(out))


if __name__ == "__main__":
    main()
