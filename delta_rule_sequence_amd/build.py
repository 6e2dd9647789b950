"""Build libprism.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m delta_rule_sequence_amd.build

Compiles every .hip source under csrc/ into one shared library next to this
file.  Uses hipcc from ROCm; no GPU is needed to build.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libprism.so")
ARCH = os.environ.get("PRISM_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in [shutil.which("hipcc"), "/opt/rocm/bin/hipcc"]:
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")


def build(verbose: bool = False) -> str:
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-I", INCLUDE, "-I", CSRC,
           # packed fp32 VALU ops are kept out of every kernel
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # the latency-bound kernels (scan, sweep phases) gain from the ILP-first
           # machine scheduler (measured: scan 19.0 -> 17.1 us at the 16K workload)
           "-mllvm", "-amdgpu-sched-strategy=max-ilp",
           *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
