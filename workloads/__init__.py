"""Seeded synthetic inputs for the PRISM rank-L gated delta-rule forward.

This module is shared by the tests, the benchmark and the smoke check.  It
holds the workload shapes and the input recipe only: no step of the method
(anchor, residual chain, recurrence, readout) is computed here.

Input recipe (seed = the workload's seed):

* Large vector tensors are filled block by block (BLOCK_ROWS rows of the last
  axis per block).  Block j of tensor i (q=0, k=1, v=2, u=3, z=4) is drawn from
  its own generator numpy.random.Generator(PCG64(SeedSequence([seed, i, j]))) as
  float32 standard normals.  Blocks are independent, so they are filled in
  parallel threads and the result does not depend on the thread count.
* Small tensors come from one numpy.random.default_rng(seed) stream, in order:
  x ~ U(lo, hi) [B, H, T] with g = exp(-x) (the scalar decay gate);
  beta = sigmoid(N(0, 1)) [B, H, T]; conv_w ~ N(0, 0.5) [H, 4, dv] (0.5 is the
  standard deviation); and, if L > 1, alpha = 0.5 * sigmoid(N(0, 1)) [B, H, T, L].
* q, k ~ N(0, 1) [B, H, T, dk] and u ~ N(0, 1) [B, H, T, L-1, dk] are
  L2-normalised over dk per row; v ~ N(0, 1) [B, H, T, dv];
  gamma = GELU'(z) = Phi(z) + z phi(z) with z ~ N(0, 1) [B, H, T, L-1, dv]
  (derivative of the exact erf GELU).
* For the nonlinear-refinement variant only (generate_gain): the gains
  p ~ N(0, 1) [B, H, T, L-1, dv], tensor id 5, in the I/O dtype.  The pages give
  no statistics for the predicted gains; unit normals put p * r across the
  GELU's curved range.  For the predicted gains instead (generate_predictor): weights
  W_p ~ N(0, 1/dv) [H, L-1, dv, dv] from default_rng(seed + 2000), in the I/O dtype.
* Vectors (q, k, v, u, gamma) are stored in the I/O dtype: float32, or
  bfloat16 values (round to nearest even of the float32 value).  The scalars g,
  beta, alpha and the conv weights are float32 in both paths.

The shapes and value ranges stand in for the pages' workloads: the 16K-long
behaviour sequences of the sequential-recommendation throughput table
(ai-engineering page, experiments table) and a 130M-parameter language-model
layer (Tencent Ads article, section 04-2).  No dataset is read.
"""
from __future__ import annotations

import dataclasses
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
from scipy.special import ndtr

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "generate_gain", "generate_predictor",
           "generate_front", "generate_state", "to_bf16_values", "manifest"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": storage type of q, k, v, u, gamma and o
    B: int
    H: int
    T: int
    dk: int
    dv: int
    L: int
    chunk: int
    x_lo: float = 0.001
    x_hi: float = 0.1
    seed: int = 0

    @property
    def pairs(self) -> int:
        return self.B * self.H

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: tiny GDN-only fp32, small rank-L fp32, the 16K
# recommendation-length sequence (the measured one), a 130M-scale LM layer
# and a 64K single sequence with a deep chain.
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_gdn_f32", "f32", B=1, H=1, T=64, dk=16, dv=16, L=1, chunk=16, seed=0),
        Workload("small_rankL_f32", "f32", B=2, H=2, T=512, dk=32, dv=32, L=3, chunk=32, seed=1),
        Workload("rec16k_bf16", "bf16", B=2, H=4, T=16384, dk=64, dv=64, L=4, chunk=64, seed=2),
        Workload("lm130m_bf16", "bf16", B=8, H=6, T=2048, dk=128, dv=128, L=4, chunk=64,
                 x_lo=0.0005, x_hi=0.05, seed=3),
        Workload("long64k_bf16", "bf16", B=1, H=8, T=65536, dk=128, dv=128, L=8, chunk=64, seed=4),
    ]
}

ORDER = list(WORKLOADS)


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[ORDER[name_or_index]]
    return WORKLOADS[name_or_index]


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (RNE on the float32 bit pattern); returns float32 arrays
    whose values are exactly representable in bfloat16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32)
    rounded = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def _cast_vec(x: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return to_bf16_values(x32)
    raise ValueError(dtype)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    x64 = np.asarray(x, dtype=np.float64)
    return x64 / np.sqrt(np.sum(x64 * x64, axis=-1, keepdims=True))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _gelu_prime(z: np.ndarray) -> np.ndarray:
    # derivative of the exact GELU z * Phi(z):  Phi(z) + z * phi(z)
    return ndtr(z) + z * np.exp(-0.5 * z * z) * np.float32(1.0 / np.sqrt(2.0 * np.pi))


BLOCK_ROWS = 8192
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _fill_rows(seed: int, tensor_id: int, shape, dtype: str, post) -> np.ndarray:
    """Fill a [..., d] tensor block by block: float32 normals from a generator
    keyed by (seed, tensor_id, block), then `post` (per-row transform), then the
    cast to the I/O dtype."""
    d = shape[-1]
    rows = int(np.prod(shape[:-1]))
    out = np.empty((rows, d), dtype=np.float32)

    def work(j):
        r0 = j * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, j])))
        x = gen.standard_normal((r1 - r0, d), dtype=np.float32)
        if post is not None:
            x = post(x)
        out[r0:r1] = _cast_vec(x, dtype)

    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    if nblk == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(nblk)))
    return out.reshape(shape)


def generate(w: Workload, seed: Optional[int] = None, keys: str = "iid") -> Dict[str, np.ndarray]:
    """Draw the inputs of workload `w`.

    Returns float32 arrays (bf16-representable values for bf16 workloads):
    q, k [B,H,T,dk]; v [B,H,T,dv]; g, beta [B,H,T]; conv_w [H,4,dv];
    and for L > 1 also u [B,H,T,L-1,dk], alpha [B,H,T,L], gamma [B,H,T,L-1,dv]
    (None for L == 1).

    keys="correlated" replaces k by one of 8 base directions per token plus
    small noise (a stress case for the intra-chunk triangular solve); the other
    tensors are unchanged.
    """
    seed = w.seed if seed is None else seed
    B, H, T, dk, dv, L = w.B, w.H, w.T, w.dk, w.dv, w.L
    rng = np.random.default_rng(seed)
    x = rng.uniform(w.x_lo, w.x_hi, size=(B, H, T))
    g = np.exp(-x)
    beta = _sigmoid(rng.standard_normal((B, H, T)))
    conv_w = rng.normal(0.0, 0.5, size=(H, 4, dv))
    alpha = 0.5 * _sigmoid(rng.standard_normal((B, H, T, L))) if L > 1 else None
    out = {
        "q": _fill_rows(seed, 0, (B, H, T, dk), w.dtype, _l2_normalise),
        "k": _fill_rows(seed, 1, (B, H, T, dk), w.dtype, _l2_normalise),
        "v": _fill_rows(seed, 2, (B, H, T, dv), w.dtype, None),
        "g": g.astype(np.float32),
        "beta": beta.astype(np.float32),
        "conv_w": conv_w.astype(np.float32),
        "u": None, "alpha": None, "gamma": None,
    }
    if L > 1:
        out["u"] = _fill_rows(seed, 3, (B, H, T, L - 1, dk), w.dtype, _l2_normalise)
        out["alpha"] = alpha.astype(np.float32)
        out["gamma"] = _fill_rows(seed, 4, (B, H, T, L - 1, dv), w.dtype, _gelu_prime)
    if keys == "correlated":
        crng = np.random.default_rng([seed, 99])
        base = crng.standard_normal((8, dk))
        idx = crng.integers(0, 8, size=(B, H, T))
        kk = base[idx] + 0.05 * crng.standard_normal((B, H, T, dk))
        out["k"] = _cast_vec(_l2_normalise(kk), w.dtype)
    elif keys != "iid":
        raise ValueError(keys)
    return out


def generate_gain(w: Workload, seed: Optional[int] = None) -> Optional[np.ndarray]:
    """Gains p [B, H, T, L-1, dv] of the nonlinear refinement (None for L = 1)."""
    if w.L == 1:
        return None
    seed = w.seed if seed is None else seed
    return _fill_rows(seed, 5, (w.B, w.H, w.T, w.L - 1, w.dv), w.dtype, None)


def generate_predictor(w: Workload, seed: Optional[int] = None) -> Optional[np.ndarray]:
    """Weights W_p [H, L-1, dv, dv] ((out, in) layout, I/O dtype) of a linear gain predictor
    on the anchor, N(0, 1/dv) entries (a random initialisation: the gains then have about
    the anchor's scale).  None for L = 1."""
    if w.L == 1:
        return None
    seed = (w.seed if seed is None else seed) + 2000
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((w.H, w.L - 1, w.dv, w.dv)) / np.sqrt(w.dv)
    return _cast_vec(W, w.dtype)


def generate_front(w: Workload, seed: Optional[int] = None) -> Optional[Dict[str, np.ndarray]]:
    """Weights of the predictor front end of the written-correction form: W_p [H, L-1, dv, dv],
    W_k [H, L-1, dk, dv] ((out, in) layouts) and W_b [H, L, dv], N(0, 1/dv) entries from
    default_rng(seed + 3000) in that order (a random initialisation: gains of about the
    anchor's scale, gate logits of about unit scale), in the I/O dtype.  None for L = 1."""
    if w.L == 1:
        return None
    seed = (w.seed if seed is None else seed) + 3000
    rng = np.random.default_rng(seed)
    sc = 1.0 / np.sqrt(w.dv)
    Wp = rng.standard_normal((w.H, w.L - 1, w.dv, w.dv)) * sc
    Wk = rng.standard_normal((w.H, w.L - 1, w.dk, w.dv)) * sc
    Wb = rng.standard_normal((w.H, w.L, w.dv)) * sc
    return {"W_p": _cast_vec(Wp, w.dtype), "W_k": _cast_vec(Wk, w.dtype), "W_b": _cast_vec(Wb, w.dtype)}


def generate_state(w: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """A starting point for a continued sequence of workload `w`: S0 [B,H,dk,dv] float32
    with N(0, 0.3^2) entries (the S_final layout) and conv_in [B,H,3,dv], values of the
    three earlier tokens drawn like v (N(0,1), representable in the I/O dtype)."""
    seed = (w.seed if seed is None else seed) + 1000
    rng = np.random.default_rng(seed)
    S0 = (0.3 * rng.standard_normal((w.B, w.H, w.dk, w.dv))).astype(np.float32)
    conv_in = _cast_vec(rng.standard_normal((w.B, w.H, 3, w.dv)), w.dtype)
    return {"S0": S0, "conv_in": conv_in}


def manifest(inputs: Dict[str, np.ndarray]) -> Dict[str, str]:
    """SHA-256 of every tensor's bytes (generator determinism check)."""
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
            for k, v in sorted(inputs.items()) if v is not None}


def to_torch(inputs: Dict[str, np.ndarray], dtype: str, device="cuda"):
    """Copy generated inputs to `device`: vectors in the I/O dtype (exact, the
    values are already representable), scalars and conv weights in float32."""
    import torch
    vt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for key, val in inputs.items():
        if val is None:
            out[key] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(val))
        if key in ("q", "k", "v", "u", "gamma", "conv_in", "p", "W_p", "W_k", "W_b"):
            t = t.to(device=device).to(vt)
        else:
            t = t.to(device=device, dtype=torch.float32)
        out[key] = t.contiguous()
    return out
