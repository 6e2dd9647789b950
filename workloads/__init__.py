"""Seeded synthetic inputs for the PRISM rank-L gated delta-rule forward.

This module is shared by the tests, the benchmark and the smoke check.  It
holds the workload shapes and the input recipe only: no step of the method
(anchor, residual chain, recurrence, readout) is computed here.

Input recipe (one ``numpy.random.default_rng(seed)`` stream, drawn in this
order, then L2-normalisation and the cast to the I/O dtype):

1. q, k, v ~ N(0, 1), each [B, H, T, d]                (drawn q, then k, then v)
2. x ~ U(lo, hi) [B, H, T];  g = exp(-x)                (the scalar decay gate)
3. beta = sigmoid(N(0, 1)) [B, H, T]
4. conv_w ~ N(0, 0.5) [H, 4, dv]  (0.5 is the standard deviation)
5. if L > 1:  u ~ N(0, 1) [B, H, T, L-1, dk];
              alpha = 0.5 * sigmoid(N(0, 1)) [B, H, T, L];
              z ~ N(0, 1) [B, H, T, L-1, dv];  gamma = GELU'(z) (exact erf GELU)

q and k are normalised over dk per (b, h, t), u over dk per (b, h, t, l), in
float64, before the cast.  Vectors (q, k, v, u, gamma) are cast to the I/O
dtype: float32 (round to nearest even from float64), or bfloat16 taken as
RNE(float32 RNE(x)).  The scalars g, beta, alpha and the conv weights are
float32 in both paths.

The shapes and value ranges stand in for the pages' workloads: the 16K-long
behaviour sequences of the sequential-recommendation throughput table
(ai-engineering page, experiments table) and a 130M-parameter language-model
layer (Tencent Ads article, section 04-2).  No dataset is read.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional

import numpy as np
from scipy.special import ndtr

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "to_bf16_values",
           "manifest"]


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


def _cast_vec(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return to_bf16_values(x32)
    raise ValueError(dtype)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _gelu_prime(z: np.ndarray) -> np.ndarray:
    # derivative of the exact GELU z * Phi(z):  Phi(z) + z * phi(z)
    return ndtr(z) + z * np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


def _normal_block(rng, shape, block_axis0_rows: int = 1 << 22):
    """Standard normals of `shape` drawn as one stream (identical to one call)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, block_axis0_rows):
        e = min(n, s + block_axis0_rows)
        out[s:e] = rng.standard_normal(e - s)
    return out.reshape(shape)


def generate(w: Workload, seed: Optional[int] = None, keys: str = "iid") -> Dict[str, np.ndarray]:
    """Draw the inputs of workload `w`.

    Returns float32 arrays (bf16-representable values for bf16 workloads):
    q, k [B,H,T,dk]; v [B,H,T,dv]; g, beta [B,H,T]; conv_w [H,4,dv];
    and for L > 1 also u [B,H,T,L-1,dk], alpha [B,H,T,L], gamma [B,H,T,L-1,dv]
    (None for L == 1).

    keys="correlated" replaces k by one of 8 base directions per token plus
    small noise (a stress case for the intra-chunk triangular solve; it is drawn
    after everything else so the other tensors are unchanged).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, H, T, dk, dv, L = w.B, w.H, w.T, w.dk, w.dv, w.L
    q = _normal_block(rng, (B, H, T, dk))
    k = _normal_block(rng, (B, H, T, dk))
    v = _normal_block(rng, (B, H, T, dv))
    x = rng.uniform(w.x_lo, w.x_hi, size=(B, H, T))
    g = np.exp(-x)
    beta = _sigmoid(rng.standard_normal((B, H, T)))
    conv_w = rng.normal(0.0, 0.5, size=(H, 4, dv))
    u = alpha = gamma = None
    if L > 1:
        u = _normal_block(rng, (B, H, T, L - 1, dk))
        alpha = 0.5 * _sigmoid(rng.standard_normal((B, H, T, L)))
        z = _normal_block(rng, (B, H, T, L - 1, dv))
        gamma = _gelu_prime(z)
        del z
    if keys == "correlated":
        base = rng.standard_normal((8, dk))
        idx = rng.integers(0, 8, size=(B, H, T))
        k = base[idx] + 0.05 * rng.standard_normal((B, H, T, dk))
    elif keys != "iid":
        raise ValueError(keys)
    out = {
        "q": _cast_vec(_l2_normalise(q), w.dtype),
        "k": _cast_vec(_l2_normalise(k), w.dtype),
        "v": _cast_vec(v, w.dtype),
        "g": g.astype(np.float32),
        "beta": beta.astype(np.float32),
        "conv_w": conv_w.astype(np.float32),
        "u": None if u is None else _cast_vec(_l2_normalise(u), w.dtype),
        "alpha": None if alpha is None else alpha.astype(np.float32),
        "gamma": None if gamma is None else _cast_vec(gamma, w.dtype),
    }
    return out


def manifest(inputs: Dict[str, np.ndarray]) -> Dict[str, str]:
    """SHA-256 of every tensor's bytes (generator determinism check)."""
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
            for k, v in sorted(inputs.items()) if v is not None}
