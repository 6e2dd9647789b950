"""Float64 oracle of PRISM's nonlinear residual refinement (the GELU write).

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Sources, by short name (as in oracle/prism.py):
  [Notes]   "PRISM: Parallel Residual Iterative Sequence Model" reading notes,
            section 2.3: each refinement layer forms a correction by passing the
            gain-modulated residual p ⊙ r through a GELU and subtracts it from the
            residual (greedy residual subtraction), so the next layer sees what is
            left; the gain p comes from a predictor on the anchor.
  [Article] Tencent Ads / Peking University article on PRISM, section 03-三: the
            GELU inside the iteration is absorbed into precomputed scaling
            coefficients (a preconditioner), which leaves a purely element-wise
            linear recursion.

The linearised chain of oracle/prism.py subtracts alpha_{l-1} gamma_{l-1} ⊙ r from
r at step l.  Here the term gamma_{l-1} ⊙ r is the GELU correction itself:

  r_{t,0} = v_t - anchor_t
  r_{t,l} = r_{t,l-1} - alpha_{t,l-1} GELU(p_{t,l-1} ⊙ r_{t,l-1}),  l = 1 .. L-1
  written values alpha_{t,l} r_{t,l}; the rest of the recurrence is unchanged.

GELU is the exact (erf) form.  p has the layout of gamma ([B, H, T, L-1, dv],
slot j holds p_{t,j}).  `preconditioner` returns the per-token, per-channel
factors that make the linear chain reproduce this one exactly: the "absorbed"
coefficients of [Article §03-三].  Pins: tests/test_oracle_nl.py.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np
from scipy.special import erf

from .prism import shortconv_anchor

F64 = np.float64


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU, x times the standard normal CDF of x."""
    x = np.asarray(x, F64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def nonlinear_chain(r0: np.ndarray, alpha_t: np.ndarray, p_t: np.ndarray,
                    L: int) -> Tuple[List[np.ndarray], List[np.ndarray]]:
    """Greedy residual subtraction with the GELU correction ([Notes §2.3]).

    r0: [..., dv]; alpha_t: [..., L]; p_t: [..., L-1, dv].
    Returns (residuals r_{t,1..L-1}, written values alpha_{t,l} r_{t,l}).
    """
    r = r0
    residuals, written = [], []
    for l in range(1, L):
        delta = gelu(p_t[..., l - 1, :] * r)
        r = r - alpha_t[..., l - 1, None] * delta
        residuals.append(r)
        written.append(alpha_t[..., l, None] * r)
    return residuals, written


def _pairs(x, hs):
    x = np.asarray(x, F64)[:, hs]
    return x.reshape((x.shape[0] * x.shape[1],) + x.shape[2:])


def forward_nl(q, k, v, g, beta, u, alpha, p, conv_w, L: int,
               heads: Optional[List[int]] = None, S0=None, conv_in=None):
    """Token-by-token forward with the nonlinear chain, in the library's layout.

    Arguments as oracle.prism.forward, with p in place of gamma.  The state
    update is the one of oracle/prism.py (GDN forgetting, rank-L write,
    readout after the write), written out again here with dense products.
    Returns o [B, H', T, dv] and S_final [B, H', dk, dv], float64.
    """
    B, H, T, dk = np.asarray(q).shape
    dv = np.asarray(v).shape[-1]
    hs = list(range(H)) if heads is None else list(heads)
    Hs = len(hs)
    qp, kp, vp = _pairs(q, hs), _pairs(k, hs), _pairs(v, hs)
    gp, bp = _pairs(g, hs), _pairs(beta, hs)
    P = B * Hs
    w = np.broadcast_to(np.asarray(conv_w, F64)[hs][None], (B, Hs, 4, dv)).reshape(P, 4, dv)
    if L > 1:
        up, ap, pp = _pairs(u, hs), _pairs(alpha, hs), _pairs(p, hs)
    S = (np.zeros((P, dv, dk), F64) if S0 is None
         else _pairs(S0, hs).transpose(0, 2, 1).copy())
    hist = np.zeros((P, 3, dv), F64) if conv_in is None else _pairs(conv_in, hs)
    v_ext = np.concatenate([hist, vp], axis=1)
    o = np.empty((P, T, dv), F64)
    for t in range(T):
        vals = [bp[:, t, None] * vp[:, t]]
        keys = [kp[:, t]]
        if L > 1:
            r0 = vp[:, t] - shortconv_anchor(v_ext, w, t + 3)
            _, written = nonlinear_chain(r0, ap[:, t], pp[:, t], L)
            vals += written
            keys += [up[:, t, l] for l in range(L - 1)]
        Bt = np.einsum("pjv,pjk->pvk", np.stack(vals, 1), np.stack(keys, 1))
        Sk = np.einsum("pvk,pk->pv", S, kp[:, t])
        S = gp[:, t, None, None] * (S - bp[:, t, None, None] * Sk[:, :, None] * kp[:, t, None, :]) + Bt
        o[:, t] = np.einsum("pvk,pk->pv", S, qp[:, t])
    return (o.reshape(B, Hs, T, dv),
            np.ascontiguousarray(S.transpose(0, 2, 1)).reshape(B, Hs, dk, dv))


def preconditioner(v, alpha, p, conv_w, L: int, conv_in=None) -> np.ndarray:
    """The factors gamma with gamma_{t,l} ⊙ r_{t,l} = GELU(p_{t,l} ⊙ r_{t,l}) along
    the nonlinear chain ([Article §03-三]: the GELU absorbed into scaling
    coefficients), so that the linear chain run with them is the nonlinear one.

    Defined as GELU(p r) / r; where r is exactly zero the limit p / 2.
    v: [B, H, T, dv]; alpha: [B, H, T, L]; p: [B, H, T, L-1, dv]; conv_w: [H, 4, dv];
    conv_in: optional [B, H, 3, dv].  Returns gamma [B, H, T, L-1, dv], float64.
    """
    v = np.asarray(v, F64)
    B, H, T, dv = v.shape
    alpha = np.asarray(alpha, F64)
    p = np.asarray(p, F64)
    w = np.asarray(conv_w, F64)
    hist = np.zeros((B, H, 3, dv), F64) if conv_in is None else np.asarray(conv_in, F64)
    v_ext = np.concatenate([hist, v], axis=2)
    gam = np.zeros((B, H, T, max(L - 1, 0), dv), F64)
    for t in range(T):
        r = v[:, :, t] - shortconv_anchor(v_ext, w[None], t + 3)
        for l in range(1, L):
            z = gelu(p[:, :, t, l - 1] * r)
            safe = np.where(r == 0.0, 1.0, r)
            gam[:, :, t, l - 1] = np.where(r == 0.0, 0.5 * p[:, :, t, l - 1], z / safe)
            r = r - alpha[:, :, t, l - 1, None] * z
    return gam


def predictor_gains(v, conv_w, W_p, L: int, conv_in=None) -> np.ndarray:
    """Gains produced by a linear predictor on the anchor ([Notes §2.3]: parallel
    predictors read the ShortConv anchor and emit each layer's gain vector):
    p_{t,l} = W_p[h, l] anchor_t, with W_p [H, L-1, dv, dv] in the (out, in) layout.

    v: [B, H, T, dv]; conv_w: [H, 4, dv]; conv_in: optional [B, H, 3, dv].
    Returns p [B, H, T, L-1, dv], float64.
    """
    v = np.asarray(v, F64)
    B, H, T, dv = v.shape
    W = np.asarray(W_p, F64)
    w = np.asarray(conv_w, F64)
    hist = np.zeros((B, H, 3, dv), F64) if conv_in is None else np.asarray(conv_in, F64)
    v_ext = np.concatenate([hist, v], axis=2)
    p = np.zeros((B, H, T, max(L - 1, 0), dv), F64)
    for t in range(T):
        anchor = shortconv_anchor(v_ext, w[None], t + 3)          # [B, H, dv]
        for l in range(L - 1):
            p[:, :, t, l] = np.einsum("hoi,bhi->bho", W[:, l], anchor)
    return p
