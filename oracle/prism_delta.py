"""Float64 oracle of PRISM's written-correction (delta) form and of its predictor front end.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Sources, by short name (as in oracle/prism.py):
  [Notes]   "PRISM: Parallel Residual Iterative Sequence Model" reading notes,
            section 2.2 (rank accumulation: every refinement layer adds one rank-1
            term, its correction written along its own basis with its own gate) and
            section 2.3 (Input-Anchored Simulation: parallel predictors read the
            ShortConv anchor and emit each layer's gain, basis and gate through
            learned projections W_p, W_k, W_beta; the layer's correction is a GELU of
            the gain-modulated residual and is subtracted from the residual as it is,
            greedy residual subtraction, so the next layer sees what is left).
  [Summary] "ICML 2026 | PRISM", section "PRISM 设计": the first write is the GDN one.

The equations of both pages were stripped from their extracted text; the readings taken
here are listed in the design notes.  With the recurrence of oracle/prism.py (GDN
forgetting, the GDN write beta v k^T as the first rank component, readout after the
write), the written components are the corrections themselves:

  r_{t,0}     = v_t - anchor_t
  delta_{t,l} = GELU(p_{t,l-1} * r_{t,l-1}),     l = 1 .. L-1   (exact erf GELU)
  r_{t,l}     = r_{t,l-1} - delta_{t,l}                         (no step size)
  B_t         = beta_t v_t k_t^T + sum_{l=1}^{L-1} alpha_{t,l} delta_{t,l} u_{t,l}^T

alpha_{t,l} is layer l's gate; alpha_{t,0} is not read (the subtraction has no step
size).  p has gamma's layout ([B, H, T, L-1, dv], slot j holds p_{t,j}).

The front end (anchor_predict) forms, from the anchor of each token,
  p_{t,l}         = W_p[h, l] anchor_t                         l = 0 .. L-2
  u_{t,l+1}       = W_k[h, l] anchor_t / |W_k[h, l] anchor_t|  l = 0 .. L-2   (unit keys)
  alpha_{t,l}     = sigmoid(W_b[h, l] . anchor_t)              l = 0 .. L-1
with W_p [H, L-1, dv, dv], W_k [H, L-1, dk, dv] ((out, in) layouts) and W_b [H, L, dv].
Pins: tests/test_oracle_delta.py.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from .prism import shortconv_anchor
from .prism_nl import gelu

F64 = np.float64


def delta_chain(r0: np.ndarray, alpha_t: np.ndarray, p_t: np.ndarray,
                L: int) -> Tuple[List[np.ndarray], List[np.ndarray]]:
    """Greedy residual subtraction with written corrections ([Notes §2.3]).

    r0: [..., dv]; alpha_t: [..., L] gates; p_t: [..., L-1, dv] gains.
    Returns (corrections delta_{t,1..L-1}, written values alpha_{t,l} delta_{t,l}).
    """
    r = r0
    deltas, written = [], []
    for l in range(1, L):
        d = gelu(p_t[..., l - 1, :] * r)
        r = r - d
        deltas.append(d)
        written.append(alpha_t[..., l, None] * d)
    return deltas, written


def _pairs(x, hs):
    x = np.asarray(x, F64)[:, hs]
    return x.reshape((x.shape[0] * x.shape[1],) + x.shape[2:])


def forward_delta(q, k, v, g, beta, u, alpha, p, conv_w, L: int,
                  heads: Optional[List[int]] = None, S0=None, conv_in=None):
    """Token-by-token forward of the written-correction form, in the library's layout.

    Arguments as oracle.prism.forward with the gains p in place of gamma; alpha holds the
    layers' gates.  The state update (GDN forgetting, GDN first write, readout after the
    write) is the one of oracle/prism.py, written out here with dense products.
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
            _, written = delta_chain(r0, ap[:, t], pp[:, t], L)
            vals += written
            keys += [up[:, t, l] for l in range(L - 1)]
        Bt = np.einsum("pjv,pjk->pvk", np.stack(vals, 1), np.stack(keys, 1))
        Sk = np.einsum("pvk,pk->pv", S, kp[:, t])
        S = gp[:, t, None, None] * (S - bp[:, t, None, None] * Sk[:, :, None] * kp[:, t, None, :]) + Bt
        o[:, t] = np.einsum("pvk,pk->pv", S, qp[:, t])
    return (o.reshape(B, Hs, T, dv),
            np.ascontiguousarray(S.transpose(0, 2, 1)).reshape(B, Hs, dk, dv))


def delta_factors(v, p, conv_w, L: int, conv_in=None, rounding=None) -> np.ndarray:
    """Per-channel factors f with f_{t,l} * r_{t,l} = delta_{t,l+1} = GELU(p_{t,l} * r_{t,l})
    along the chain (the GELU absorbed into scaling coefficients, as the Tencent Ads
    article, section 03-三, does for the linear chain), so that the chain becomes
    r <- r - f * r with written values alpha * f * r.  Where r is exactly zero the limit
    p / 2.  Returns [B, H, T, L-1, dv], float64.

    rounding: optional element-wise map applied to each factor before the chain continues
    with it (a storage type's rounding: factors handed to a forward in that type are
    defined on the residuals that forward will see)."""
    v = np.asarray(v, F64)
    B, H, T, dv = v.shape
    p = np.asarray(p, F64)
    w = np.asarray(conv_w, F64)
    hist = np.zeros((B, H, 3, dv), F64) if conv_in is None else np.asarray(conv_in, F64)
    v_ext = np.concatenate([hist, v], axis=2)
    fac = np.zeros((B, H, T, max(L - 1, 0), dv), F64)
    for t in range(T):
        r = v[:, :, t] - shortconv_anchor(v_ext, w[None], t + 3)
        for l in range(1, L):
            z = gelu(p[:, :, t, l - 1] * r)
            safe = np.where(r == 0.0, 1.0, r)
            f = np.where(r == 0.0, 0.5 * p[:, :, t, l - 1], z / safe)
            if rounding is not None:
                f = np.asarray(rounding(f), F64)
            fac[:, :, t, l - 1] = f
            r = r - f * r
    return fac


def forward_delta_factors(q, k, v, g, beta, u, alpha, fac, conv_w, L: int, heads=None):
    """The written-correction forward with the corrections given as factors of the
    residual (r <- r - f r, written alpha f r): the form the kernels run once the factors
    are formed.  Token by token, float64; arguments as forward_delta with fac in place of
    p.  Returns o [B, H', T, dv] and S_final [B, H', dk, dv]."""
    B, H, T, dk = np.asarray(q).shape
    dv = np.asarray(v).shape[-1]
    hs = list(range(H)) if heads is None else list(heads)
    Hs = len(hs)
    qp, kp, vp = _pairs(q, hs), _pairs(k, hs), _pairs(v, hs)
    gp, bp = _pairs(g, hs), _pairs(beta, hs)
    P = B * Hs
    w = np.broadcast_to(np.asarray(conv_w, F64)[hs][None], (B, Hs, 4, dv)).reshape(P, 4, dv)
    if L > 1:
        up, ap, fp = _pairs(u, hs), _pairs(alpha, hs), _pairs(fac, hs)
    S = np.zeros((P, dv, dk), F64)
    v_ext = np.concatenate([np.zeros((P, 3, dv), F64), vp], axis=1)
    o = np.empty((P, T, dv), F64)
    for t in range(T):
        vals = [bp[:, t, None] * vp[:, t]]
        keys = [kp[:, t]]
        if L > 1:
            r = vp[:, t] - shortconv_anchor(v_ext, w, t + 3)
            for l in range(1, L):
                d = fp[:, t, l - 1] * r
                r = r - d
                vals.append(ap[:, t, l, None] * d)
                keys.append(up[:, t, l - 1])
        Bt = np.einsum("pjv,pjk->pvk", np.stack(vals, 1), np.stack(keys, 1))
        Sk = np.einsum("pvk,pk->pv", S, kp[:, t])
        S = gp[:, t, None, None] * (S - bp[:, t, None, None] * Sk[:, :, None] * kp[:, t, None, :]) + Bt
        o[:, t] = np.einsum("pvk,pk->pv", S, qp[:, t])
    return (o.reshape(B, Hs, T, dv),
            np.ascontiguousarray(S.transpose(0, 2, 1)).reshape(B, Hs, dk, dv))


def anchor_predict(v, conv_w, W_p, W_k, W_b, L: int, conv_in=None, anchor_rounding=None):
    """The predictor front end ([Notes §2.3]): gains, unit keys and gates from the anchor.

    v: [B, H, T, dv]; conv_w: [H, 4, dv]; W_p: [H, L-1, dv, dv]; W_k: [H, L-1, dk, dv];
    W_b: [H, L, dv]; conv_in: optional [B, H, 3, dv].
    Returns p [B, H, T, L-1, dv], u [B, H, T, L-1, dk], alpha [B, H, T, L], float64.
    anchor_rounding: optional element-wise map applied to the anchor before the
    projections (a storage type for the projections' operand).
    """
    v = np.asarray(v, F64)
    B, H, T, dv = v.shape
    Wp, Wk, Wb = (np.asarray(W_p, F64), np.asarray(W_k, F64), np.asarray(W_b, F64))
    dk = Wk.shape[2]
    w = np.asarray(conv_w, F64)
    hist = np.zeros((B, H, 3, dv), F64) if conv_in is None else np.asarray(conv_in, F64)
    v_ext = np.concatenate([hist, v], axis=2)
    p = np.zeros((B, H, T, L - 1, dv), F64)
    u = np.zeros((B, H, T, L - 1, dk), F64)
    alpha = np.zeros((B, H, T, L), F64)
    for t in range(T):
        anc = shortconv_anchor(v_ext, w[None], t + 3)                  # [B, H, dv]
        if anchor_rounding is not None:
            anc = np.asarray(anchor_rounding(anc), F64)
        for l in range(L - 1):
            p[:, :, t, l] = np.einsum("hoi,bhi->bho", Wp[:, l], anc)
            key = np.einsum("hoi,bhi->bho", Wk[:, l], anc)
            u[:, :, t, l] = key / np.sqrt(np.sum(key * key, axis=-1, keepdims=True))
        for l in range(L):
            alpha[:, :, t, l] = 1.0 / (1.0 + np.exp(-np.einsum("hi,bhi->bh", Wb[:, l], anc)))
    return p, u, alpha
