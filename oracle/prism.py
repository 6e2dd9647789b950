"""Float64 token-by-token oracle of the PRISM rank-L gated delta-rule forward.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Sources, by short name:
  [Notes]   "PRISM: Parallel Residual Iterative Sequence Model" reading notes
            (liuzhao09.github.io/papers/prism.html), sections 2.1-2.4.
  [Summary] "ICML 2026 | PRISM: Parallel Residual Iterative Sequence Model"
            (ai-engineering-6yk.pages.dev), sections "PRISM 设计" and
            "架构全貌".
  [Article] Tencent Ads / Peking University article on PRISM ("当线性注意力学会
            「写入前思考」", youzy.cn), sections 01-二, 01-四 and 03-一..四.

The pages print the structure but their equations were stripped, so the
concrete form is the one the task fixes (and the pages outline):

  S_t = S_{t-1} A_t + B_t,            S_0 = 0 (or a given state), S is dv x dk
  A_t = g_t (I - beta_t k_t k_t^T)                       GDN forgetting
  B_t = beta_t v_t k_t^T + sum_{l=1}^{L-1} (alpha_{t,l} r_{t,l}) u_{t,l}^T
  anchor_t = sum_{j=0}^{3} w_j * v_{t-3+j}   (zero where t-3+j < 0, unless the
                                              values of those tokens are given)
  r_{t,0} = v_t - anchor_t
  r_{t,l} = r_{t,l-1} - alpha_{t,l-1} gamma_{t,l-1} * r_{t,l-1}
  o_t = S_t q_t

Parity pins for every function here live in tests/test_oracle_pins.py.  The
conventions that no page fixes (conv tap order, conv weights per head, the
readout after the write, the slot layout of u/alpha/gamma) are pinned only by
this module and the kernel agreeing.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

F64 = np.float64


def shortconv_anchor(v: np.ndarray, w: np.ndarray, t: int) -> np.ndarray:
    """Depthwise causal ShortConv of window 4 over the value history at token t.

    v: [..., T, dv] value rows; w: [..., 4, dv] taps (tap j multiplies
    v_{t-3+j}); rows before the sequence start count as zero.
    [Notes §2.3]: the anchor is a short convolution over the input prefix,
    used in place of the state-dependent read S_{t-1} k_t.  Window 4 is the
    upper end of the "3-4 tokens" window in [Article §05-一] / [Summary,
    混合架构是必然].
    """
    acc = np.zeros(v.shape[:-2] + v.shape[-1:], dtype=F64)
    for j in range(4):
        s = t - 3 + j
        if s >= 0:
            acc = acc + w[..., j, :] * v[..., s, :]
    return acc


def residual_chain(r0: np.ndarray, alpha_t: np.ndarray, gamma_t: np.ndarray,
                   L: int) -> Tuple[List[np.ndarray], List[np.ndarray]]:
    """Run the linearised residual chain one refinement step at a time.

    r0: [..., dv] initial residual v_t - anchor_t ([Notes §2.3]: the first
    residual is the value minus the input-anchored proxy).
    alpha_t: [..., L] step sizes; gamma_t: [..., L-1, dv] preconditioners (the
    GELU gain absorbed into a fixed per-channel factor, [Article §03-三],
    [Summary, 消除 Step 间串行]).
    Each step subtracts the step-scaled, gain-scaled residual from itself
    ([Notes §2.3], greedy residual subtraction r^{(l+1)} = r^{(l)} - delta^{(l)}).
    Returns (residuals r_{t,1..L-1}, written values alpha_{t,l} r_{t,l}).
    """
    r = r0
    residuals, written = [], []
    for l in range(1, L):
        r = r - alpha_t[..., l - 1, None] * gamma_t[..., l - 1, :] * r
        residuals.append(r)
        written.append(alpha_t[..., l, None] * r)
    return residuals, written


def token_step(S: np.ndarray, q_t, k_t, v_t, g_t, beta_t, anchor_t,
               u_t: Optional[np.ndarray], alpha_t: Optional[np.ndarray],
               gamma_t: Optional[np.ndarray], L: int):
    """One token of the recurrence for a batch of (b, h) pairs.

    S: [P, dv, dk]; q_t, k_t: [P, dk]; v_t, anchor_t: [P, dv]; g_t, beta_t: [P];
    u_t: [P, L-1, dk]; alpha_t: [P, L]; gamma_t: [P, L-1, dv].
    Returns (S_t, o_t).

    Forgetting, [Article §01-四] and [Notes §2.2]: a scalar gate decays the
    whole state and a rank-1 term selectively forgets along k_t:
        S_{t-1} A_t = g_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T).
    Writing, [Notes §2.2] rank accumulation and [Summary, 架构全貌]
    (Delta S = Delta S_gdn + Delta S_residual): the GDN write beta_t v_t k_t^T
    plus one rank-1 term per refinement step.  The decay does not touch B_t.
    Readout: o_t = S_t q_t, after token t's own write.
    """
    vals = [beta_t[:, None] * v_t]
    keys = [k_t]
    if L > 1:
        _, written = residual_chain(v_t - anchor_t, alpha_t, gamma_t, L)
        for l in range(1, L):
            vals.append(written[l - 1])
            keys.append(u_t[:, l - 1, :])
    Vf = np.stack(vals, axis=2)            # [P, dv, L]  value factors
    Kf = np.stack(keys, axis=1)            # [P, L, dk]  key factors
    B_t = np.matmul(Vf, Kf)                # [P, dv, dk] = sum_j val_j key_j^T
    Sk = np.matmul(S, k_t[:, :, None])[:, :, 0]                     # S_{t-1} k_t
    SA = g_t[:, None, None] * (S - beta_t[:, None, None] * Sk[:, :, None] * k_t[:, None, :])
    S_new = SA + B_t
    o_t = np.matmul(S_new, q_t[:, :, None])[:, :, 0]
    return S_new, o_t


def forward_pairs(q, k, v, g, beta, u, alpha, gamma, w, L: int,
                  S0: Optional[np.ndarray] = None, v_hist: Optional[np.ndarray] = None):
    """Oracle over P independent (b, h) pairs.

    q, k: [P, T, dk]; v: [P, T, dv]; g, beta: [P, T]; u: [P, T, L-1, dk];
    alpha: [P, T, L]; gamma: [P, T, L-1, dv]; w: [P, 4, dv] (each pair's
    head's conv taps).  Returns o [P, T, dv] and S_T [P, dv, dk], float64.

    S0: optional starting state [P, dv, dk] (zero when None).  v_hist: optional
    value rows [P, 3, dv] of the tokens just before the sequence (t = -3, -2,
    -1) for the ShortConv window (zero when None).  Resuming a sequence from
    its previous state and last three values continues the same recurrence:
    the fixed-size state is all a linear recurrence carries forward
    ([Article §01-二]), and the anchor only looks back over its window.
    """
    q = np.asarray(q, F64); k = np.asarray(k, F64); v = np.asarray(v, F64)
    g = np.asarray(g, F64); beta = np.asarray(beta, F64); w = np.asarray(w, F64)
    if L > 1:
        u = np.asarray(u, F64); alpha = np.asarray(alpha, F64); gamma = np.asarray(gamma, F64)
    P, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((P, dv, dk), dtype=F64) if S0 is None else np.array(S0, dtype=F64)
    o = np.empty((P, T, dv), dtype=F64)
    # the value rows the anchor reads: the history (or zeros) followed by the sequence
    hist = np.zeros((P, 3, dv), dtype=F64) if v_hist is None else np.asarray(v_hist, F64)
    v_ext = np.concatenate([hist, v], axis=1)
    for t in range(T):
        anchor = shortconv_anchor(v_ext, w, t + 3)
        S, o[:, t] = token_step(
            S, q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], anchor,
            u[:, t] if L > 1 else None, alpha[:, t] if L > 1 else None,
            gamma[:, t] if L > 1 else None, L)
    return o, S


def forward(q, k, v, g, beta, u, alpha, gamma, conv_w, L: int,
            heads: Optional[List[int]] = None, S0=None, conv_in=None):
    """Oracle in the library's layout.

    q, k: [B, H, T, dk]; v: [B, H, T, dv]; g, beta: [B, H, T];
    u: [B, H, T, L-1, dk] (slot j holds u_{t,j+1}); alpha: [B, H, T, L];
    gamma: [B, H, T, L-1, dv] (slot j holds gamma_{t,j}); conv_w: [H, 4, dv].
    u, alpha, gamma may be None when L == 1.
    heads: optionally restrict to these head indices (all batches).
    S0: optional starting state [B, H, dk, dv] in the S_final layout (the
    transpose of S_0); conv_in: optional value rows [B, H, 3, dv] of the three
    tokens before the sequence.  Both are zero when None.
    Returns o [B, H', T, dv] and S_final [B, H', dk, dv] (the transpose of
    the dv x dk state S_T), float64.
    """
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    hs = list(range(H)) if heads is None else list(heads)
    Hs = len(hs)

    def pick(x):
        x = np.asarray(x)[:, hs]
        return x.reshape((B * Hs,) + x.shape[2:])

    w = np.asarray(conv_w, F64)[hs]                    # [Hs, 4, dv]
    w_pairs = np.broadcast_to(w[None], (B, Hs, 4, dv)).reshape(B * Hs, 4, dv)
    S0p = None if S0 is None else pick(S0).astype(F64).transpose(0, 2, 1)   # [P, dv, dk]
    o, S = forward_pairs(
        pick(q), pick(k), pick(v), pick(g), pick(beta),
        pick(u) if L > 1 else None, pick(alpha) if L > 1 else None,
        pick(gamma) if L > 1 else None, w_pairs, L,
        S0=S0p, v_hist=None if conv_in is None else pick(conv_in))
    return (o.reshape(B, Hs, T, dv),
            np.ascontiguousarray(S.transpose(0, 2, 1)).reshape(B, Hs, dk, dv))


def conv_tail(v, conv_in=None) -> np.ndarray:
    """The ShortConv window a continuation needs: the value rows of the last
    three tokens of [conv_in; v] along T ([B, H, 3, dv]; conv_in zero when None,
    so a sequence shorter than 3 tokens keeps part of the earlier history)."""
    v = np.asarray(v, F64)
    B, H, T, dv = v.shape
    hist = np.zeros((B, H, 3, dv), F64) if conv_in is None else np.asarray(conv_in, F64)
    return np.concatenate([hist, v], axis=2)[:, :, T:T + 3]


def decode_step(S, conv_state, q, k, v, g, beta, u, alpha, gamma, conv_w, L: int):
    """One token for every (b, h) pair, in the library's layout.

    S: [B, H, dk, dv] state (the S_final layout); conv_state: [B, H, 3, dv]
    values of the previous three tokens; q, k: [B, H, dk]; v: [B, H, dv];
    g, beta: [B, H]; u: [B, H, L-1, dk]; alpha: [B, H, L]; gamma: [B, H, L-1, dv];
    conv_w: [H, 4, dv].  Returns (o [B, H, dv], S' [B, H, dk, dv],
    conv_state' [B, H, 3, dv]) -- the same token step as forward(), run alone.
    """
    B, H, dk, dv = np.asarray(S).shape
    P = B * H
    Sp = np.asarray(S, F64).reshape(P, dk, dv).transpose(0, 2, 1)
    hist = np.asarray(conv_state, F64).reshape(P, 3, dv)
    vt = np.asarray(v, F64).reshape(P, dv)
    window = np.concatenate([hist, vt[:, None]], axis=1)                 # rows t-3 .. t
    w = np.broadcast_to(np.asarray(conv_w, F64)[None], (B, H, 4, dv)).reshape(P, 4, dv)
    anchor = shortconv_anchor(window, w, 3)
    S_new, o = token_step(
        Sp, np.asarray(q, F64).reshape(P, dk), np.asarray(k, F64).reshape(P, dk), vt,
        np.asarray(g, F64).reshape(P), np.asarray(beta, F64).reshape(P), anchor,
        np.asarray(u, F64).reshape(P, L - 1, dk) if L > 1 else None,
        np.asarray(alpha, F64).reshape(P, L) if L > 1 else None,
        np.asarray(gamma, F64).reshape(P, L - 1, dv) if L > 1 else None, L)
    return (o.reshape(B, H, dv), np.ascontiguousarray(S_new.transpose(0, 2, 1)).reshape(B, H, dk, dv),
            window[:, 1:].reshape(B, H, 3, dv))
