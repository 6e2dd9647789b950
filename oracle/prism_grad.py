"""Float64 gradients of the PRISM rank-L gated delta-rule forward.

TEST INFRASTRUCTURE ONLY (tests and the smoke check).

The gradients are the reverse-mode derivative of the plain token-by-token
recurrence (the same definitions as ``oracle.prism``), taken by torch autograd
on the CPU in float64, so the only step here is the forward itself written
once more with differentiable tensor operations:

  anchor_t = sum_{j=0}^{3} w_j * v_{t-3+j}        (zero before the sequence start)
  r_{t,0}  = v_t - anchor_t,  r_{t,l} = r_{t,l-1} - alpha_{t,l-1} gamma_{t,l-1} * r_{t,l-1}
  S_t      = g_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T
             + sum_{l=1}^{L-1} (alpha_{t,l} r_{t,l}) u_{t,l}^T
  o_t      = S_t q_t

([Notes] sections 2.1-2.3 of the PRISM reading notes; [Article] sections 01-四 and
03-三 of the Tencent / PKU article; [Summary] "架构全貌".)  The pages train the
layer end to end (throughput is quoted for training, [Notes] section 3.3), which
needs exactly these derivatives; they print no gradient formulas.

The scalar being differentiated is  sum_t <do_t, o_t> + <dS_final, S_final>,
with S_final = S_T^T in the library's [dk, dv] layout, so (do, dS_final) are the
incoming gradients of (o, S_final).  Pinned in tests/test_oracle_grad.py by
central finite differences of ``oracle.prism.forward`` (independent numpy code).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def _forward_pairs(q, k, v, g, beta, u, alpha, gamma, w, L: int):
    """The recurrence over P pairs with torch float64 tensors (differentiable).

    q, k: [P, T, dk]; v: [P, T, dv]; g, beta: [P, T]; u: [P, T, L-1, dk];
    alpha: [P, T, L]; gamma: [P, T, L-1, dv]; w: [P, 4, dv].
    Returns o [P, T, dv] and S_T [P, dv, dk].
    """
    import torch
    P, T, dk = q.shape
    dv = v.shape[-1]
    S = torch.zeros(P, dv, dk, dtype=torch.float64)
    v_ext = torch.cat([torch.zeros(P, 3, dv, dtype=torch.float64), v], dim=1)
    outs = []
    for t in range(T):
        kt = k[:, t]
        Sk = torch.einsum("pij,pj->pi", S, kt)
        S = g[:, t, None, None] * (S - beta[:, t, None, None] * Sk[:, :, None] * kt[:, None, :])
        S = S + beta[:, t, None, None] * v[:, t, :, None] * kt[:, None, :]
        if L > 1:
            anchor = sum(w[:, j] * v_ext[:, t + j] for j in range(4))
            r = v[:, t] - anchor
            for l in range(1, L):
                r = r - alpha[:, t, l - 1, None] * gamma[:, t, l - 1] * r
                S = S + (alpha[:, t, l, None] * r)[:, :, None] * u[:, t, l - 1, None, :]
        outs.append(torch.einsum("pij,pj->pi", S, q[:, t]))
    return torch.stack(outs, dim=1), S


def backward(q, k, v, g, beta, u, alpha, gamma, conv_w, L: int, d_o,
             dS_final: Optional[np.ndarray] = None) -> Dict[str, Optional[np.ndarray]]:
    """Gradients in the library's layout (all float64 numpy).

    Inputs as ``oracle.prism.forward``: q, k [B,H,T,dk]; v [B,H,T,dv]; g, beta
    [B,H,T]; u [B,H,T,L-1,dk]; alpha [B,H,T,L]; gamma [B,H,T,L-1,dv]; conv_w
    [H,4,dv] (u, alpha, gamma unused when L == 1).  d_o: [B,H,T,dv] gradient of o;
    dS_final: [B,H,dk,dv] gradient of S_final (zero when None).
    Returns dq, dk, dv, dg, dbeta, du, dalpha, dgamma, dconv_w with the shapes of
    the corresponding inputs (the four rank-L entries are None when L == 1).
    """
    import torch
    B, H, T, dk = np.asarray(q).shape
    dv = np.asarray(v).shape[-1]
    P = B * H

    def leaf(x):
        return torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)

    names = ["q", "k", "v", "g", "beta"] + (["u", "alpha", "gamma", "conv_w"] if L > 1 else [])
    src = dict(q=q, k=k, v=v, g=g, beta=beta, u=u, alpha=alpha, gamma=gamma, conv_w=conv_w)
    lv = {n: leaf(src[n]) for n in names}

    def pairs(x):
        return x.reshape((P,) + tuple(x.shape[2:]))

    if L > 1:
        w = lv["conv_w"][None].expand(B, H, 4, dv).reshape(P, 4, dv)
        u_, a_, gm_ = pairs(lv["u"]), pairs(lv["alpha"]), pairs(lv["gamma"])
    else:
        w = u_ = a_ = gm_ = None
    o, S = _forward_pairs(pairs(lv["q"]), pairs(lv["k"]), pairs(lv["v"]), pairs(lv["g"]),
                          pairs(lv["beta"]), u_, a_, gm_, w, L)
    loss = (o * torch.tensor(np.asarray(d_o, np.float64)).reshape(P, T, dv)).sum()
    if dS_final is not None:
        dSf = torch.tensor(np.asarray(dS_final, np.float64)).reshape(P, dk, dv)
        loss = loss + (S.transpose(1, 2) * dSf).sum()
    grads = torch.autograd.grad(loss, [lv[n] for n in names], allow_unused=True)
    out: Dict[str, Optional[np.ndarray]] = {f"d{n}": None for n in
                                            ["q", "k", "v", "g", "beta", "u", "alpha", "gamma", "conv_w"]}
    for n, gr in zip(names, grads):
        out["d" + n] = np.zeros(lv[n].shape) if gr is None else gr.detach().numpy()
    return out


def loss(q, k, v, g, beta, u, alpha, gamma, conv_w, L: int, d_o, dS_final=None) -> float:
    """The differentiated scalar, evaluated with the numpy oracle (used by the
    finite-difference pins: an independent implementation of the forward)."""
    from .prism import forward
    o, S = forward(q, k, v, g, beta, u, alpha, gamma, conv_w, L)
    val = float(np.sum(o * np.asarray(d_o, np.float64)))
    if dS_final is not None:
        val += float(np.sum(S * np.asarray(dS_final, np.float64)))
    return val
