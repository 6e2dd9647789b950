"""Float64 numpy mirror of the chunked algebra that the HIP kernels run (forward and
backward).

A test aid, not the oracle: it lets the chunk / segment / output-correction
algebra be checked against the token-by-token oracle on the CPU, at 1e-12,
before and independently of any GPU code.  It imports neither the oracle nor
the HIP library.

State H = S^T (dk x dv).  Per chunk of C tokens with start state H:
  b = cumsum(log g), G = exp(b), D_j = exp(b_C - b_j), Gam_ij = exp(b_i - b_j) (j <= i)
  M  = I + strict(diag(beta) (Gam * K K^T))           unit lower triangular
  V' = V - sum_l strict(Gam * K U_l^T) R_l
  Uc = M^-1 diag(beta) V',   Wc = M^-1 diag(beta G) K
  E  = Uc - Wc H                                      (the delta-rule new values)
  O  = diag(G) Q H + lower(Gam * Q K^T) E + sum_l lower(Gam * Q U_l^T) R_l
  H' = G_C H + K^T diag(D) E + sum_l U_l^T diag(D) R_l
Segments run the same sweep from H = 0 with the augmented state (Acc, H_loc),
Acc starting at I, so that H' = Acc_seg H_in + H_loc_seg, and the outputs are
corrected afterwards with  O = O_loc + Qhat H_in,  Qhat = (diag(G) Q - P Wc) Acc.
"""
import numpy as np


def unit_lower_inverse_blocked(M, bs=16):
    """Inverse of a unit lower-triangular matrix, by diagonal blocks of `bs`:
    diagonal blocks by forward substitution, off-diagonal blocks by
    T_ij = -T_ii sum_{k=j}^{i-1} M_ik T_kj."""
    C = M.shape[0]
    nb = (C + bs - 1) // bs
    T = np.zeros_like(M)
    for i in range(nb):
        s, e = i * bs, min(C, (i + 1) * bs)
        blk = M[s:e, s:e]
        inv = np.zeros_like(blk)
        for c in range(e - s):
            x = np.zeros(e - s)
            x[c] = 1.0
            for r in range(c + 1, e - s):
                x[r] = -blk[r, c:r] @ x[c:r]
            inv[:, c] = x
        T[s:e, s:e] = inv
    for d in range(1, nb):
        for i in range(d, nb):
            j = i - d
            si, ei = i * bs, min(C, (i + 1) * bs)
            sj, ej = j * bs, min(C, (j + 1) * bs)
            acc = np.zeros((ei - si, ej - sj))
            for k in range(j, i):
                sk, ek = k * bs, min(C, (k + 1) * bs)
                acc += M[si:ei, sk:ek] @ T[sk:ek, sj:ej]
            T[si:ei, sj:ej] = -T[si:ei, si:ei] @ acc
    return T


def prologue(v, w, alpha, gamma, L):
    """Written values R[T, L-1, dv]:  anchor by ShortConv over v (window 4,
    zero history), r_0 = v - anchor, r_l = r_{l-1} (1 - alpha_{l-1} gamma_{l-1}),
    R_l = alpha_l r_l."""
    T, dv = v.shape
    pad = np.concatenate([np.zeros((3, dv)), v], axis=0)
    anchor = sum(w[j] * pad[j:j + T] for j in range(4))
    r = v - anchor
    R = np.zeros((T, max(L - 1, 0), dv))
    for l in range(1, L):
        r = r * (1.0 - alpha[:, l - 1, None] * gamma[:, l - 1, :])
        R[:, l - 1] = alpha[:, l, None] * r
    return R


def chunk_terms(Q, K, V, U, R, g, beta):
    """Per-chunk quantities that do not depend on the start state."""
    C = Q.shape[0]
    Lm1 = U.shape[1]
    b = np.cumsum(np.log(g))
    G = np.exp(b)
    D = np.exp(b[-1] - b)
    diff = b[:, None] - b[None, :]
    low = np.tril(np.ones((C, C), dtype=bool))
    strict = np.tril(np.ones((C, C), dtype=bool), -1)
    Gam = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)
    M = np.eye(C) + np.where(strict, beta[:, None] * Gam * (K @ K.T), 0.0)
    Vp = V.copy()
    PU = []
    for l in range(Lm1):
        Vp -= np.where(strict, Gam * (K @ U[:, l].T), 0.0) @ R[:, l]
        PU.append(np.where(low, Gam * (Q @ U[:, l].T), 0.0))
    Tinv = unit_lower_inverse_blocked(M)
    Uc = Tinv @ (beta[:, None] * Vp)
    Wc = Tinv @ ((beta * G)[:, None] * K)
    P = np.where(low, Gam * (Q @ K.T), 0.0)
    O0 = P @ Uc + sum((PU[l] @ R[:, l] for l in range(Lm1)), np.zeros_like(V))
    Qt = G[:, None] * Q - P @ Wc
    HB = sum((U[:, l].T @ (D[:, None] * R[:, l]) for l in range(Lm1)), np.zeros((K.shape[1], V.shape[1])))
    return dict(G=G, D=D, GC=G[-1], Uc=Uc, Wc=Wc, P=P, O0=O0, Qt=Qt, HB=HB)


def forward_chunked(q, k, v, g, beta, u, alpha, gamma, w, L, chunk, seg_chunks=None):
    """One (b, h) pair.  q, k [T, dk]; v [T, dv]; g, beta [T]; u [T, L-1, dk];
    alpha [T, L]; gamma [T, L-1, dv]; w [4, dv].  Returns o [T, dv], H_final [dk, dv]."""
    T, dk = q.shape
    dv = v.shape[1]
    Lm1 = max(L - 1, 0)
    if L == 1:
        u = np.zeros((T, 0, dk)); alpha = np.zeros((T, 1)); gamma = np.zeros((T, 0, dv))
    R = prologue(v, w, alpha, gamma, L)
    nchunks = (T + chunk - 1) // chunk
    Tp = nchunks * chunk
    def pad(x, fill=0.0):
        out = np.full((Tp,) + x.shape[1:], fill)
        out[:T] = x
        return out
    qp, kp, vp, up, Rp = pad(q), pad(k), pad(v), pad(u), pad(R)
    gp, bp = pad(g, 1.0), pad(beta, 0.0)
    seg_chunks = nchunks if seg_chunks is None else seg_chunks
    nseg = (nchunks + seg_chunks - 1) // seg_chunks
    o = np.zeros((Tp, dv))
    aggs = []
    local = []
    for s in range(nseg):
        Acc = np.eye(dk)
        Hl = np.zeros((dk, dv))
        seg_out = []
        for c in range(s * seg_chunks, min(nchunks, (s + 1) * seg_chunks)):
            sl = slice(c * chunk, (c + 1) * chunk)
            t = chunk_terms(qp[sl], kp[sl], vp[sl], up[sl], Rp[sl], gp[sl], bp[sl])
            O_loc = t["Qt"] @ Hl + t["O0"]
            Qhat = t["Qt"] @ Acc
            seg_out.append((sl, O_loc, Qhat))
            E = t["Uc"] - t["Wc"] @ Hl
            KD = kp[sl].T * t["D"][None, :]
            Hl = t["GC"] * Hl + KD @ E + t["HB"]
            Acc = t["GC"] * Acc - KD @ (t["Wc"] @ Acc)
        aggs.append((Acc, Hl))
        local.append(seg_out)
    Hin = np.zeros((dk, dv))
    for s in range(nseg):
        for sl, O_loc, Qhat in local[s]:
            o[sl] = O_loc + Qhat @ Hin
        Acc, Hl = aggs[s]
        Hin = Acc @ Hin + Hl
    return o[:T], Hin


# ---------------------------------------------------------------------------------------
# The chunked backward.  Per chunk, with E = Uc - Wc H the delta-rule new values,
#   O  = diag(G) Q H + P E + sum_l PU_l R_l,     P = lower(Gam * Q K^T), PU_l = lower(Gam * Q U_l^T)
#   H' = G_C H + K^T diag(D) E + sum_l U_l^T diag(D) R_l
# every step is a matrix product, so its adjoint is one too.  Given dO and the adjoint dH'
# of the chunk's end state, the adjoint of its start state is
#   dH = Qt^T dO + Acc^T dH',   Qt = diag(G) Q - P Wc,   Acc = G_C I - K^T diag(D) Wc,
# which is the segment form with (Acc, ell = Qt^T dO) per chunk.
def chunk_grads(Q, K, V, U, R, g, beta, H, dHp, dO):
    """Adjoint of one chunk from its start state H and the adjoint dH' of its end state.
    Returns dQ, dK, dV (direct path), dU [C, Lm1, dk], dR [C, Lm1, dv], dbeta, dg, dH."""
    C = Q.shape[0]
    Lm1 = U.shape[1]
    b = np.cumsum(np.log(g))
    G = np.exp(b)
    D = np.exp(b[-1] - b)
    low = np.tril(np.ones((C, C), dtype=bool))
    strict = np.tril(np.ones((C, C), dtype=bool), -1)
    Gam = np.where(low, np.exp(np.where(low, b[:, None] - b[None, :], 0.0)), 0.0)
    KK = K @ K.T
    A = np.where(strict, beta[:, None] * Gam * KK, 0.0)
    Tinv = np.linalg.inv(np.eye(C) + A)
    N = [np.where(strict, Gam * (K @ U[:, l].T), 0.0) for l in range(Lm1)]
    PU = [np.where(low, Gam * (Q @ U[:, l].T), 0.0) for l in range(Lm1)]
    Vp = V - sum((N[l] @ R[:, l] for l in range(Lm1)), np.zeros_like(V))
    X1 = beta[:, None] * Vp
    X2 = (beta * G)[:, None] * K
    Uc, Wc = Tinv @ X1, Tinv @ X2
    E = Uc - Wc @ H
    P = np.where(low, Gam * (Q @ K.T), 0.0)
    # readout and end-state terms
    dE = P.T @ dO + D[:, None] * (K @ dHp)
    dH = Q.T @ (G[:, None] * dO) + G[-1] * dHp - Wc.T @ dE
    EdH = E @ dHp.T
    dK = D[:, None] * EdH
    dD = np.sum(K * EdH, axis=1)
    dGv = np.sum(dO * (Q @ H), axis=1)
    dQ = G[:, None] * (dO @ H.T)
    dGC = float(np.sum(dHp * H))
    dP = np.where(low, dO @ E.T, 0.0)
    dQ += (Gam * dP) @ K
    dK += (Gam * dP).T @ Q
    dlG = dP * P
    dU = np.zeros_like(U)
    dR = np.zeros_like(R)
    for l in range(Lm1):
        RdH = R[:, l] @ dHp.T
        dU[:, l] += D[:, None] * RdH
        dR[:, l] += D[:, None] * (U[:, l] @ dHp) + PU[l].T @ dO
        dD += np.sum(U[:, l] * RdH, axis=1)
        dPU = np.where(low, dO @ R[:, l].T, 0.0)
        dQ += (Gam * dPU) @ U[:, l]
        dU[:, l] += (Gam * dPU).T @ Q
        dlG += dPU * PU[l]
    # through the UT transform: Uc = T X1, Wc = T X2, T = (I + A)^-1
    dX1 = Tinv.T @ dE
    dX2 = Tinv.T @ (-(dE @ H.T))
    dVp = beta[:, None] * dX1
    rk = np.sum(K * dX2, axis=1)
    dbeta = np.sum(Vp * dX1, axis=1) + G * rk
    dGv += beta * rk
    dK += (beta * G)[:, None] * dX2
    dA = np.where(strict, -(dX1 @ Uc.T) - dX2 @ Wc.T, 0.0)
    dbeta += np.sum(dA * Gam * KK, axis=1)
    Z = beta[:, None] * Gam * dA
    dK += Z @ K + Z.T @ K
    dlG += dA * A
    for l in range(Lm1):
        dN = np.where(strict, -(dVp @ R[:, l].T), 0.0)
        dR[:, l] -= N[l].T @ dVp
        dK += (Gam * dN) @ U[:, l]
        dU[:, l] += (Gam * dN).T @ K
        dlG += dN * N[l]
    # decays: Gam_ij = exp(b_i - b_j), G_i = exp(b_i), D_j = exp(b_C - b_j), b = cumsum(log g)
    db = dGv * G - dD * D + dlG.sum(axis=1) - dlG.sum(axis=0)
    db[-1] += np.sum(dD * D) + dGC * G[-1]
    dg = np.cumsum(db[::-1])[::-1] / g
    return dQ, dK, dVp, dU, dR, dbeta, dg, dH


def chain_backward(v, w, alpha, gamma, L, dR):
    """Adjoint of the written values R_l = alpha_l r_l through the residual chain and the
    ShortConv anchor (zero history).  Returns dv, dalpha [T, L], dgamma [T, L-1, dv], dw."""
    T, dv = v.shape
    pad = np.concatenate([np.zeros((3, dv)), v], axis=0)
    anchor = sum(w[j] * pad[j:j + T] for j in range(4))
    r = [v - anchor]
    for l in range(1, L):
        r.append(r[-1] * (1.0 - alpha[:, l - 1, None] * gamma[:, l - 1, :]))
    dalpha = np.zeros((T, L))
    dgamma = np.zeros((T, max(L - 1, 0), dv))
    dr = np.zeros((T, dv))
    for l in range(L - 1, 0, -1):
        dalpha[:, l] += np.sum(dR[:, l - 1] * r[l], axis=1)
        dr = dr + alpha[:, l, None] * dR[:, l - 1]
        f = alpha[:, l - 1, None] * gamma[:, l - 1, :]
        dalpha[:, l - 1] -= np.sum(dr * gamma[:, l - 1, :] * r[l - 1], axis=1)
        dgamma[:, l - 1] = -dr * alpha[:, l - 1, None] * r[l - 1]
        dr = dr * (1.0 - f)
    dv_out = dr.copy()
    dw = np.zeros((4, dv))
    dpad = np.zeros((T + 3, dv))
    for j in range(4):
        dw[j] = -np.sum(dr * pad[j:j + T], axis=0)
        dpad[j:j + T] -= w[j] * dr
    dv_out += dpad[3:]
    return dv_out, dalpha, dgamma, dw


def backward_chunked(q, k, v, g, beta, u, alpha, gamma, w, L, chunk, d_o, dS_final=None):
    """Gradients of sum <d_o, o> + <dS_final, S_final> for one (b, h) pair, by chunks:
    a forward over the chunks keeping each chunk's start state, then the chunk adjoints
    last first.  Shapes as forward_chunked; d_o [T, dv]; dS_final [dk, dv] or None.
    Returns dq, dk, dv, dg, dbeta, du, dalpha, dgamma, dconv_w (per pair)."""
    T, dk = q.shape
    dv = v.shape[1]
    Lm1 = max(L - 1, 0)
    if L == 1:
        u = np.zeros((T, 0, dk)); alpha = np.zeros((T, 1)); gamma = np.zeros((T, 0, dv))
    R = prologue(v, w, alpha, gamma, L)
    nch = (T + chunk - 1) // chunk
    Tp = nch * chunk

    def pad(x, fill=0.0):
        out = np.full((Tp,) + x.shape[1:], fill)
        out[:T] = x
        return out
    qp, kp, vp, up, Rp, dop = pad(q), pad(k), pad(v), pad(u), pad(R), pad(d_o)
    gp, bp = pad(g, 1.0), pad(beta, 0.0)
    starts = []
    H = np.zeros((dk, dv))
    for c in range(nch):
        sl = slice(c * chunk, (c + 1) * chunk)
        t = chunk_terms(qp[sl], kp[sl], vp[sl], up[sl], Rp[sl], gp[sl], bp[sl])
        starts.append(H)
        E = t["Uc"] - t["Wc"] @ H
        H = t["GC"] * H + (kp[sl].T * t["D"][None, :]) @ E + t["HB"]
    out = {n: np.zeros((Tp,) + s) for n, s in
           [("dq", (dk,)), ("dk", (dk,)), ("dv", (dv,)), ("dg", ()), ("dbeta", ()),
            ("du", (Lm1, dk)), ("dR", (Lm1, dv))]}
    dH = np.zeros((dk, dv)) if dS_final is None else np.asarray(dS_final, np.float64)
    for c in range(nch - 1, -1, -1):
        sl = slice(c * chunk, (c + 1) * chunk)
        dQ, dK, dV, dU, dRc, dB, dG, dH = chunk_grads(qp[sl], kp[sl], vp[sl], up[sl], Rp[sl], gp[sl], bp[sl],
                                                       starts[c], dH, dop[sl])
        out["dq"][sl], out["dk"][sl], out["dv"][sl] = dQ, dK, dV
        out["du"][sl], out["dR"][sl], out["dbeta"][sl], out["dg"][sl] = dU, dRc, dB, dG
    res = {n: out[n][:T] for n in ["dq", "dk", "dv", "dg", "dbeta", "du"]}
    dvc, dalpha, dgamma, dw = chain_backward(v, w, alpha, gamma, L, out["dR"][:T])
    res["dv"] = res["dv"] + dvc
    res["dalpha"], res["dgamma"], res["dconv_w"] = dalpha, dgamma, dw
    return res
