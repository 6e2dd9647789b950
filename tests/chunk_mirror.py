"""Float64 numpy mirror of the chunked algebra that the HIP kernels run.

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
