// prism_kernels.h - HIP kernels of the PRISM rank-L gated delta-rule forward (gfx950).
//
// Three launches per forward:
//   seg_local  : one workgroup per (segment, pair).  Sweeps the segment's chunks
//                from a zero state with the chunked UT/WY form of the delta rule,
//                fusing the ShortConv anchor and the residual chain (prologue),
//                and writes the zero-start outputs O_loc, the output-correction
//                rows Qhat and the segment operator (A_seg, B_seg).
//   seg_scan   : one workgroup per (pair, 16 state columns).  Runs the short
//                sequential recurrence H_in(s+1) = A_s H_in(s) + B_s over the
//                segments (float32) and writes the final state.
//   seg_fixup  : one workgroup per (chunk, pair).  o = O_loc + Qhat H_in(seg).
//
// Math (state H = S^T, dk x dv; per chunk of C tokens, start state H):
//   b = cumsum(log g), G = exp(b), D_j = exp(b_last - b_j), Gam_ij = exp(b_i - b_j), j <= i
//   M  = I + strict(diag(beta) (Gam * K K^T))                (unit lower triangular)
//   V' = V - sum_l strict(Gam * K U_l^T) R_l
//   Uc = M^-1 diag(beta) V',   Wc = M^-1 diag(beta G) K
//   E  = Uc - Wc H
//   O  = diag(G) Q H + lower(Gam * Q K^T) E + sum_l lower(Gam * Q U_l^T) R_l
//   H' = G_last H + K^T diag(D) E + sum_l U_l^T diag(D) R_l
// The forgetting operator is the Gated DeltaNet one and the write is the rank-L
// injection of the PRISM reading notes (liuzhao09.github.io, "PRISM", sections
// 2.2-2.3); associativity of S_t = S_{t-1} A_t + B_t (notes section 2.1, Tencent
// Ads article section 01-二) is what lets segments start from zero and be
// corrected afterwards:  H_chunk_start = H_loc + A_acc H_in,
//   O = O_loc + Qhat H_in,  Qhat = (diag(G) Q - lower(Gam * Q K^T) Wc) A_acc.
#pragma once
#include "prism_tile.h"

namespace prism {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* u;
  const void* gamma;
  const float* g;
  const float* beta;
  const float* alpha;
  const float* conv_w;
  void* o;
  float* S_final;
  const float* S0;       // [P][dk][dv] starting state (the S_final layout), or null for zero
  const void* conv_in;   // [P][3][dv] values of the 3 tokens before the sequence, or null
  void* conv_out;        // [P][3][dv] values of the last 3 tokens of [conv_in; v], or null
  float* Oloc;   // [P][Tpad][dv], I/O type (bf16 fast path: fragment order)
  float* Qhat;   // [P][Tpad][dk], I/O type (bf16 fast path: fragment order)
  float* Aagg;   // [P][nseg][dk][dk]
  float* Bagg;   // [P][nseg][dk][dv]
  float* Hin;    // [P][nseg][dk][dv]
  int B, H, T, L;
  int nch;          // chunks per sequence
  int seg_chunks;   // chunks per segment
  int nseg;         // segments per sequence
  // residual chain: 0 = r_l = r_{l-1} (1 - alpha_{l-1} gamma_{l-1}), written alpha_l r_l;
  // 1 = written corrections: d_l = gamma_{l-1} r_{l-1}, r_l = r_{l-1} - d_l, written
  // alpha_l d_l (gamma then holds per-channel factors of the corrections)
  int chain_delta;
};

// LDS plan of seg_local (bytes).  Row strides are padded by 16 bytes.
template <class E, int DK, int DV, int C>
struct SegLds {
  static constexpr int PADE = 16 / (int)sizeof(E);
  static constexpr int LDK = DK + PADE, LDC = C + PADE;
  static constexpr int SROWS = DV > DK ? DV : DK;
  static constexpr int LDF = C + 1;  // float32 solve arrays
  static constexpr size_t oQ = 0;
  static constexpr size_t oK = oQ + (size_t)C * LDK * sizeof(E);
  static constexpr size_t oP = oK + (size_t)C * LDK * sizeof(E);
  static constexpr size_t oT = oP + (size_t)C * LDC * sizeof(E);
  static constexpr size_t oW = oT + (size_t)C * LDC * sizeof(E);
  static constexpr size_t oS = oW + (size_t)C * LDK * sizeof(E);
  static constexpr size_t oGate = oS + (size_t)SROWS * LDK * sizeof(E);
  static constexpr size_t nGate = 5 * C + 8 * C;  // b, G, D, beta, beta*G, alpha[C][8]
  static constexpr size_t oX = oGate + nGate * sizeof(float);
  static constexpr size_t xLoop = (size_t)C * LDK * sizeof(E) + 2 * (size_t)C * LDC * sizeof(E);
  static constexpr size_t xSolve = 2 * (size_t)C * LDF * sizeof(float) + 3 * 16 * 17 * sizeof(float);
  static constexpr size_t xQt = (size_t)C * LDK * sizeof(E);
  static constexpr size_t xSize = xLoop > xSolve ? (xLoop > xQt ? xLoop : xQt) : (xSolve > xQt ? xSolve : xQt);
  static constexpr size_t total = oX + xSize;
  static constexpr bool fits = total <= 160 * 1024;
};

template <class E, int DK, int DV, int C, int NW>
__global__ __launch_bounds__(64 * NW, 1) void seg_local_kernel(FwdArgs a) {
  using Ly = SegLds<E, DK, DV, C>;
  constexpr int LDK = Ly::LDK, LDC = Ly::LDC, LDF = Ly::LDF;
  constexpr int MT = C / 16, KT = DK / 16, VT = DV / 16;
  constexpr int NVW = (VT + NW - 1) / NW;  // value column blocks per wave
  constexpr int NKW = (KT + NW - 1) / NW;  // key column blocks per wave
  constexpr int NT = 64 * NW;              // threads
  __shared__ __align__(16) unsigned char smem[Ly::total];
  E* sQ = reinterpret_cast<E*>(smem + Ly::oQ);
  E* sK = reinterpret_cast<E*>(smem + Ly::oK);
  E* sP = reinterpret_cast<E*>(smem + Ly::oP);
  E* sT = reinterpret_cast<E*>(smem + Ly::oT);
  E* sW = reinterpret_cast<E*>(smem + Ly::oW);
  E* sS = reinterpret_cast<E*>(smem + Ly::oS);
  float* sB = reinterpret_cast<float*>(smem + Ly::oGate);
  float* sG = sB + C;
  float* sD = sG + C;
  float* sBeta = sD + C;
  float* sBG = sBeta + C;
  float* sAlpha = sBG + C;  // [C][8]
  unsigned char* X = smem + Ly::oX;
  E* sU = reinterpret_cast<E*>(X);
  E* sX1 = reinterpret_cast<E*>(X + (size_t)C * LDK * sizeof(E));
  E* sX2 = sX1 + C * LDC;
  float* sMf = reinterpret_cast<float*>(X);
  float* sTf = sMf + C * LDF;
  float* sTmp = sTf + C * LDF;  // [3][16][17]
  E* sQt = reinterpret_cast<E*>(X);

  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), g4 = (l >> 4) * 4, li = l & 15;
  const int seg = blockIdx.x, pr = blockIdx.y;
  const int hd = pr % a.H;
  const int T = a.T, L = a.L, Lm1 = L - 1;
  const int c_begin = seg * a.seg_chunks;
  const int c_end = min(a.nch, c_begin + a.seg_chunks);
  const int Tpad = a.nch * C;
  const E* q = reinterpret_cast<const E*>(a.q) + (size_t)pr * T * DK;
  const E* k = reinterpret_cast<const E*>(a.k) + (size_t)pr * T * DK;
  const E* v = reinterpret_cast<const E*>(a.v) + (size_t)pr * T * DV;
  const E* u = L > 1 ? reinterpret_cast<const E*>(a.u) + (size_t)pr * T * Lm1 * DK : nullptr;
  const E* gam = L > 1 ? reinterpret_cast<const E*>(a.gamma) + (size_t)pr * T * Lm1 * DV : nullptr;
  const float* gg = a.g + (size_t)pr * T;
  const float* bb = a.beta + (size_t)pr * T;
  const float* al = L > 1 ? a.alpha + (size_t)pr * T * L : nullptr;
  const float* cw = L > 1 ? a.conv_w + (size_t)hd * 4 * DV : nullptr;

  // State tiles owned by this wave: value column blocks vt = w + NW*jv, key
  // column blocks kt' = w + NW*jk.
  f32x4 Hs[NVW][KT];   // H(kt, vt)
  f32x4 As[NKW][KT];   // A_acc(kt, kt')
#pragma unroll
  for (int jv = 0; jv < NVW; ++jv)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) Hs[jv][kt] = zero4();
#pragma unroll
  for (int jk = 0; jk < NKW; ++jk)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int kc = w + NW * jk;
      f32x4 t = zero4();
      if (kc == kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (g4 + r == li) ? 1.f : 0.f;
      }
      As[jk][kt] = t;
    }

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * C;
    const int nvalid = min(C, T - t0);

    // ---- stage 0: state operand (H^T) into LDS, Q / K rows, gates --------------
#pragma unroll
    for (int jv = 0; jv < NVW; ++jv) {
      const int vt = w + NW * jv;
      if (vt < VT) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sS[(16 * vt + li) * LDK + 16 * kt + g4 + r] = from_f<E>(Hs[jv][kt][r]);
      }
    }
    {
      constexpr int VEC = 16 / sizeof(E);
      constexpr int PER_ROW = DK / VEC;
      for (int idx = tid; idx < C * PER_ROW; idx += NT) {
        const int row = idx / PER_ROW, cv = (idx % PER_ROW) * VEC;
        uint4 qv = make_uint4(0, 0, 0, 0), kv = make_uint4(0, 0, 0, 0);
        if (row < nvalid) {
          qv = *reinterpret_cast<const uint4*>(q + (size_t)(t0 + row) * DK + cv);
          kv = *reinterpret_cast<const uint4*>(k + (size_t)(t0 + row) * DK + cv);
        }
        *reinterpret_cast<uint4*>(sQ + row * LDK + cv) = qv;
        *reinterpret_cast<uint4*>(sK + row * LDK + cv) = kv;
      }
    }
    if (w == 0) {
      const bool ok = l < nvalid;
      float lam = (ok && l < C) ? __logf(gg[t0 + l]) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        float y = __shfl_up(lam, off);
        if (l >= off) lam += y;
      }
      const float blast = __shfl(lam, C - 1);
      if (l < C) {
        const float be = ok ? bb[t0 + l] : 0.f;
        const float G = __expf(lam);
        sB[l] = lam;
        sG[l] = G;
        sD[l] = __expf(blast - lam);
        sBeta[l] = be;
        sBG[l] = be * G;
        for (int j = 0; j < L; ++j) sAlpha[l * 8 + j] = (ok && L > 1) ? al[(size_t)(t0 + l) * L + j] : 0.f;
      }
    }
    __syncthreads();

    // ---- prologue: V' init, anchor and initial residual, in tile layout ------
    // The state's operand copy in LDS (stage 0) is all the chunk reads of the old H; the
    // registers now take the decayed state G_C H, and the chunk's write terms accumulate
    // into them (H' = G_C H + sum_l U_l^T D R_l + K^T D E).
    f32x4 Vp[NVW][MT], Oc[NVW][MT], Rr[NVW][MT];
#pragma unroll
    for (int jv = 0; jv < NVW; ++jv) {
      const int vt = w + NW * jv;
      const float GC0 = sG[C - 1];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) Hs[jv][kt][r] *= GC0;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        Oc[jv][mt] = zero4();
        f32x4 vv = zero4(), rr = zero4();
        if (vt < VT) {
          const int col = 16 * vt + li;
          const E* hist = a.conv_in != nullptr ? reinterpret_cast<const E*>(a.conv_in) + (size_t)pr * 3 * DV : nullptr;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * mt + g4 + r;
            if (t < nvalid) {
              const int tg = t0 + t;
              const float x = to_f(v[(size_t)tg * DV + col]);
              vv[r] = x;
              if (L > 1) {
                float anc = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const int ts = tg - 3 + j;
                  if (ts >= 0) anc += cw[j * DV + col] * to_f(v[(size_t)ts * DV + col]);
                  else if (hist != nullptr) anc += cw[j * DV + col] * to_f(hist[(ts + 3) * DV + col]);
                }
                rr[r] = x - anc;
              }
            }
          }
        }
        Vp[jv][mt] = vv;
        Rr[jv][mt] = rr;
      }
    }

    // ---- P = lower(Gam * Q K^T) -----------------------------------------------
    for (int tI = w; tI < MT * MT; tI += NW) {
      const int mt = tI / MT, jt = tI % MT;
      f32x4 acc = zero4();
      if (jt <= mt) mm_ll<E>(acc, sQ, LDK, 16 * mt, sK, LDK, 16 * jt, DK);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * mt + g4 + r, j = 16 * jt + li;
        const float val = (j <= i) ? __expf(sB[i] - sB[j]) * acc[r] : 0.f;
        sP[i * LDC + j] = from_f<E>(val);
      }
    }

    // ---- rank-L terms, one refinement step at a time ---------------------------
    for (int lr = 1; lr < L; ++lr) {
      {  // U_l rows into LDS
        constexpr int VEC = 16 / sizeof(E);
        constexpr int PER_ROW = DK / VEC;
        for (int idx = tid; idx < C * PER_ROW; idx += NT) {
          const int row = idx / PER_ROW, cv = (idx % PER_ROW) * VEC;
          uint4 uv = make_uint4(0, 0, 0, 0);
          if (row < nvalid)
            uv = *reinterpret_cast<const uint4*>(u + ((size_t)(t0 + row) * Lm1 + (lr - 1)) * DK + cv);
          *reinterpret_cast<uint4*>(sU + row * LDK + cv) = uv;
        }
      }
      // residual step and written values R_l = alpha_l r_l (tile layout)
      f32x4 R[NVW][MT];
#pragma unroll
      for (int jv = 0; jv < NVW; ++jv) {
        const int vt = w + NW * jv;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 rv = zero4();
          if (vt < VT) {
            const int col = 16 * vt + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 16 * mt + g4 + r;
              if (t < nvalid) {
                const float gm = to_f(gam[((size_t)(t0 + t) * Lm1 + (lr - 1)) * DV + col]);
                if (a.chain_delta) {  // the correction itself is written and subtracted
                  const float d = gm * Rr[jv][mt][r];
                  Rr[jv][mt][r] -= d;
                  rv[r] = sAlpha[t * 8 + lr] * d;
                } else {
                  const float x = Rr[jv][mt][r] * (1.f - sAlpha[t * 8 + lr - 1] * gm);
                  Rr[jv][mt][r] = x;
                  rv[r] = sAlpha[t * 8 + lr] * x;
                }
              }
            }
          }
          R[jv][mt] = rv;
        }
      }
      __syncthreads();
      // X1 = -strict(Gam * K U^T), X2 = lower(Gam * Q U^T)
      for (int tI = w; tI < 2 * MT * MT; tI += NW) {
        const int which = tI / (MT * MT), t2 = tI % (MT * MT);
        const int mt = t2 / MT, jt = t2 % MT;
        f32x4 acc = zero4();
        if (jt <= mt) mm_ll<E>(acc, which ? sQ : sK, LDK, 16 * mt, sU, LDK, 16 * jt, DK);
        E* dst = which ? sX2 : sX1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * mt + g4 + r, j = 16 * jt + li;
          float val = 0.f;
          if (which ? (j <= i) : (j < i)) val = __expf(sB[i] - sB[j]) * acc[r];
          dst[i * LDC + j] = from_f<E>(which ? val : -val);
        }
      }
      __syncthreads();
#pragma unroll
      for (int jv = 0; jv < NVW; ++jv) {
        if (w + NW * jv < VT) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            mm_lt<E, MT>(Vp[jv][mt], sX1, LDC, 16 * mt, R[jv], nullptr, C);
            mm_lt<E, MT>(Oc[jv][mt], sX2, LDC, 16 * mt, R[jv], nullptr, C);
          }
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) mm_tt<E, MT>(Hs[jv][kt], sU, LDK, 16 * kt, sD, R[jv], C);
        }
      }
      __syncthreads();
    }

    // ---- UT transform: T = (I + strict(diag(beta) Gam * K K^T))^-1 -------------
    for (int tI = w; tI < MT * MT; tI += NW) {
      const int mt = tI / MT, jt = tI % MT;
      f32x4 acc = zero4();
      if (jt <= mt) mm_ll<E>(acc, sK, LDK, 16 * mt, sK, LDK, 16 * jt, DK);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * mt + g4 + r, j = 16 * jt + li;
        sMf[i * LDF + j] = (j < i) ? sBeta[i] * __expf(sB[i] - sB[j]) * acc[r] : 0.f;
      }
    }
    __syncthreads();
    if (w < MT && l < 16) {  // diagonal 16x16 blocks by forward substitution, one column per lane
      const int base = 16 * w, cc = l;
      float x[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float s = (rr == cc) ? 1.f : 0.f;
        if (rr > cc) {
#pragma unroll
          for (int kk = 0; kk < rr; ++kk)
            if (kk >= cc) s -= sMf[(base + rr) * LDF + base + kk] * x[kk];
        }
        x[rr] = s;
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sTf[(base + rr) * LDF + base + cc] = x[rr];
    }
    __syncthreads();
    for (int d = 1; d < MT; ++d) {  // off-diagonal blocks, T_ij = -T_ii sum_k M_ik T_kj
      // thread (r, cc) of each group of 256 threads takes element (r, cc) of every
      // (NW / 4)-th block of the diagonal d
      const int r = (tid >> 4) & 15, cc = tid & 15, grp = tid >> 8;
      for (int bi = d + grp; bi < MT; bi += NW / 4) {
        const int bj = bi - d;
        float s = 0.f;
        for (int kk = 16 * bj; kk < 16 * bi; ++kk) s += sMf[(16 * bi + r) * LDF + kk] * sTf[kk * LDF + 16 * bj + cc];
        sTmp[(bi - d) * 272 + r * 17 + cc] = s;
      }
      __syncthreads();
      for (int bi = d + grp; bi < MT; bi += NW / 4) {
        const int bj = bi - d;
        float s = 0.f;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) s += sTf[(16 * bi + r) * LDF + 16 * bi + kk] * sTmp[(bi - d) * 272 + kk * 17 + cc];
        sTf[(16 * bi + r) * LDF + 16 * bj + cc] = -s;
      }
      __syncthreads();
    }
    for (int idx = tid; idx < C * C; idx += NT) {
      const int i = idx / C, j = idx % C;
      sT[i * LDC + j] = from_f<E>(j <= i ? sTf[i * LDF + j] : 0.f);
    }
    __syncthreads();

    // ---- Uc = T diag(beta) V',  Wc = T diag(beta G) K ---------------------------
    f32x4 Wc[NKW][MT];
#pragma unroll
    for (int jv = 0; jv < NVW; ++jv) {
      f32x4 Uc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        Uc[mt] = zero4();
        if (w + NW * jv < VT) mm_lt<E, MT>(Uc[mt], sT, LDC, 16 * mt, Vp[jv], sBeta, C);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) Vp[jv][mt] = Uc[mt];
    }
#pragma unroll
    for (int jk = 0; jk < NKW; ++jk) {
      const int kc = w + NW * jk;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = zero4();
        if (kc < KT) {
          mm_ls<E>(acc, sT, LDC, 16 * mt, sK, LDK, 16 * kc, sBG, C);
#pragma unroll
          for (int r = 0; r < 4; ++r) sW[(16 * mt + g4 + r) * LDK + 16 * kc + li] = from_f<E>(acc[r]);
        }
        Wc[jk][mt] = acc;
      }
    }
    __syncthreads();

    // ---- E = Uc - Wc H;  O_loc;  H update ---------------------------------------
    E* oloc = reinterpret_cast<E*>(a.Oloc) + ((size_t)pr * Tpad + t0) * DV;
#pragma unroll
    for (int jv = 0; jv < NVW; ++jv) {
      const int vt = w + NW * jv;
      if (vt >= VT) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 wh = zero4(), qh = zero4();
        mm_ll<E>(wh, sW, LDK, 16 * mt, sS, LDK, 16 * vt, DK);
        mm_ll<E>(qh, sQ, LDK, 16 * mt, sS, LDK, 16 * vt, DK);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Vp[jv][mt][r] -= wh[r];                       // E
          Oc[jv][mt][r] += sG[16 * mt + g4 + r] * qh[r];  // diag(G) Q H
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        mm_lt<E, MT>(Oc[jv][mt], sP, LDC, 16 * mt, Vp[jv], nullptr, C);
#pragma unroll
        for (int r = 0; r < 4; ++r) oloc[(size_t)(16 * mt + g4 + r) * DV + 16 * vt + li] = from_f<E>(Oc[jv][mt][r]);
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) mm_tt<E, MT>(Hs[jv][kt], sK, LDK, 16 * kt, sD, Vp[jv], C);
    }
    __syncthreads();
    // A_acc^T into the state-operand buffer
#pragma unroll
    for (int jk = 0; jk < NKW; ++jk) {
      const int kc = w + NW * jk;
      if (kc < KT) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sS[(16 * kc + li) * LDK + 16 * kt + g4 + r] = from_f<E>(As[jk][kt][r]);
      }
    }
    __syncthreads();

    // ---- Qtilde = diag(G) Q - P Wc;  A_acc update ------------------------------
    {
      const float GC = sG[C - 1];
#pragma unroll
      for (int jk = 0; jk < NKW; ++jk) {
        const int kc = w + NW * jk;
        if (kc >= KT) continue;
        f32x4 WA[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 pw = zero4();
          mm_lt<E, MT>(pw, sP, LDC, 16 * mt, Wc[jk], nullptr, C);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * mt + g4 + r;
            sQt[i * LDK + 16 * kc + li] = from_f<E>(sG[i] * to_f(sQ[i * LDK + 16 * kc + li]) - pw[r]);
          }
          WA[mt] = zero4();
          mm_ll<E>(WA[mt], sW, LDK, 16 * mt, sS, LDK, 16 * kc, DK);
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          f32x4 acc = zero4();
          mm_tt<E, MT>(acc, sK, LDK, 16 * kt, sD, WA, C);
#pragma unroll
          for (int r = 0; r < 4; ++r) As[jk][kt][r] = GC * As[jk][kt][r] - acc[r];
        }
      }
    }
    __syncthreads();
    // ---- Qhat = Qtilde A_acc (A_acc before this chunk) --------------------------
    {
      E* qhat = reinterpret_cast<E*>(a.Qhat) + ((size_t)pr * Tpad + t0) * DK;
      for (int tI = w; tI < MT * KT; tI += NW) {
        const int mt = tI / KT, kc = tI % KT;
        f32x4 acc = zero4();
        mm_ll<E>(acc, sQt, LDK, 16 * mt, sS, LDK, 16 * kc, DK);
#pragma unroll
        for (int r = 0; r < 4; ++r) qhat[(size_t)(16 * mt + g4 + r) * DK + 16 * kc + li] = from_f<E>(acc[r]);
      }
    }
    __syncthreads();
  }

  // ---- segment operator ---------------------------------------------------------
  float* Ag = a.Aagg + ((size_t)pr * a.nseg + seg) * DK * DK;
  float* Bg = a.Bagg + ((size_t)pr * a.nseg + seg) * DK * DV;
#pragma unroll
  for (int jk = 0; jk < NKW; ++jk) {
    const int kc = w + NW * jk;
    if (kc >= KT) continue;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Ag[(16 * kt + g4 + r) * DK + 16 * kc + li] = As[jk][kt][r];
  }
#pragma unroll
  for (int jv = 0; jv < NVW; ++jv) {
    const int vt = w + NW * jv;
    if (vt >= VT) continue;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Bg[(16 * kt + g4 + r) * DV + 16 * vt + li] = Hs[jv][kt][r];
  }
}

// x from the lane the DPP control CTRL names (within a row of 16 lanes)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Inter-segment recurrence H_in(s+1) = A_s H_in(s) + B_s (float32) for NQ state columns of
// one pair (NQ = 8 at DK = 128, else 4).  Thread (i, q) = (tid / NQ, tid % NQ) takes row i of
// A_s over the contraction slice k = q DK/NQ .. + DK/NQ - 1, kept in registers and loaded
// DEPTH steps ahead (so a step waits on LDS only); it forms partial sums for the NQ columns
// from the LDS copy of H_in(s) (row r at r + r / (DK/NQ): the slices' rows fall on different
// banks), and DPP exchanges inside the group of NQ lanes leave lane q with column c0 + q:
// partner 7 - q (bit 2) for NQ = 8, then 3 - q (bit 1), then q ^ 1 (bit 0).  One barrier
// per step.  Eight columns per workgroup at DK = 128 halve the workgroups that read each
// A_s, against four.  FEW (nseg <= DEPTH): every step's operands come with the first loads,
// each segment's once.  H_in is stored in float32 [k][col].
template <int DK, int DV, bool FEW = false>
__global__ __launch_bounds__(DK >= 128 ? 8 * DK : 4 * DK) void seg_scan_kernel(FwdArgs a) {
  constexpr int NQ = DK >= 128 ? 8 : 4;       // contraction slices = columns per workgroup
  static_assert(DV % NQ == 0, "NQ state columns per workgroup");
  constexpr int KQ = DK / NQ;                 // contraction entries per thread
  constexpr int NF = KQ / 4;                  // float4 loads per step
  constexpr int NH = NQ / 4;                  // float4 per LDS row
  constexpr int DEPTH = NQ == 8 ? 4 : 8;      // steps loaded ahead (1024 threads: 128 VGPRs)
  constexpr int HS = DK + NQ;                 // skewed rows of the LDS copy
  __shared__ __align__(16) float4 sH[2][HS][NH];
  const int tid = threadIdx.x, i = tid / NQ, q = tid % NQ;
  const int pr = blockIdx.x, c0 = NQ * blockIdx.y, col = c0 + q;
  const int nseg = a.nseg;
  const float* A0 = a.Aagg + (size_t)pr * nseg * DK * DK + (size_t)i * DK + q * KQ;
  const float* B0 = a.Bagg + (size_t)pr * nseg * DK * DV + (size_t)i * DV + col;
  float* H0 = a.Hin + (size_t)pr * nseg * DK * DV + (size_t)i * DV + col;
  auto hrow = [](int r) { return r + r / KQ; };
  float h = a.S0 != nullptr ? a.S0[(size_t)pr * DK * DV + (size_t)i * DV + col] : 0.f;
  reinterpret_cast<float*>(&sH[0][hrow(i)][0])[q] = h;
  float4 ra[DEPTH][NF];
  float rb[DEPTH];
  auto fetch = [&](float4 (&x)[NF], float& b, int s) {
    const size_t sn = (size_t)(s < nseg ? s : nseg - 1);  // unconditional: waits stay exact
    const float4* src = reinterpret_cast<const float4*>(A0 + sn * DK * DK);
#pragma unroll
    for (int f = 0; f < NF; ++f) x[f] = src[f];
    b = B0[sn * DK * DV];
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (!FEW || d < nseg) fetch(ra[d], rb[d], d);
  __syncthreads();
  int cur = 0;
  for (int s0 = 0; s0 < nseg; s0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int s = s0 + d;
      if (s < nseg) {
        H0[(size_t)s * DK * DV] = h;
        float v[NQ];
#pragma unroll
        for (int c = 0; c < NQ; ++c) v[c] = 0.f;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const float am[4] = {ra[d][f].x, ra[d][f].y, ra[d][f].z, ra[d][f].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
              const float4 hv = sH[cur][hrow(q * KQ + 4 * f + e)][hh];
              v[4 * hh + 0] += am[e] * hv.x;
              v[4 * hh + 1] += am[e] * hv.y;
              v[4 * hh + 2] += am[e] * hv.z;
              v[4 * hh + 3] += am[e] * hv.w;
            }
          }
        }
        const float bv = rb[d];
        if constexpr (!FEW) fetch(ra[d], rb[d], s + DEPTH);
        // reduce-scatter over the NQ lanes: keep the half, then the pair, then the column
        float n4[4];
        if constexpr (NQ == 8) {
          const bool up = (q & 4) != 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) n4[j] = (up ? v[4 + j] : v[j]) + dpp_mov<0x141>(up ? v[j] : v[4 + j]);  // 7 - q
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) n4[j] = v[j];
        }
        const bool hi2 = (q & 2) != 0, hi1 = (q & 1) != 0;
        float n2[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // 3 - q for NQ = 8 (bits 1 and 0 both flip; bit 1 decides), q ^ 2 for NQ = 4
          const float recv = dpp_mov<NQ == 8 ? 0x1B : 0x4E>(hi2 ? n4[j] : n4[2 + j]);
          n2[j] = (hi2 ? n4[2 + j] : n4[j]) + recv;
        }
        h = (hi1 ? n2[1] : n2[0]) + dpp_mov<0xB1>(hi1 ? n2[0] : n2[1]) + bv;  // q ^ 1
        reinterpret_cast<float*>(&sH[cur ^ 1][hrow(i)][0])[q] = h;
        cur ^= 1;
        __syncthreads();
      }
    }
  }
  a.S_final[(size_t)pr * DK * DV + (size_t)i * DV + col] = h;
}

// o = O_loc + Qhat H_in(segment) for one chunk of one pair (float32 VALU).
template <class E, int DK, int DV, int C>
__global__ __launch_bounds__(256) void seg_fixup_kernel(FwdArgs a) {
  __shared__ float sH[DK * DV];
  __shared__ float sQh[C * (DK + 1)];
  const int tid = threadIdx.x, c = blockIdx.x, pr = blockIdx.y;
  const int seg = c / a.seg_chunks;
  const int t0 = c * C, nvalid = min(C, a.T - t0);
  const int Tpad = a.nch * C;
  const float* Hi = a.Hin + ((size_t)pr * a.nseg + seg) * DK * DV;
  const E* qh = reinterpret_cast<const E*>(a.Qhat) + ((size_t)pr * Tpad + t0) * DK;
  const E* ol = reinterpret_cast<const E*>(a.Oloc) + ((size_t)pr * Tpad + t0) * DV;
  E* o = reinterpret_cast<E*>(a.o) + ((size_t)pr * a.T + t0) * DV;
  for (int idx = tid; idx < DK * DV / 4; idx += 256)
    reinterpret_cast<float4*>(sH)[idx] = reinterpret_cast<const float4*>(Hi)[idx];
  for (int idx = tid; idx < C * DK; idx += 256) sQh[(idx / DK) * (DK + 1) + idx % DK] = to_f(qh[idx]);
  __syncthreads();
  for (int idx = tid; idx < nvalid * DV; idx += 256) {
    const int t = idx / DV, jj = idx % DV;
    float acc = to_f(ol[(size_t)t * DV + jj]);
    for (int kk = 0; kk < DK; ++kk) acc += sQh[t * (DK + 1) + kk] * sH[kk * DV + jj];
    o[(size_t)t * DV + jj] = from_f<E>(acc);
  }
}

// o = O_loc + Qhat H_in(segment) on MFMA, for bfloat16 I/O at d = 128 and 64-token
// chunks: bfloat16 operands (Qhat as stored, H_in rounded once, as the output itself is),
// float32 accumulation started from O_loc (stored in bfloat16).  One workgroup takes
// kFixupChunks consecutive chunks of a pair and stages H_in^T of their segment in LDS once
// (again only where a segment starts among them), with the contraction index permuted
// inside each 32-block (k = 32 kb + 16 h + 4 q + e at 32 kb + 8 q + 4 h + e) so a lane's
// 8-value operand (k0 + 4 q .. + 3 and k0 + 16 + 4 q .. + 3) is one 16-byte read.  Wave w
// takes token rows 16 w .. 16 w + 15 of each chunk and forms o^T = H_in^T Qhat^T + O_loc^T:
// lane (li, q) of tile vt holds value columns 16 vt + 4 q .. + 3 of token 16 w + li, so
// O_loc is read and o written 8 bytes at a time.  The next chunk's Qhat and O_loc
// fragments are loaded into a second register set while the current chunk is finished.
constexpr int kFixupChunks = 4;

template <int D, int C, bool HB16 = false>
__global__ __launch_bounds__(256) void seg_fixup_mfma_kernel(FwdArgs a) {
  static_assert(D == 128 && C == 64, "written for d = 128 and 64-token chunks");
  constexpr int LH = D + 8;  // row stride of the staged H_in^T (bfloat16 elements)
  __shared__ __align__(16) bf16_t sHt[D * LH];
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), q = l >> 4, li = l & 15;
  const int pr = blockIdx.y;
  const int c_lo = blockIdx.x * kFixupChunks, c_hi = min(a.nch, c_lo + kFixupChunks);
  const int Tpad = a.nch * C;
  const int row = 16 * w + li;
  // this wave's Qhat rows (B operands, 4 blocks of 32 along k) and O_loc entries of one
  // chunk, in two register sets: the next chunk's are loaded while the current one is
  // finished.  Chunk indices are clamped to the last (padded) chunk, so every load is in
  // bounds and none is conditional.
  const bf16_t* Qb = reinterpret_cast<const bf16_t*>(a.Qhat) + ((size_t)pr * Tpad + row) * D;
  const bf16_t* Ob = reinterpret_cast<const bf16_t*>(a.Oloc) + ((size_t)pr * Tpad + row) * D;
  bf16x4 qx[2][D / 32][2], ox[2][D / 16];
  auto fetch = [&](int set, int c) {
    const size_t off = (size_t)min(c, a.nch - 1) * C * D;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      qx[set][kb][0] = *reinterpret_cast<const bf16x4*>(Qb + off + 32 * kb + 4 * q);
      qx[set][kb][1] = *reinterpret_cast<const bf16x4*>(Qb + off + 32 * kb + 16 + 4 * q);
    }
#pragma unroll
    for (int vt = 0; vt < D / 16; ++vt) ox[set][vt] = *reinterpret_cast<const bf16x4*>(Ob + off + 16 * vt + 4 * q);
  };
  fetch(0, c_lo);
  int staged = -1;
#pragma unroll
  for (int i = 0; i < kFixupChunks; ++i) {
    const int c = c_lo + i, cur = i & 1;
    if (c < c_hi) {
      const int seg = c / a.seg_chunks;  // the same for every thread of the workgroup
      const int t0 = c * C, nvalid = min(C, a.T - t0);
      if (seg != staged) {
        if (staged >= 0) __syncthreads();  // every read of the previous segment's H_in is done
        if constexpr (HB16) {  // already bfloat16 [col][k'] (the scan's layout): 16-byte copies
          const uint4* Hb = reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.Hin) +
                                                           ((size_t)pr * a.nseg + seg) * D * D);
          for (int idx = tid; idx < D * D / 8; idx += 256)
            *reinterpret_cast<uint4*>(&sHt[(idx >> 4) * LH + 8 * (idx & 15)]) = Hb[idx];
        } else {
          const float* Hi = a.Hin + ((size_t)pr * a.nseg + seg) * D * D;  // [k][col]
          for (int idx = tid; idx < D * D; idx += 256) {
            const int k = idx / D, col = idx % D;
            const int kp = (k & ~31) | ((k & 12) << 1) | ((k & 16) >> 2) | (k & 3);
            sHt[col * LH + kp] = (bf16_t)Hi[idx];
          }
        }
        __syncthreads();
        staged = seg;
      }
      // after the staging, whose wait would otherwise also drain these loads
      if (i + 1 < kFixupChunks) fetch(cur ^ 1, c + 1);
      f32x4 acc[D / 16];
#pragma unroll
      for (int vt = 0; vt < D / 16; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[vt][r] = (float)ox[cur][vt][r];
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8 bq = __builtin_shufflevector(qx[cur][kb][0], qx[cur][kb][1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int vt = 0; vt < D / 16; ++vt)
          acc[vt] = mfma(*reinterpret_cast<const bf16x8*>(&sHt[(16 * vt + li) * LH + 32 * kb + 8 * q]), bq, acc[vt]);
      }
      if (row < nvalid) {
        bf16_t* o = reinterpret_cast<bf16_t*>(a.o) + ((size_t)pr * a.T + t0 + row) * D;
#pragma unroll
        for (int vt = 0; vt < D / 16; ++vt) {
          bf16x4 y;
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = (bf16_t)acc[vt][r];
          *reinterpret_cast<bf16x4*>(o + 16 * vt + 4 * q) = y;
        }
      }
    }
  }
}

}  // namespace prism
