// prism_fast.h - the bfloat16 segment sweep for head dim 64 (gfx950).
//
// Same mathematics as seg_local_kernel (see prism_kernels.h), organised for
// throughput on CDNA4:
//   * one workgroup (4 waves) per segment, one segment per CU;
//   * inputs staged in LDS with 16-byte coalesced loads, rank-L inputs streamed
//     one refinement step at a time through two LDS slots;
//   * mixed ownership of the 64-token chunk: wave w owns token rows
//     16w..16w+15 for the products that contract over tokens j <= i (masked
//     Gram tiles stay in registers and feed the next MFMA directly as its A
//     operand), and owns the 16 value / key columns 16w..16w+15 for the
//     triangular solve, the state H and the segment operator A_acc (no
//     cross-wave traffic for those);
//   * the 16x16 diagonal blocks of (I + M)^-1 are inverted in registers by the
//     product (I + Y)(I + Y^2)(I + Y^4)(I + Y^8), Y = -M_ii strictly lower
//     (exact for a nilpotent Y), with float32 MFMAs;
//   * the block forward substitution for Uc and Wc runs wave-locally per
//     column block with 16-deep bf16 MFMAs.
#pragma once
#include "prism_kernels.h"

namespace prism {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}

// Z = A * B for 16x16 float32 tiles, A given by the tile of A^T, B by its tile.
__device__ __forceinline__ f32x4 mm16_f32(const f32x4& At, const f32x4& Bt) {
  f32x4 acc = zero4();
#pragma unroll
  for (int r = 0; r < 4; ++r) acc = mfma(At[r], Bt[r], acc);
  return acc;
}

__device__ __forceinline__ f32x4 plus_identity(f32x4 x) {
  const int l = lane_id(), g4 = (l >> 4) * 4, li = l & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] += (g4 + r == li) ? 1.f : 0.f;
  return x;
}

__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4& x) {
  bf16x4 y;
#pragma unroll
  for (int r = 0; r < 4; ++r) y[r] = (bf16_t)x[r];
  return y;
}

__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS plan of the fast sweep (bytes).
template <int D, int C>
struct FastLds {
  static constexpr int LD = D + 8;    // row stride of [token][d] arrays (bf16)
  static constexpr int LDC = C + 8;   // row stride of [d][token] arrays (bf16)
  static constexpr int LDT = 16 + 8;  // row stride of a 16x16 diagonal inverse block
  static constexpr size_t szTD = (size_t)C * LD * 2;   // [C][LD]
  static constexpr size_t szDT = (size_t)D * LDC * 2;  // [D][LDC]
  static constexpr size_t szDD = (size_t)D * LD * 2;   // [D][LD]
  static constexpr size_t oQ = 0;
  static constexpr size_t oK = oQ + szTD;
  static constexpr size_t oKt = oK + szTD;
  static constexpr size_t oHt = oKt + szDT;
  static constexpr size_t oAt = oHt + szDD;
  static constexpr size_t oM = oAt + szDD;
  static constexpr size_t oTd = oM + (size_t)C * LDC * 2;
  static constexpr size_t oV = oTd + (size_t)(C / 16) * 16 * LDT * 2;
  static constexpr size_t oGate = oV + (size_t)(C + 3) * LD * 2;
  static constexpr size_t nGate = 5 * C + 8 * C;
  // two slots of (U_l [C][LD], gamma_l [C][LD], R_l^T [D][LDC]); after the
  // refinement loop the region holds V'^T, Wc, Wc^T and E^T.
  static constexpr size_t oSlot = oGate + nGate * 4;
  static constexpr size_t szSlot = 2 * szTD + szDT;
  static constexpr size_t total = oSlot + 2 * szSlot;
  static_assert(szTD + 2 * szDT <= szSlot, "Wc, Wc^T and E^T must fit one slot");
  static constexpr bool fits = total <= 160 * 1024;
};

// Row-major [ROWS][D] bf16 tile load from global (16-byte pieces) into LDS with
// row stride LD.  Tile row r is global row row0 + r of `src` (row stride
// `row_stride` elements); rows outside [0, hi) read as zero.  Optionally also
// writes the transposed copy dstT[c][r] (row stride LDC).
template <int D, int ROWS, int LD, int LDC>
__device__ __forceinline__ void load_rows(bf16_t* dst, bf16_t* dstT, const bf16_t* src, size_t row_stride,
                                          int row0, int hi) {
  constexpr int PER_ROW = D / 8;
  constexpr int NP = ROWS * PER_ROW;
  constexpr int NIT = (NP + 255) / 256;
  uint4 buf[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int idx = threadIdx.x + 256 * it;
    const int row = idx / PER_ROW, cv = (idx % PER_ROW) * 8;
    const int gr = row0 + row;
    const bool ok = idx < NP && gr >= 0 && gr < hi;
    const size_t rc = ok ? (size_t)gr : 0;
    uint4 x = *reinterpret_cast<const uint4*>(src + rc * row_stride + cv);
    buf[it] = ok ? x : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int idx = threadIdx.x + 256 * it;
    if (idx >= NP) break;
    const int row = idx / PER_ROW, cv = (idx % PER_ROW) * 8;
    *reinterpret_cast<uint4*>(dst + row * LD + cv) = buf[it];
    if (dstT != nullptr) {
      const bf16_t* e = reinterpret_cast<const bf16_t*>(&buf[it]);
#pragma unroll
      for (int j = 0; j < 8; ++j) dstT[(cv + j) * LDC + row] = e[j];
    }
  }
}

// B operand (16-deep, k = tokens 16*kb + 4g..4g+3, n = column li) from a [col][token]
// LDS array (row stride ldc); optionally scaled by s[k].
__device__ __forceinline__ bf16x4 ldsT_b4(const bf16_t* T, int ldc, int col0, int k0) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x4*>(T + (col0 + (l & 15)) * ldc + k0 + 4 * (l >> 4));
}

template <int D, int C>
__global__ __launch_bounds__(256, 1) void seg_fast_kernel(FwdArgs a) {
  using Ly = FastLds<D, C>;
  constexpr int LD = Ly::LD, LDC = Ly::LDC, LDT = Ly::LDT;
  constexpr int MT = C / 16;  // token blocks = waves
  constexpr int KT = D / 16;  // column blocks = waves
  static_assert(MT == 4 && KT == 4, "the fast sweep maps 4 waves to 4 token blocks and 4 column blocks");
  __shared__ __align__(16) unsigned char smem[Ly::total];
  bf16_t* sQ = reinterpret_cast<bf16_t*>(smem + Ly::oQ);
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem + Ly::oK);
  bf16_t* sKt = reinterpret_cast<bf16_t*>(smem + Ly::oKt);
  bf16_t* sHt = reinterpret_cast<bf16_t*>(smem + Ly::oHt);
  bf16_t* sAt = reinterpret_cast<bf16_t*>(smem + Ly::oAt);
  bf16_t* sM = reinterpret_cast<bf16_t*>(smem + Ly::oM);
  bf16_t* sTd = reinterpret_cast<bf16_t*>(smem + Ly::oTd);
  bf16_t* sV = reinterpret_cast<bf16_t*>(smem + Ly::oV);  // rows t0-3 .. t0+C-1
  float* sB = reinterpret_cast<float*>(smem + Ly::oGate);
  float* sG = sB + C;
  float* sD = sG + C;
  float* sBeta = sD + C;
  float* sBG = sBeta + C;
  float* sAlpha = sBG + C;  // [C][8]
  unsigned char* slot0 = smem + Ly::oSlot;

  const int w = wave_id(), l = lane_id(), g = l >> 4, g4 = g * 4, li = l & 15;
  const int seg = blockIdx.x, pr = blockIdx.y;
  const int hd = pr % a.H;
  const int T = a.T, L = a.L, Lm1 = L - 1;
  const int c_begin = seg * a.seg_chunks;
  const int c_end = min(a.nch, c_begin + a.seg_chunks);
  const int Tpad = a.nch * C;
  const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q) + (size_t)pr * T * D;
  const bf16_t* k = reinterpret_cast<const bf16_t*>(a.k) + (size_t)pr * T * D;
  const bf16_t* v = reinterpret_cast<const bf16_t*>(a.v) + (size_t)pr * T * D;
  const bf16_t* u = L > 1 ? reinterpret_cast<const bf16_t*>(a.u) + (size_t)pr * T * Lm1 * D : nullptr;
  const bf16_t* gam = L > 1 ? reinterpret_cast<const bf16_t*>(a.gamma) + (size_t)pr * T * Lm1 * D : nullptr;
  const float* gg = a.g + (size_t)pr * T;
  const float* bb = a.beta + (size_t)pr * T;
  const float* al = L > 1 ? a.alpha + (size_t)pr * T * L : nullptr;
  const float* cw = L > 1 ? a.conv_w + (size_t)hd * 4 * D : nullptr;
  bf16_t* qhat_out = reinterpret_cast<bf16_t*>(a.Qhat);

  // conv taps for this lane's value columns (column block vt, lane column li)
  float taps[KT][4];
#pragma unroll
  for (int vt = 0; vt < KT; ++vt)
#pragma unroll
    for (int j = 0; j < 4; ++j) taps[vt][j] = L > 1 ? cw[j * D + 16 * vt + li] : 0.f;

  // column-owned state: H(:, w) and A_acc(:, w), tiles over row blocks kt
  f32x4 Hs[KT], As[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    Hs[kt] = zero4();
    f32x4 t = zero4();
    if (kt == w) {
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = (g4 + r == li) ? 1.f : 0.f;
    }
    As[kt] = t;
  }
  // LDS copies of the state operands: H^T = 0, A_acc^T = I
  for (int idx = threadIdx.x; idx < D * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    sHt[r * LD + c] = (bf16_t)0.f;
    sAt[r * LD + c] = (bf16_t)(r == c ? 1.f : 0.f);
  }

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * C;
    const int nvalid = min(C, T - t0);
    // ---- loads: Q, K (+K^T), V with a 3-row halo, gates ------------------------------
    const int hi = t0 + nvalid;
    load_rows<D, C, LD, LDC>(sQ, nullptr, q, D, t0, hi);
    load_rows<D, C, LD, LDC>(sK, sKt, k, D, t0, hi);
    load_rows<D, C + 3, LD, LDC>(sV, nullptr, v, D, t0 - 3, hi);
    if (w == 0) {
      const bool ok = l < nvalid;
      float lam = ok ? __logf(gg[t0 + min(l, nvalid - 1)]) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        float y = __shfl_up(lam, off);
        if (l >= off) lam += y;
      }
      const float blast = __shfl(lam, C - 1);
      const float be = ok ? bb[t0 + min(l, nvalid - 1)] : 0.f;
      const float G = __expf(lam);
      sB[l] = lam;
      sG[l] = G;
      sD[l] = __expf(blast - lam);
      sBeta[l] = be;
      sBG[l] = be * G;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        sAlpha[l * 8 + j] = (ok && j < L && L > 1) ? al[(size_t)(t0 + min(l, nvalid - 1)) * L + j] : 0.f;
    }
    __syncthreads();

    // ---- row-owned prologue: V' = V, residual r0 = V - anchor (tiles: rows 16w.., cols 16vt..)
    const int i0 = 16 * w;
    f32x4 Vp[KT], Oc[KT], Rr[KT];
#pragma unroll
    for (int vt = 0; vt < KT; ++vt) {
      const int col = 16 * vt + li;
      float vv[7];
#pragma unroll
      for (int j = 0; j < 7; ++j) vv[j] = to_f(sV[(i0 + g4 + j) * LD + col]);  // rows t-3..t+3 (+3 halo offset)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = vv[r + 3];
        Vp[vt][r] = x;
        const float anc = taps[vt][0] * vv[r] + taps[vt][1] * vv[r + 1] + taps[vt][2] * vv[r + 2] +
                          taps[vt][3] * vv[r + 3];
        Rr[vt][r] = x - anc;
      }
      Oc[vt] = zero4();
    }
    // ---- P(w, j) = lower(Gam * Q K^T) as chained A fragments; M(w, j) -> LDS -------------
    bf16x8 Pa[2];
    {
      f32x4 praw[MT], mraw[MT];
#pragma unroll
      for (int jt = 0; jt < MT; ++jt) {
        praw[jt] = zero4();
        mraw[jt] = zero4();
        if (jt <= w) {
          mm_ll<bf16_t>(praw[jt], sK, LD, 16 * jt, sQ, LD, i0, D);   // (K_j Q_w^T): [j][i]
          mm_ll<bf16_t>(mraw[jt], sK, LD, i0, sK, LD, 16 * jt, D);   // (K_w K_j^T): [i][j]
        }
      }
      const float bi_lane = sB[i0 + li];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int jt = 2 * kb + h;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jj = 16 * jt + g4 + r, ii = i0 + li;
            const float val = (jt <= w && jj <= ii) ? __expf(bi_lane - sB[jj]) * praw[jt][r] : 0.f;
            Pa[kb][4 * h + r] = (bf16_t)val;
          }
        }
      }
      // M tiles (row-major [i][j], strict lower, beta_i Gam_ij K_i.K_j)
#pragma unroll
      for (int jt = 0; jt < MT; ++jt) {
        if (jt <= w) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int ii = i0 + g4 + r, jj = 16 * jt + li;
            const float val = (jj < ii) ? sBeta[ii] * __expf(sB[ii] - sB[jj]) * mraw[jt][r] : 0.f;
            sM[ii * LDC + jj] = (bf16_t)val;
          }
        }
      }
      // diagonal block inverse: Y = -M_ww (and Y^T, from the symmetric raw Gram tile)
      f32x4 Y, Yt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = i0 + g4 + r, jj = i0 + li;
        const float raw = mraw[w][r];
        Y[r] = (jj < ii) ? -sBeta[ii] * __expf(sB[ii] - sB[jj]) * raw : 0.f;
        Yt[r] = (ii < jj) ? -sBeta[jj] * __expf(sB[jj] - sB[ii]) * raw : 0.f;
      }
      const f32x4 Y2 = mm16_f32(Yt, Y), Y2t = mm16_f32(Y, Yt);
      const f32x4 Y4 = mm16_f32(Y2t, Y2), Y4t = mm16_f32(Y2, Y2t);
      const f32x4 Y8 = mm16_f32(Y4t, Y4);
      f32x4 Pt = plus_identity(Yt);
      Pt = mm16_f32(plus_identity(Y2), Pt);
      Pt = mm16_f32(plus_identity(Y4), Pt);
      Pt = mm16_f32(plus_identity(Y8), Pt);  // Pt = T_ww^T
      // T_ww row-major: T[li][g4 + r] = Pt[r]
      bf16x4 tv = to_bf16x4(Pt);
      *reinterpret_cast<bf16x4*>(sTd + (w * 16 + li) * LDT + g4) = tv;
    }

    // ---- rank-L injection, one refinement step at a time --------------------------------
    f32x4 HB[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) HB[kt] = zero4();
    for (int lr = 1; lr < L; ++lr) {
      unsigned char* slot = slot0 + (size_t)((lr - 1) & 1) * Ly::szSlot;
      bf16_t* sU = reinterpret_cast<bf16_t*>(slot);
      bf16_t* sGm = reinterpret_cast<bf16_t*>(slot + Ly::szTD);
      bf16_t* sRt = reinterpret_cast<bf16_t*>(slot + 2 * Ly::szTD);
      load_rows<D, C, LD, LDC>(sU, nullptr, u + (size_t)(lr - 1) * D, (size_t)Lm1 * D, t0, hi);
      load_rows<D, C, LD, LDC>(sGm, nullptr, gam + (size_t)(lr - 1) * D, (size_t)Lm1 * D, t0, hi);
      __syncthreads();
      // residual step and R_l = alpha_l r_l for rows 16w.., written transposed
#pragma unroll
      for (int vt = 0; vt < KT; ++vt) {
        const int col = 16 * vt + li;
        bf16x4 rv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = i0 + g4 + r;
          const float gm = to_f(sGm[t * LD + col]);
          const float x = Rr[vt][r] * (1.f - sAlpha[t * 8 + lr - 1] * gm);
          Rr[vt][r] = x;
          rv[r] = (bf16_t)(sAlpha[t * 8 + lr] * x);
        }
        *reinterpret_cast<bf16x4*>(sRt + col * LDC + i0 + g4) = rv;
      }
      __syncthreads();
      // row-owned: X1 = -strict(Gam * K U^T), X2 = lower(Gam * Q U^T) as A fragments
      {
        f32x4 x1raw[MT], x2raw[MT];
#pragma unroll
        for (int jt = 0; jt < MT; ++jt) {
          x1raw[jt] = zero4();
          x2raw[jt] = zero4();
          if (jt <= w) {
            mm_ll<bf16_t>(x1raw[jt], sU, LD, 16 * jt, sK, LD, i0, D);  // (U_j K_w^T): [j][i]
            mm_ll<bf16_t>(x2raw[jt], sU, LD, 16 * jt, sQ, LD, i0, D);  // (U_j Q_w^T): [j][i]
          }
        }
        const float bi_lane = sB[i0 + li];
        bf16x8 X1a[2], X2a[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int jt = 2 * kb + h;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int jj = 16 * jt + g4 + r, ii = i0 + li;
              const float gm = (jt <= w && jj <= ii) ? __expf(bi_lane - sB[jj]) : 0.f;
              X1a[kb][4 * h + r] = (bf16_t)((jj < ii) ? -gm * x1raw[jt][r] : 0.f);
              X2a[kb][4 * h + r] = (bf16_t)(gm * x2raw[jt][r]);
            }
          }
        const int nkb = (w + 2) / 2;
#pragma unroll
        for (int vt = 0; vt < KT; ++vt) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (kb < nkb) {
              const bf16x8 rb = cat8(ldsT_b4(sRt, LDC, 16 * vt, 32 * kb), ldsT_b4(sRt, LDC, 16 * vt, 32 * kb + 16));
              Vp[vt] = mfma(X1a[kb], rb, Vp[vt]);
              Oc[vt] = mfma(X2a[kb], rb, Oc[vt]);
            }
          }
        }
      }
      // column-owned: HB(:, w) += U^T diag(D) R(:, w)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bf16x8 ua;
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            const int tk = 32 * kb + ((p >> 2) << 4) + g4 + (p & 3);
            ua[p] = (bf16_t)(sD[tk] * to_f(sU[tk * LD + 16 * kt + li]));
          }
          const bf16x8 rb = cat8(ldsT_b4(sRt, LDC, 16 * w, 32 * kb), ldsT_b4(sRt, LDC, 16 * w, 32 * kb + 16));
          HB[kt] = mfma(ua, rb, HB[kt]);
        }
      }
    }

    // ---- exchange beta * V' (transposed) for the column-owned solve -------------------
    // After the refinement loop: slot F (not used by the last step, so free while other
    // waves finish that step) takes V'^T; slot U (used by the last step, free after the
    // next barrier) takes Wc, Wc^T and E^T.
    const int slotF = (L - 1) & 1, slotU = slotF ^ 1;
    bf16_t* sVt = reinterpret_cast<bf16_t*>(slot0 + (size_t)slotF * Ly::szSlot);
    bf16_t* sWc = reinterpret_cast<bf16_t*>(slot0 + (size_t)slotU * Ly::szSlot);
    bf16_t* sWct = sWc + C * LD;
    bf16_t* sEt = sWct + D * LDC;
#pragma unroll
    for (int vt = 0; vt < KT; ++vt) {
      bf16x4 x;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = (bf16_t)(sBeta[i0 + g4 + r] * Vp[vt][r]);
      *reinterpret_cast<bf16x4*>(sVt + (16 * vt + li) * LDC + i0 + g4) = x;
    }
    __syncthreads();

    // ---- column-owned block forward substitution: (I + M) [Uc | Wc] = [beta V' | beta G K]
    f32x4 Uc[MT], Wc[MT];
    {
#pragma unroll
      for (int side = 0; side < 2; ++side) {
        f32x4 X[MT];
#pragma unroll
        for (int it = 0; it < MT; ++it) {
          f32x4 acc;
          if (side == 0) {
            const bf16x4 y = ldsT_b4(sVt, LDC, 16 * w, 16 * it);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = (float)y[r];
          } else {
            const bf16x4 y = ldsT_b4(sKt, LDC, 16 * w, 16 * it);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = sBG[16 * it + g4 + r] * (float)y[r];
          }
          f32x4 s = zero4();
#pragma unroll
          for (int kt = 0; kt < MT; ++kt) {
            if (kt < it) {
              const bf16x4 am = *reinterpret_cast<const bf16x4*>(sM + (16 * it + li) * LDC + 16 * kt + g4);
              s = mfma16(am, to_bf16x4(X[kt]), s);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] -= s[r];
          const bf16x4 at = *reinterpret_cast<const bf16x4*>(sTd + (16 * it + li) * LDT + g4);
          X[it] = mfma16(at, to_bf16x4(acc), zero4());
        }
#pragma unroll
        for (int it = 0; it < MT; ++it) {
          if (side == 0) Uc[it] = X[it];
          else Wc[it] = X[it];
        }
      }
    }
    // Wc (column block w) to LDS, row-major and transposed
    {
#pragma unroll
      for (int it = 0; it < MT; ++it) {
        bf16x4 x = to_bf16x4(Wc[it]);
#pragma unroll
        for (int r = 0; r < 4; ++r) sWc[(16 * it + g4 + r) * LD + 16 * w + li] = x[r];
        *reinterpret_cast<bf16x4*>(sWct + (16 * w + li) * LDC + 16 * it + g4) = x;
      }
    }
    __syncthreads();

    // ---- column-owned: E = Uc - Wc H(:, w),  WA = Wc A_acc(:, w) -------------------------
    f32x4 E[MT], WA[MT];
    {
      bf16x8 hb[2], ab[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        hb[kb] = cat8(to_bf16x4(Hs[2 * kb]), to_bf16x4(Hs[2 * kb + 1]));
        ab[kb] = cat8(to_bf16x4(As[2 * kb]), to_bf16x4(As[2 * kb + 1]));
      }
#pragma unroll
      for (int it = 0; it < MT; ++it) {
        f32x4 wh = zero4(), wa = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16_t* ar = sWc + (16 * it + li) * LD + 32 * kb + g4;
          const bf16x8 af = cat8(*reinterpret_cast<const bf16x4*>(ar), *reinterpret_cast<const bf16x4*>(ar + 16));
          wh = mfma(af, hb[kb], wh);
          wa = mfma(af, ab[kb], wa);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) E[it][r] = Uc[it][r] - wh[r];
        WA[it] = wa;
        *reinterpret_cast<bf16x4*>(sEt + (16 * w + li) * LDC + 16 * it + g4) = to_bf16x4(E[it]);
      }
    }
    // ---- row-owned: O += diag(G) Q H;  Qtilde^T = (diag(G) Q)^T - Wc^T P^T;  Qhat^T = A_acc^T Qtilde^T
    {
      const float Gr0 = sG[i0 + g4 + 0], Gr1 = sG[i0 + g4 + 1], Gr2 = sG[i0 + g4 + 2], Gr3 = sG[i0 + g4 + 3];
#pragma unroll
      for (int vt = 0; vt < KT; ++vt) {
        f32x4 qh = zero4();
        mm_ll<bf16_t>(qh, sQ, LD, i0, sHt, LD, 16 * vt, D);
        Oc[vt][0] += Gr0 * qh[0];
        Oc[vt][1] += Gr1 * qh[1];
        Oc[vt][2] += Gr2 * qh[2];
        Oc[vt][3] += Gr3 * qh[3];
      }
      const float Gi = sG[i0 + li];
      f32x4 Qt[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const bf16x4 qv = *reinterpret_cast<const bf16x4*>(sQ + (i0 + li) * LD + 16 * kt + g4);
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = Gi * (float)qv[r];
        f32x4 pw = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16_t* ar = sWct + (16 * kt + li) * LDC + 32 * kb + g4;
          const bf16x8 af = cat8(*reinterpret_cast<const bf16x4*>(ar), *reinterpret_cast<const bf16x4*>(ar + 16));
          pw = mfma(af, Pa[kb], pw);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] -= pw[r];
        Qt[kt] = acc;  // tile (dk rows 16kt.., tokens 16w..)
      }
      bf16x8 qb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) qb[kb] = cat8(to_bf16x4(Qt[2 * kb]), to_bf16x4(Qt[2 * kb + 1]));
      bf16_t* qh_out = qhat_out + ((size_t)pr * Tpad + t0 + i0) * D;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16_t* ar = sAt + (16 * kt + li) * LD + 32 * kb + g4;
          const bf16x8 af = cat8(*reinterpret_cast<const bf16x4*>(ar), *reinterpret_cast<const bf16x4*>(ar + 16));
          acc = mfma(af, qb[kb], acc);
        }
        // acc = Qhat^T tile (dk rows 16kt.., tokens 16w..): Qhat[li][16kt + g4 + r]
        *reinterpret_cast<bf16x4*>(qh_out + (size_t)li * D + 16 * kt + g4) = to_bf16x4(acc);
      }
    }
    __syncthreads();

    // ---- row-owned: O += P E, write O_loc ---------------------------------------------------
    {
      float* oloc = a.Oloc + ((size_t)pr * Tpad + t0 + i0) * D;
      const int nkb = (w + 2) / 2;
#pragma unroll
      for (int vt = 0; vt < KT; ++vt) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb < nkb) {
            const bf16x8 eb = cat8(ldsT_b4(sEt, LDC, 16 * vt, 32 * kb), ldsT_b4(sEt, LDC, 16 * vt, 32 * kb + 16));
            Oc[vt] = mfma(Pa[kb], eb, Oc[vt]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) oloc[(size_t)(g4 + r) * D + 16 * vt + li] = Oc[vt][r];
      }
    }
    // ---- column-owned: H(:, w) = G_C H + K^T D E + HB;  A_acc(:, w) = G_C A_acc - K^T D WA
    {
      const float GC = sG[C - 1];
      bf16x8 eb[2], wb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        eb[kb] = cat8(to_bf16x4(E[2 * kb]), to_bf16x4(E[2 * kb + 1]));
        wb[kb] = cat8(to_bf16x4(WA[2 * kb]), to_bf16x4(WA[2 * kb + 1]));
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        f32x4 he = zero4(), aw = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bf16x8 kd;
          const bf16_t* ar = sKt + (16 * kt + li) * LDC + 32 * kb + g4;
          const bf16x4 k0 = *reinterpret_cast<const bf16x4*>(ar);
          const bf16x4 k1 = *reinterpret_cast<const bf16x4*>(ar + 16);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            kd[r] = (bf16_t)(sD[32 * kb + g4 + r] * (float)k0[r]);
            kd[4 + r] = (bf16_t)(sD[32 * kb + 16 + g4 + r] * (float)k1[r]);
          }
          he = mfma(kd, eb[kb], he);
          aw = mfma(kd, wb[kb], aw);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Hs[kt][r] = GC * Hs[kt][r] + he[r] + HB[kt][r];
          As[kt][r] = GC * As[kt][r] - aw[r];
        }
      }
    }
    __syncthreads();
    // new H^T and A_acc^T into LDS for the next chunk
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      *reinterpret_cast<bf16x4*>(sHt + (16 * w + li) * LD + 16 * kt + g4) = to_bf16x4(Hs[kt]);
      *reinterpret_cast<bf16x4*>(sAt + (16 * w + li) * LD + 16 * kt + g4) = to_bf16x4(As[kt]);
    }
  }

  // ---- segment operator (float32) ---------------------------------------------------------
  float* Ag = a.Aagg + ((size_t)pr * a.nseg + seg) * D * D;
  float* Bg = a.Bagg + ((size_t)pr * a.nseg + seg) * D * D;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Ag[(16 * kt + g4 + r) * D + 16 * w + li] = As[kt][r];
      Bg[(16 * kt + g4 + r) * D + 16 * w + li] = Hs[kt][r];
    }
}

// Inter-segment recurrence H_in(s+1) = A_s H_in(s) + B_s (float32), JW state
// columns per workgroup; each thread owns one (row, column) and prefetches the
// next segment's operator row while the current step runs.
template <int DK, int DV>
__global__ __launch_bounds__(256) void seg_scan_fast_kernel(FwdArgs a) {
  constexpr int JW = 256 / DK;
  __shared__ __align__(16) float sH[2][JW][DK];
  const int tid = threadIdx.x, pr = blockIdx.x, c0 = JW * blockIdx.y;
  const int i = tid / JW, j = tid % JW;
  sH[0][j][i] = 0.f;
  float4 arow[DK / 4], nrow[DK / 4];
  const float* A0 = a.Aagg + (size_t)pr * a.nseg * DK * DK;
  const float* B0 = a.Bagg + (size_t)pr * a.nseg * DK * DV;
#pragma unroll
  for (int q = 0; q < DK / 4; ++q) arow[q] = reinterpret_cast<const float4*>(A0 + (size_t)i * DK)[q];
  float bcur = B0[(size_t)i * DV + c0 + j];
  __syncthreads();
  int cur = 0;
  for (int s = 0; s < a.nseg; ++s) {
    float* Hi = a.Hin + ((size_t)pr * a.nseg + s) * DK * DV;
    Hi[(size_t)i * DV + c0 + j] = sH[cur][j][i];
    const int sn = s + 1 < a.nseg ? s + 1 : s;
    const float* An = A0 + (size_t)sn * DK * DK;
#pragma unroll
    for (int q = 0; q < DK / 4; ++q) nrow[q] = reinterpret_cast<const float4*>(An + (size_t)i * DK)[q];
    const float bnext = B0[(size_t)sn * DK * DV + (size_t)i * DV + c0 + j];
    float acc = bcur;
    const float4* hcol = reinterpret_cast<const float4*>(&sH[cur][j][0]);
#pragma unroll
    for (int q = 0; q < DK / 4; ++q) {
      const float4 hv = hcol[q];
      acc += arow[q].x * hv.x + arow[q].y * hv.y + arow[q].z * hv.z + arow[q].w * hv.w;
    }
    sH[cur ^ 1][j][i] = acc;
    __syncthreads();
    cur ^= 1;
#pragma unroll
    for (int q = 0; q < DK / 4; ++q) arow[q] = nrow[q];
    bcur = bnext;
  }
  a.S_final[(size_t)pr * DK * DV + (size_t)i * DV + c0 + j] = sH[cur][j][i];
}

// o = O_loc + Qhat H_in(segment) with MFMA; one workgroup per chunk, wave w owns
// token rows 16w.., output staged in LDS for 16-byte stores.
template <int D, int C>
__global__ __launch_bounds__(256) void seg_fixup_fast_kernel(FwdArgs a) {
  constexpr int LD = D + 8;
  __shared__ __align__(16) bf16_t sHt[D * LD];
  __shared__ __align__(16) bf16_t sO[C * LD];
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), g4 = (l >> 4) * 4, li = l & 15;
  const int c = blockIdx.x, pr = blockIdx.y;
  const int seg = c / a.seg_chunks;
  const int t0 = c * C, nvalid = min(C, a.T - t0);
  const int Tpad = a.nch * C;
  const float* Hi = a.Hin + ((size_t)pr * a.nseg + seg) * D * D;
  for (int idx = tid; idx < D * D; idx += 256) {
    const int kk = idx / D, jj = idx % D;
    sHt[jj * LD + kk] = (bf16_t)Hi[idx];
  }
  __syncthreads();
  const bf16_t* qh = reinterpret_cast<const bf16_t*>(a.Qhat) + ((size_t)pr * Tpad + t0 + 16 * w) * D;
  const float* ol = a.Oloc + ((size_t)pr * Tpad + t0 + 16 * w) * D;
  bf16x8 af[D / 32];
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) {
    const bf16_t* ar = qh + (size_t)li * D + 32 * kb + g4;
    af[kb] = cat8(*reinterpret_cast<const bf16x4*>(ar), *reinterpret_cast<const bf16x4*>(ar + 16));
  }
#pragma unroll
  for (int vt = 0; vt < D / 16; ++vt) {
    f32x4 acc;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = ol[(size_t)(g4 + r) * D + 16 * vt + li];
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      const bf16_t* br = sHt + (16 * vt + li) * LD + 32 * kb + g4;
      const bf16x8 bf = cat8(*reinterpret_cast<const bf16x4*>(br), *reinterpret_cast<const bf16x4*>(br + 16));
      acc = mfma(af[kb], bf, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sO[(16 * w + g4 + r) * LD + 16 * vt + li] = (bf16_t)acc[r];
  }
  __syncthreads();
  bf16_t* o = reinterpret_cast<bf16_t*>(a.o) + ((size_t)pr * a.T + t0) * D;
  constexpr int PER_ROW = D / 8;
  for (int idx = tid; idx < nvalid * PER_ROW; idx += 256) {
    const int row = idx / PER_ROW, cv = (idx % PER_ROW) * 8;
    *reinterpret_cast<uint4*>(o + (size_t)row * D + cv) = *reinterpret_cast<const uint4*>(sO + row * LD + cv);
  }
}

}  // namespace prism
