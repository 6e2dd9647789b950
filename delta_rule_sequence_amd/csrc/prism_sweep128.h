// prism_sweep128.h - the bfloat16 segment sweep for head dim 128 (gfx950).
//
// Same chunked UT / WY mathematics as seg_local_kernel (prism_kernels.h) and the d = 64
// sweep (prism_sweep8.h): per 64-token chunk the gated delta rule with the rank-L writes
// folded in (PRISM reading notes, sections 2.2-2.3; PRISM summary page, "architecture"
// section), carried over the chunks of a segment with the segment operator A_acc.
// Organisation for CDNA4 at d = 128:
//
//   * two workgroups per segment: workgroup half h owns value columns 64 h .. 64 h + 63 (of
//     the state, the outputs and the corrected values) and the same columns of A_acc; the
//     value side of every product splits along those columns, while the key side (the Gram
//     tiles over dk = 128, the inverse, Wc) is formed in both halves;
//   * eight waves per workgroup with the d = 64 roles: waves 0-3 ("K waves") take the key
//     side Gram rows, V', Wc (dk column blocks w and w + 4) and the state columns
//     16 w .. of the half; waves 4-7 ("Q waves") the query side Gram rows, the output, the
//     inverse's column blocks, A_acc's columns 16 (w - 4) .. of the half and Qhat;
//   * the 160 KB of LDS hold every [64][128] tile once, row-major: the products that
//     contract over tokens read their transposed operands with gfx950's transposing LDS
//     read (ds_read_b64_tr_b16) instead of a second, transposed copy;
//   * M and the diagonal inverse blocks live in Wc's space until Wc is formed.
//
// Outputs: O_loc and Qhat row-major [pair][token][128] in bfloat16, the segment operators
// A_acc [dk][dk] and B [dk][dv] in float32, the layouts the d = 128 scan and output
// correction (prism_kernels.h) read.
#pragma once
#include "prism_sweep8.h"

namespace prism {

struct Sweep128Lds {
  static constexpr int DK = 128, DV = 64, C = 64;
  static constexpr int LK = 136;  // row stride of the [64][128] tiles (68 dwords)
  static constexpr int LC = 72;   // row stride of the [64][64] tiles (36 dwords)
  static constexpr int LDT = 20;  // row stride of a 16x16 inverse block
  static constexpr size_t szK = (size_t)64 * LK * 2;
  static constexpr size_t szC = (size_t)64 * LC * 2;
  static constexpr size_t oQ = 0;             // Q [token][dk]
  static constexpr size_t oK = oQ + szK;      // K [token][dk]
  static constexpr size_t oHt = oK + szK;     // H^T [value column of the half][dk]
  static constexpr size_t oAt = oHt + szK;    // A_acc^T [column of the half][dk]
  static constexpr size_t oWc = oAt + szK;    // Wc [token][dk]; before it M and the blocks
  static constexpr size_t oM = oWc;           // M strict lower [i][j]
  static constexpr size_t oTd = oWc + szC;    // diagonal inverse blocks [4][16][LDT]
  static constexpr size_t oMt = oTd + (size_t)4 * 16 * LDT * 2;  // the K waves' float32 M^T blocks
  static constexpr size_t oVt = oWc + szK;    // V^T, later (beta V')^T [value][token]
  static constexpr size_t oMinv = oVt + szC;  // (I + M)^-1 [i][j]
  static constexpr size_t oGate = oMinv + szC;
  // b, G, D, beta, beta*G [C]; alpha^T [8][C]; conv taps of the half [4][DV]
  static constexpr size_t nGate = 5 * C + 8 * C + 4 * DV;
  // two slots of (U_l [token][dk], R_l^T [value][token]); slot 1's U_l space holds E^T
  // between the state phase and the output phase
  static constexpr size_t oSlot = oGate + nGate * 4;
  static constexpr size_t szSlot = szK + szC;
  static constexpr size_t total = oSlot + 2 * szSlot;
  static_assert(oMt + (size_t)4 * 16 * kMtLd * 4 <= oVt, "M, the diagonal blocks and M^T fit in Wc's space");
  static_assert(total <= 160 * 1024, "LDS plan exceeds the 160 KB of a CU");
};

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// 8 bf16 of a 32-deep MFMA operand from row r0 + lane%16 of a column-permuted LDS tile
// with row stride LD, in the k order of frag8 (one 16-byte read).
template <int LD>
__device__ __forceinline__ bf16x8 lfragL(const bf16_t* X, int r0, int k0) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x8*>(X + (r0 + (l & 15)) * LD + k0 + 8 * (l >> 4));
}

// The operand for row m0 + lane%16 of X^T, X a column-permuted [k][m] LDS tile: two
// transposing reads, k0 + 4g .. +3 and k0 + 16 + 4g .. +3.  In each 16-lane group lane
// 4 a + b names row k0 + 4 g + a (+16), columns m0 + 4 b .. +3, and receives column m0 + lane.
template <int LD>
__device__ __forceinline__ bf16x8 tfrag(const bf16_t* X, int m0, int k0) {
  const int l = lane_id(), g = l >> 4, i = l & 15;
  const bf16_t* s = X + (k0 + 4 * g + (i >> 2)) * LD + pcol(m0 + 4 * (i & 3));
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<bf16_t*>(s)));
  const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<bf16_t*>(s + 16 * LD)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
}

// An operand scaled by sc[k] (k in the logical order of the contraction).
__device__ __forceinline__ bf16x8 scale_k(const bf16x8& x, const float* sc, int k0) {
  const int g4 = 4 * (lane_id() >> 4);
  const float4 a = *reinterpret_cast<const float4*>(sc + k0 + g4);
  const float4 b = *reinterpret_cast<const float4*>(sc + k0 + 16 + g4);
  bf16x8 r;
  r[0] = (bf16_t)((float)x[0] * a.x);
  r[1] = (bf16_t)((float)x[1] * a.y);
  r[2] = (bf16_t)((float)x[2] * a.z);
  r[3] = (bf16_t)((float)x[3] * a.w);
  r[4] = (bf16_t)((float)x[4] * b.x);
  r[5] = (bf16_t)((float)x[5] * b.y);
  r[6] = (bf16_t)((float)x[6] * b.z);
  r[7] = (bf16_t)((float)x[7] * b.w);
  return r;
}

// [64][128] token tiles move in 16-byte LDS pieces: role thread tq takes pieces
// p = tq + 256 j (j < 4): token row p / 16, 32-column block (p / 4) % 4 and lane group
// g = p % 4, i.e. logical columns 32 blk + 4 g .. +3 and 32 blk + 16 + 4 g .. +3, which
// sit side by side in the column-permuted row.
__device__ __forceinline__ void row_fetch(uint2 (&x)[8], rsrc_t r, int tq, int t0, int row_bytes, int col_bytes) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = tq + 256 * j, row = p >> 4, blk = (p >> 2) & 3, g = p & 3;
    const int off = (t0 + row) * row_bytes + col_bytes + 64 * blk + 8 * g;
    x[2 * j] = bload8(r, off);
    x[2 * j + 1] = bload8(r, off + 32);
  }
}
__device__ __forceinline__ void row_store(const uint2 (&x)[8], bf16_t* dst, int tq) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = tq + 256 * j, row = p >> 4, blk = (p >> 2) & 3, g = p & 3;
    *reinterpret_cast<uint4*>(dst + row * Sweep128Lds::LK + 32 * blk + 8 * g) =
        make_uint4(x[2 * j].x, x[2 * j].y, x[2 * j + 1].x, x[2 * j + 1].y);
  }
}

struct Sweep128Ctx {
  unsigned char* smem;
  rsrc_t rq_, rk_, rv_, ru_, rg_;  // buffers over the pair's q, k, v, u, gamma
  rsrc_t rh_;                      // buffer over the pair's 3 value rows before the sequence
  bool hist;
  const float *gg, *bb, *al;
  bf16_t *oloc, *qhat;  // the pair's O_loc and Qhat rows
  float* agg;           // the segment's B (K waves) or A_acc (Q waves)
  int T, Lm1, c_begin, c_end, h;
  int urow;  // bytes per token row of u / gamma
};

struct Sweep128View {
  bf16_t *sQ, *sK, *sHt, *sAt, *sWc, *sM, *sTd, *sVt, *sMinv, *sEt;
  float *sB, *sG, *sD, *sBeta, *sBG, *sAlphaT, *sTaps;
  unsigned char* slot0;
  __device__ __forceinline__ explicit Sweep128View(unsigned char* smem) {
    using Ly = Sweep128Lds;
    sQ = reinterpret_cast<bf16_t*>(smem + Ly::oQ);
    sK = reinterpret_cast<bf16_t*>(smem + Ly::oK);
    sHt = reinterpret_cast<bf16_t*>(smem + Ly::oHt);
    sAt = reinterpret_cast<bf16_t*>(smem + Ly::oAt);
    sWc = reinterpret_cast<bf16_t*>(smem + Ly::oWc);
    sM = reinterpret_cast<bf16_t*>(smem + Ly::oM);
    sTd = reinterpret_cast<bf16_t*>(smem + Ly::oTd);
    sVt = reinterpret_cast<bf16_t*>(smem + Ly::oVt);
    sMinv = reinterpret_cast<bf16_t*>(smem + Ly::oMinv);
    sB = reinterpret_cast<float*>(smem + Ly::oGate);
    sG = sB + 64;
    sD = sG + 64;
    sBeta = sD + 64;
    sBG = sBeta + 64;
    sAlphaT = sBG + 64;
    sTaps = sAlphaT + 8 * 64;
    slot0 = smem + Ly::oSlot;
    sEt = slotU(1);
  }
  __device__ __forceinline__ bf16_t* slotU(int s) const {
    return reinterpret_cast<bf16_t*>(slot0 + (size_t)s * Sweep128Lds::szSlot);
  }
  __device__ __forceinline__ bf16_t* slotRt(int s) const {
    return reinterpret_cast<bf16_t*>(slot0 + (size_t)s * Sweep128Lds::szSlot + Sweep128Lds::szK);
  }
};

// Masked, decayed Gram rows rb of (X Y^T) over dk = 128 as a 64-deep A operand
// (contraction over the token j): raw tiles [j][i] = Y_j . X_i, `sign` folded in.
__device__ __forceinline__ void gram_rows128(bf16x8 (&fa)[2], const bf16_t* sY, const bf16_t* sX, int rb,
                                             const float (&dec)[4][4], float sign) {
  constexpr int LK = Sweep128Lds::LK;
  bf16x8 xf[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) xf[kb] = lfragL<LK>(sX, 16 * rb, 32 * kb);
  f32x4 raw[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    raw[jt] = zero4();
    if (jt <= rb) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) raw[jt] = mfma(lfragL<LK>(sY, 16 * jt, 32 * kb), xf[kb], raw[jt]);
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) fa[kb][4 * h + r] = (bf16_t)(sign * dec[2 * kb + h][r] * raw[2 * kb + h][r]);
}

// ---- the K waves ------------------------------------------------------------------------
template <int LM1S>
__device__ __forceinline__ void sweep128_kwave(const Sweep128Ctx& x, int wq) {
  constexpr int LK = Sweep128Lds::LK, LC = Sweep128Lds::LC, LDT = Sweep128Lds::LDT, C = 64;
  const Sweep128View V(x.smem);
  const int l = lane_id(), g4 = 4 * (l >> 4), li = l & 15;
  const int rb = 3 - wq, cb = wq;
  const int tq = threadIdx.x & 255;
  // LM1S >= 0 fixes L - 1 at compile time (the rank-L steps unrolled)
  const int Lm1 = LM1S >= 0 ? LM1S : x.Lm1;
  const int NL = Lm1 > 3 ? Lm1 : 3, L = Lm1 + 1;

  f32x4 H[8], Vp[4], HB[8], WH[4];
  float dec[4][4];
  uint2 pk[8], pu[8], lpf[8];
  float glg = 1.f, gbe = 0.f, gal[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) H[kt] = zero4();
#pragma unroll
  for (int j = 0; j < 8; ++j) gal[j] = 0.f;

  auto fetch_chunk = [&](int c) {
    const int t0 = c * C;
    row_fetch(pk, x.rk_, tq, t0, 256, 0);
    if (L > 1) row_fetch(pu, x.ru_, tq, t0, x.urow, 0);
    if (wq == 0) {
      const int hi = min(x.T, t0 + C);
      const int tl = t0 + l < hi ? t0 + l : 0;
      glg = x.gg[tl];
      gbe = x.bb[tl];
      if (L > 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) gal[j] = x.al[(size_t)tl * L + (j < L ? j : 0)];
      }
    }
  };
  auto store_chunk = [&](int c) {
    row_store(pk, V.sK, tq);
    if (L > 1) row_store(pu, V.slotU(0), tq);
    if (wq == 0) {  // b = cumsum(log g) over the chunk, G = exp(b), D = exp(b_last - b)
      const int t0 = c * C, hi = min(x.T, t0 + C);
      const bool ok = t0 + l < hi;  // tokens past the end: g = 1, beta = alpha = 0
      const float lam = wave_inclusive_sum(ok ? __logf(glg) : 0.f);
      const float blast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), C - 1));
      const float G = __expf(lam);
      V.sB[l] = lam;
      V.sG[l] = G;
      V.sD[l] = __expf(blast - lam);
      const float be = ok ? gbe : 0.f;
      V.sBeta[l] = be;
      V.sBG[l] = be * G;
#pragma unroll
      for (int j = 0; j < 8; ++j) V.sAlphaT[j * C + l] = (ok && L > 1 && j < L) ? gal[j] : 0.f;
    }
  };

  if (x.c_begin < x.c_end) {
    fetch_chunk(x.c_begin);
    store_chunk(x.c_begin);
  }
  for (int c = x.c_begin; c < x.c_end; ++c) {
    const int t0 = c * C;
    __syncthreads();  // B0: the chunk's inputs, gates and H^T are in LDS
    const int cn = c + 1 < x.c_end ? c + 1 : c;  // next chunk (unconditional loads)

    // ---- P0: M rows rb over dk = 128; diagonal inverse block -----------------------------
    {
      bf16x8 kf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kf[kb] = lfragL<LK>(V.sK, 16 * rb, 32 * kb);
      f32x4 draw = mfma(kf[0], kf[0], zero4()), draw2 = mfma(kf[2], kf[2], zero4());
      draw = mfma(kf[1], kf[1], draw);
      draw2 = mfma(kf[3], kf[3], draw2);
      decay_factors(dec, V.sB, rb, true);
      f32x4 mraw[3];
#pragma unroll
      for (int jt = 0; jt < 3; ++jt) {
        mraw[jt] = zero4();
        if (jt < rb) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) mraw[jt] = mfma(lfragL<LK>(V.sK, 16 * jt, 32 * kb), kf[kb], mraw[jt]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) draw[r] += draw2[r];
      const float beil = V.sBeta[16 * rb + li];
#pragma unroll
      for (int jt = 0; jt < 3; ++jt) {
        if (jt < rb) {
          bf16x4 mv;
#pragma unroll
          for (int r = 0; r < 4; ++r) mv[r] = (bf16_t)(beil * dec[jt][r] * mraw[jt][r]);
          *reinterpret_cast<bf16x4*>(V.sM + (16 * rb + li) * LC + pcol(16 * jt + g4)) = mv;
        }
      }
      // T_rb = (I + M_rb,rb)^-1 = (I + Y)(I + Y^2)(I + Y^4)(I + Y^8), Y = -M_rb,rb
      const float4 bi4 = *reinterpret_cast<const float4*>(V.sB + 16 * rb + g4);
      const float4 be4 = *reinterpret_cast<const float4*>(V.sBeta + 16 * rb + g4);
      const float bir[4] = {bi4.x, bi4.y, bi4.z, bi4.w};
      const float ber[4] = {be4.x, be4.y, be4.z, be4.w};
      const float bl = V.sB[16 * rb + li];
      f32x4 Y, Yt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float dd = rb == 0 ? dec[0][r] : rb == 1 ? dec[1][r] : rb == 2 ? dec[2][r] : dec[3][r];
        Y[r] = (li < g4 + r) ? -ber[r] * __expf(bir[r] - bl) * draw[r] : 0.f;  // Y[g4 + r][li]
        Yt[r] = -beil * dd * draw[r];                                        // Y[li][g4 + r]
      }
      const f32x4 Y2 = mm16_bf16(Yt, Y), Y2t = mm16_bf16(Y, Yt);
      const f32x4 Y4 = mm16_bf16(Y2t, Y2), Y4t = mm16_bf16(Y2, Y2t);
      // a power of Y past 1: the product cancels large terms, so float32 substitution
      float grow = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) grow = fmaxf(grow, fmaxf(fabsf(Y2[r]), fabsf(Y4[r])));
      if (!__any(grow > 1.f)) {
        const f32x4 Y8 = mm16_bf16(Y4t, Y4);
        f32x4 Pt = plus_identity(Yt);
        Pt = mm16_bf16(plus_identity(Y2), Pt);
        Pt = mm16_bf16(plus_identity(Y4), Pt);
        Pt = mm16_bf16(plus_identity(Y8), Pt);  // Pt = T^T: T[li][g4 + r] = Pt[r]
        *reinterpret_cast<bf16x4*>(V.sTd + (16 * rb + li) * LDT + g4) = to_bf16x4(Pt);
      } else {
        float* Mt = reinterpret_cast<float*>(x.smem + Sweep128Lds::oMt) + wq * 16 * kMtLd;
        *reinterpret_cast<float4*>(Mt + li * kMtLd + g4) = make_float4(-Y[0], -Y[1], -Y[2], -Y[3]);
        __builtin_amdgcn_wave_barrier();  // the wave's LDS stores land before its reads (in order)
        const f32x4 tc = diag_inverse_subst(Mt);  // T[g4 + r][li]
#pragma unroll
        for (int r = 0; r < 4; ++r) V.sTd[(16 * rb + g4 + r) * LDT + li] = (bf16_t)tc[r];
      }
    }
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) {  // V' starts as V (rows rb)
      const bf16x4 xv = *reinterpret_cast<const bf16x4*>(V.sVt + (16 * vt + li) * LC + pcol(16 * rb + g4));
#pragma unroll
      for (int r = 0; r < 4; ++r) Vp[vt][r] = (float)xv[r];
    }
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) HB[kt] = zero4();
    if (Lm1 >= 2) row_fetch(lpf, x.ru_, tq, t0, x.urow, 256);  // U_2
    __syncthreads();  // B1: M, diagonal inverse blocks, R_1

    // ---- P1 .. P_NL: rank-L steps ---------------------------------------------------------
    auto level_phase = [&](const int lv) {
      const int s = (lv - 1) & 1;
      if (lv <= Lm1) {
        const bf16_t* sU = V.slotU(s);
        const bf16_t* sRt = V.slotRt(s);
        bf16x8 xa[2];  // -strict(Gam * K U_l^T) rows rb
        gram_rows128(xa, sU, V.sK, rb, dec, -1.f);
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) {  // V' += X1 R_l
          Vp[vt] = mfma(xa[0], lfragL<LC>(sRt, 16 * vt, 0), Vp[vt]);
          if (rb >= 2) Vp[vt] = mfma(xa[1], lfragL<LC>(sRt, 16 * vt, 32), Vp[vt]);
        }
        // HB(:, cb) += U_l^T diag(D) R_l(:, cb) over the 8 dk tiles
        const bf16x8 rd0 = scale_k(lfragL<LC>(sRt, 16 * cb, 0), V.sD, 0);
        const bf16x8 rd1 = scale_k(lfragL<LC>(sRt, 16 * cb, 32), V.sD, 32);
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
          HB[kt] = mfma(tfrag<LK>(sU, 16 * kt, 0), rd0, HB[kt]);
          HB[kt] = mfma(tfrag<LK>(sU, 16 * kt, 32), rd1, HB[kt]);
        }
      }
      if (lv == 2) {
        // Wc = (I + M)^-1 diag(beta G) K for dk column blocks cb and cb + 4, formed as
        // Wc^T tiles (K^T diag(beta G) Minv^T) so each lane stores 4 adjacent dk columns
        bf16x8 ka[2][2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          ka[jj][0] = scale_k(tfrag<LK>(V.sK, 16 * (cb + 4 * jj), 0), V.sBG, 0);
          ka[jj][1] = scale_k(tfrag<LK>(V.sK, 16 * (cb + 4 * jj), 32), V.sBG, 32);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const bf16x8 m0 = lfragL<LC>(V.sMinv, 16 * it, 0);
          const bf16x8 m1 = lfragL<LC>(V.sMinv, 16 * it, 32);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            f32x4 acc = mfma(ka[jj][0], m0, zero4());
            if (it >= 2) acc = mfma(ka[jj][1], m1, acc);
            // acc[r] = Wc[16 it + li][16 (cb + 4 jj) + g4 + r]
            *reinterpret_cast<bf16x4*>(V.sWc + (16 * it + li) * LK + pcol(16 * (cb + 4 * jj) + g4)) = to_bf16x4(acc);
          }
        }
      }
      if (lv == NL) {  // WH = Wc H(:, cb), Wc from phase 2 (formed last: fewer live registers)
        bf16x8 hf[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) hf[kb] = pair8(H[2 * kb], H[2 * kb + 1]);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          f32x4 acc = mfma(lfragL<LK>(V.sWc, 16 * it, 0), hf[0], zero4());
          f32x4 acc2 = mfma(lfragL<LK>(V.sWc, 16 * it, 64), hf[2], zero4());
          acc = mfma(lfragL<LK>(V.sWc, 16 * it, 32), hf[1], acc);
          acc2 = mfma(lfragL<LK>(V.sWc, 16 * it, 96), hf[3], acc2);
#pragma unroll
          for (int r = 0; r < 4; ++r) WH[it][r] = acc[r] + acc2[r];
        }
      }
      if (lv + 1 <= Lm1) {  // U_{lv+1} into the other slot, then fetch U_{lv+2}
        row_store(lpf, V.slotU(s ^ 1), tq);
        if (lv + 2 <= Lm1) row_fetch(lpf, x.ru_, tq, t0, x.urow, (lv + 1) * 256);
      }
      // next chunk's inputs in the last level phase (fewer live registers before it)
      if (lv == NL) fetch_chunk(cn);
      if (lv == NL) {  // (beta V')^T rows rb for the per-column solve
        const float4 be = *reinterpret_cast<const float4*>(V.sBeta + 16 * rb + g4);
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) {
          const bf16x4 xv = {(bf16_t)(be.x * Vp[vt][0]), (bf16_t)(be.y * Vp[vt][1]), (bf16_t)(be.z * Vp[vt][2]),
                             (bf16_t)(be.w * Vp[vt][3])};
          *reinterpret_cast<bf16x4*>(V.sVt + (16 * vt + li) * LC + pcol(16 * rb + g4)) = xv;
        }
      }
      __syncthreads();
    };
    if constexpr (LM1S >= 0) {
#pragma unroll
      for (int lv = 1; lv <= (LM1S > 3 ? LM1S : 3); ++lv) level_phase(lv);
    } else {
      for (int lv = 1; lv <= NL; ++lv) level_phase(lv);
    }

    // ---- P_S: Uc = M^-1 (beta V')(:, cb), E = Uc - WH, H(:, cb) update -------------------------
    {
      const float GC = V.sG[C - 1];
      const bf16x8 v0 = lfragL<LC>(V.sVt, 16 * cb, 0), v1 = lfragL<LC>(V.sVt, 16 * cb, 32);
      f32x4 E[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 acc = mfma(lfragL<LC>(V.sMinv, 16 * it, 0), v0, zero4());
        if (it >= 2) acc = mfma(lfragL<LC>(V.sMinv, 16 * it, 32), v1, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) E[it][r] = acc[r] - WH[it][r];
        *reinterpret_cast<bf16x4*>(V.sEt + (16 * cb + li) * LC + pcol(16 * it + g4)) = to_bf16x4(E[it]);
      }
      const bf16x8 e0 = scaled_pair(E[0], E[1], V.sD, 0), e1 = scaled_pair(E[2], E[3], V.sD, 32);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        f32x4 he = mfma(tfrag<LK>(V.sK, 16 * kt, 0), e0, zero4());
        he = mfma(tfrag<LK>(V.sK, 16 * kt, 32), e1, he);
#pragma unroll
        for (int r = 0; r < 4; ++r) H[kt][r] = GC * H[kt][r] + he[r] + HB[kt][r];
      }
    }
    __syncthreads();  // E^T in LDS; every read of the old H^T and of K is done

    // ---- P_O: new H^T; next chunk into LDS ---------------------------------------------------
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
      *reinterpret_cast<bf16x4*>(V.sHt + (16 * cb + li) * LK + pcol(16 * kt + g4)) = to_bf16x4(H[kt]);
    if (c + 1 < x.c_end) store_chunk(c + 1);
  }
  // B of the segment: state columns 64 h + 16 cb + li, all dk rows
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) x.agg[(16 * kt + g4 + r) * 128 + 64 * x.h + 16 * cb + li] = H[kt][r];
}

// ---- the Q waves ------------------------------------------------------------------------
// NLG: each factor is p Phi(p r) of the running residual (the factor slots hold gains p);
// DLT: the written-correction chain (d = gamma r, r <- r - d, written alpha d).
template <int LM1S, bool NLG, bool DLT>
__device__ __forceinline__ void sweep128_qwave(const Sweep128Ctx& x, int wq) {
  constexpr int LK = Sweep128Lds::LK, LC = Sweep128Lds::LC, LDT = Sweep128Lds::LDT, C = 64;
  const Sweep128View V(x.smem);
  const int l = lane_id(), g4 = 4 * (l >> 4), li = l & 15;
  const int rb = wq, cb = wq;
  const int tq = threadIdx.x & 255;
  int rq, c4;
  quad_map(tq, rq, c4);
  const int Lm1 = LM1S >= 0 ? LM1S : x.Lm1;
  const int NL = Lm1 > 3 ? Lm1 : 3, L = Lm1 + 1;
  const int vcol = 128 * x.h + 2 * c4;  // byte offset of this thread's 4 value columns

  f32x4 A[8], O[4], WA[4];  // O^T tiles: [value 16 vt ..][token 16 rb ..]
  float rr[4][4];  // residual r_l of this lane's 4x4 block [row][col]
  float dec[4][4];
  bf16x8 Pa[2];
  uint2 pq[8], pv[8], pg[4], lpf[4];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {  // A_acc starts as the identity (columns 64 h + 16 cb ..)
    f32x4 t;
#pragma unroll
    for (int r = 0; r < 4; ++r) t[r] = (16 * kt + g4 + r == 64 * x.h + 16 * cb + li) ? 1.f : 0.f;
    A[kt] = t;
  }

  auto fetch_chunk = [&](int c) {
    const int t0 = c * C;
    row_fetch(pq, x.rq_, tq, t0, 256, 0);
    // the 4 value rows before the block, then the block (a negative base only ever
    // occurs for the first, whose rows are then padding)
    quad_fetch<4>(pv + 0, x.rv_, (t0 - 4 + 4 * rq) * 256 + vcol, 256);
    quad_fetch<4>(pv + 4, x.rv_, (t0 + 4 * rq) * 256 + vcol, 256);
    if (L > 1) quad_fetch<4>(pg, x.rg_, (t0 + 4 * rq) * x.urow + vcol, x.urow);  // gamma_0
  };
  auto store_chunk = [&]() {
    row_store(pq, V.sQ, tq);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const bf16x4 col = {__builtin_bit_cast(bf16x4, pv[4])[cc], __builtin_bit_cast(bf16x4, pv[5])[cc],
                          __builtin_bit_cast(bf16x4, pv[6])[cc], __builtin_bit_cast(bf16x4, pv[7])[cc]};
      *reinterpret_cast<bf16x4*>(V.sVt + (c4 + cc) * LC + pcol(4 * rq)) = col;
    }
  };
  // r_0 = v - anchor of the block (anchor_t = sum_j w_j v_{t-3+j})
  auto anchor = [&]() {
    float vv[8][4];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const bf16x4 b4 = __builtin_bit_cast(bf16x4, pv[r]);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) vv[r][cc] = (float)b4[cc];
    }
    const float4 w0 = *reinterpret_cast<const float4*>(V.sTaps + c4);
    const float4 w1 = *reinterpret_cast<const float4*>(V.sTaps + 64 + c4);
    const float4 w2 = *reinterpret_cast<const float4*>(V.sTaps + 128 + c4);
    const float4 w3 = *reinterpret_cast<const float4*>(V.sTaps + 192 + c4);
    const float t0w[4] = {w0.x, w0.y, w0.z, w0.w}, t1w[4] = {w1.x, w1.y, w1.z, w1.w};
    const float t2w[4] = {w2.x, w2.y, w2.z, w2.w}, t3w[4] = {w3.x, w3.y, w3.z, w3.w};
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        rr[r][cc] = vv[4 + r][cc] - (t0w[cc] * vv[1 + r][cc] + t1w[cc] * vv[2 + r][cc] +
                                     t2w[cc] * vv[3 + r][cc] + t3w[cc] * vv[4 + r][cc]);
  };
  // R_lv = alpha_lv r_lv from r_{lv-1} and the factor gamma_{lv-1} in gx, written transposed
  // into slot s
  auto residual_step = [&](const uint2* gx, int lv, int s) {
    const float4 ap = *reinterpret_cast<const float4*>(V.sAlphaT + (lv - 1) * C + 4 * rq);
    const float4 aw = *reinterpret_cast<const float4*>(V.sAlphaT + lv * C + 4 * rq);
    const float apr[4] = {ap.x, ap.y, ap.z, ap.w}, awr[4] = {aw.x, aw.y, aw.z, aw.w};
    float R[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bf16x4 gv = __builtin_bit_cast(bf16x4, gx[r]);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        float gm = (float)gv[cc];
        if constexpr (NLG) gm = (float)(bf16_t)(gm * std_normal_cdf(gm * rr[r][cc]));
        if constexpr (DLT) {
          const float d = gm * rr[r][cc];
          rr[r][cc] -= d;
          R[r][cc] = awr[r] * d;
        } else {
          const float xr = rr[r][cc] * (1.f - apr[r] * gm);
          rr[r][cc] = xr;
          R[r][cc] = awr[r] * xr;
        }
      }
    }
    bf16_t* dst = V.slotRt(s);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const bf16x4 col = {(bf16_t)R[0][cc], (bf16_t)R[1][cc], (bf16_t)R[2][cc], (bf16_t)R[3][cc]};
      *reinterpret_cast<bf16x4*>(dst + (c4 + cc) * LC + pcol(4 * rq)) = col;
    }
  };

  if (x.c_begin < x.c_end) {
    fetch_chunk(x.c_begin);
    if (x.c_begin == 0 && x.hist) {
      // tokens -3 .. -1 of the anchor window from the given history (block row rq = 0
      // holds tokens -4 .. -1; the other lanes read past the buffer, which returns zero)
      const int base = rq == 0 ? vcol : 4096;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const uint2 hv = bload8(x.rh_, base + j * 256);
        pv[1 + j].x |= hv.x;
        pv[1 + j].y |= hv.y;
      }
    }
    store_chunk();
  }
  for (int c = x.c_begin; c < x.c_end; ++c) {
    const int t0 = c * C;
    const int cn = c + 1 < x.c_end ? c + 1 : c;
    __syncthreads();  // B0

    // ---- P0: P = lower(Gam * Q K^T) rows rb; r_0 and R_1 ------------------------------------
    if (L > 1) anchor();
    decay_factors(dec, V.sB, rb, false);
    gram_rows128(Pa, V.sK, V.sQ, rb, dec, 1.f);
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) O[vt] = zero4();
    if (Lm1 >= 1) residual_step(pg, 1, 0);
    if (Lm1 >= 2) quad_fetch<4>(lpf, x.rg_, (t0 + 4 * rq) * x.urow + 256 + vcol, x.urow);  // gamma_1
    __syncthreads();  // B1

    // ---- P1 .. P_NL: rank-L steps; M^-1 (P1), WA and Qhat (P_NL) -----------------------------
    auto level_phase = [&](const int lv) {
      const int s = (lv - 1) & 1;
      if (lv <= Lm1) {  // O += lower(Gam * Q U_l^T) R_l
        const bf16_t* sU = V.slotU(s);
        const bf16_t* sRt = V.slotRt(s);
        bf16x8 xa[2];
        gram_rows128(xa, sU, V.sQ, rb, dec, 1.f);
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) {
          O[vt] = mfma(lfragL<LC>(sRt, 16 * vt, 0), xa[0], O[vt]);
          if (rb >= 2) O[vt] = mfma(lfragL<LC>(sRt, 16 * vt, 32), xa[1], O[vt]);
        }
      }
      if (lv == 1) {
        // column block cb of (I + M)^-1: X_cb = T_cb, X_i = -T_i sum_{cb <= k < i} M_ik X_k
        bf16x4 ident;
#pragma unroll
        for (int r = 0; r < 4; ++r) ident[r] = (bf16_t)((g4 + r == li) ? 1.f : 0.f);
        f32x4 X[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          X[i] = zero4();
          const bf16x4 ti = *reinterpret_cast<const bf16x4*>(V.sTd + (16 * i + li) * LDT + g4);
          if (i == cb) {
            X[i] = mfma16(ti, ident, zero4());
          } else if (i > cb) {
            f32x4 sacc = zero4();
#pragma unroll
            for (int kk = 0; kk < i; ++kk) {
              if (kk >= cb) {
                const bf16x4 am = *reinterpret_cast<const bf16x4*>(V.sM + (16 * i + li) * LC + pcol(16 * kk + g4));
                sacc = mfma16(am, to_bf16x4(X[kk]), sacc);
              }
            }
            f32x4 neg;
#pragma unroll
            for (int r = 0; r < 4; ++r) neg[r] = -sacc[r];
            X[i] = mfma16(ti, to_bf16x4(neg), zero4());
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // zero above the diagonal blocks
          const bf16x4 xv = to_bf16x4(X[i]);
#pragma unroll
          for (int r = 0; r < 4; ++r) V.sMinv[(16 * i + g4 + r) * LC + pcol(16 * cb + li)] = xv[r];
        }
      }
      if (lv == NL) {
        // WA = Wc A_acc(:, cb)
        bf16x8 af[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) af[kb] = pair8(A[2 * kb], A[2 * kb + 1]);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          f32x4 acc = mfma(lfragL<LK>(V.sWc, 16 * it, 0), af[0], zero4());
          f32x4 acc2 = mfma(lfragL<LK>(V.sWc, 16 * it, 64), af[2], zero4());
          acc = mfma(lfragL<LK>(V.sWc, 16 * it, 32), af[1], acc);
          acc2 = mfma(lfragL<LK>(V.sWc, 16 * it, 96), af[3], acc2);
#pragma unroll
          for (int r = 0; r < 4; ++r) WA[it][r] = acc[r] + acc2[r];
        }
        // Qtilde^T = (diag(G) Q)^T - Wc^T P^T (dk rows kt, tokens rb)
        const float Gi = V.sG[16 * rb + li];
        bf16x8 qf[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          f32x4 Qt[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int kt = 2 * kb + hh;
            const bf16x4 qv = *reinterpret_cast<const bf16x4*>(V.sQ + (16 * rb + li) * LK + pcol(16 * kt + g4));
            f32x4 pw = mfma(tfrag<LK>(V.sWc, 16 * kt, 0), Pa[0], zero4());
            if (rb >= 2) pw = mfma(tfrag<LK>(V.sWc, 16 * kt, 32), Pa[1], pw);
#pragma unroll
            for (int r = 0; r < 4; ++r) Qt[hh][r] = Gi * (float)qv[r] - pw[r];
          }
          qf[kb] = pair8(Qt[0], Qt[1]);
        }
        // Qhat^T = A_acc^T Qtilde^T for the half's columns: lane (li, g) ends with
        // Qhat[16 rb + li][64 h + 16 jt + g4 .. +3]
        bf16_t* qrow = x.qhat + (size_t)(t0 + 16 * rb + li) * 128 + 64 * x.h + g4;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          f32x4 e = mfma(lfragL<LK>(V.sAt, 16 * jt, 0), qf[0], zero4());
          f32x4 e2 = mfma(lfragL<LK>(V.sAt, 16 * jt, 64), qf[2], zero4());
          e = mfma(lfragL<LK>(V.sAt, 16 * jt, 32), qf[1], e);
          e2 = mfma(lfragL<LK>(V.sAt, 16 * jt, 96), qf[3], e2);
#pragma unroll
          for (int r = 0; r < 4; ++r) e[r] += e2[r];
          *reinterpret_cast<bf16x4*>(qrow + 16 * jt) = to_bf16x4(e);
        }
      }
      if (lv + 1 <= Lm1) {  // R_{lv+1} into the other slot, then fetch gamma_{lv+1}
        residual_step(lpf, lv + 1, s ^ 1);
        if (lv + 2 <= Lm1)
          quad_fetch<4>(lpf, x.rg_, (t0 + 4 * rq) * x.urow + (lv + 1) * 256 + vcol, x.urow);
      }
      if (lv == NL) fetch_chunk(cn);
      __syncthreads();
    };
    if constexpr (LM1S >= 0) {
#pragma unroll
      for (int lv = 1; lv <= (LM1S > 3 ? LM1S : 3); ++lv) level_phase(lv);
    } else {
      for (int lv = 1; lv <= NL; ++lv) level_phase(lv);
    }

    // ---- P_S: O += diag(G) Q H;  A_acc(:, cb) = G_C A_acc - K^T D WA ---------------------------
    {
      const float GC = V.sG[C - 1];
      const float Gi = V.sG[16 * rb + li];
      bf16x8 qf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) qf[kb] = lfragL<LK>(V.sQ, 16 * rb, 32 * kb);
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) {  // O^T += H^T Q^T diag(G)
        f32x4 qh = mfma(lfragL<LK>(V.sHt, 16 * vt, 0), qf[0], zero4());
        f32x4 qh2 = mfma(lfragL<LK>(V.sHt, 16 * vt, 64), qf[2], zero4());
        qh = mfma(lfragL<LK>(V.sHt, 16 * vt, 32), qf[1], qh);
        qh2 = mfma(lfragL<LK>(V.sHt, 16 * vt, 96), qf[3], qh2);
#pragma unroll
        for (int r = 0; r < 4; ++r) O[vt][r] += Gi * (qh[r] + qh2[r]);
      }
      const bf16x8 w0 = scaled_pair(WA[0], WA[1], V.sD, 0), w1 = scaled_pair(WA[2], WA[3], V.sD, 32);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        f32x4 aw = mfma(tfrag<LK>(V.sK, 16 * kt, 0), w0, zero4());
        aw = mfma(tfrag<LK>(V.sK, 16 * kt, 32), w1, aw);
#pragma unroll
        for (int r = 0; r < 4; ++r) A[kt][r] = GC * A[kt][r] - aw[r];
        *reinterpret_cast<bf16x4*>(V.sAt + (16 * cb + li) * LK + pcol(16 * kt + g4)) = to_bf16x4(A[kt]);
      }
    }
    __syncthreads();  // E^T in LDS

    // ---- P_O: O += P E, write O_loc; next chunk's Q, V^T and residual --------------------------
    {
      // lane (li, g) holds O^T[16 vt + g4 + r][16 rb + li]: four adjacent values of token
      // 16 rb + li, one 8-byte store per tile
      bf16_t* orow = x.oloc + (size_t)(t0 + 16 * rb + li) * 128 + 64 * x.h + g4;
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) {
        O[vt] = mfma(lfragL<LC>(V.sEt, 16 * vt, 0), Pa[0], O[vt]);
        if (rb >= 2) O[vt] = mfma(lfragL<LC>(V.sEt, 16 * vt, 32), Pa[1], O[vt]);
        *reinterpret_cast<bf16x4*>(orow + 16 * vt) = to_bf16x4(O[vt]);
      }
    }
    if (c + 1 < x.c_end) store_chunk();
  }
  // A_acc of the segment: columns 64 h + 16 cb + li, all dk rows
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) x.agg[(16 * kt + g4 + r) * 128 + 64 * x.h + 16 * cb + li] = A[kt][r];
}

// One workgroup per (segment, pair, value half): grid (nseg, P, 2), 512 threads.
template <int LM1S, bool NLG, bool DLT>
__device__ __forceinline__ void sweep128_run(FwdArgs a) {
  constexpr int D = 128, C = 64, LK = Sweep128Lds::LK;
  __shared__ __align__(16) unsigned char smem[Sweep128Lds::total];
  const Sweep128View V(smem);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seg = blockIdx.x, pr = blockIdx.y, h = blockIdx.z;
  const int hd = pr % a.H;
  const int T = a.T, L = a.L, Lm1 = L - 1;

  Sweep128Ctx x;
  x.smem = smem;
  x.T = T;
  x.Lm1 = Lm1;
  x.h = h;
  x.c_begin = seg * a.seg_chunks;
  x.c_end = min(a.nch, x.c_begin + a.seg_chunks);
  x.urow = (L > 1 ? Lm1 : 1) * D * 2;
  const size_t pair_rows = (size_t)pr * T;
  const unsigned rbytes = (unsigned)T * D * 2;
  const unsigned ubytes_all = (unsigned)T * (unsigned)x.urow;
  x.rq_ = make_rsrc(reinterpret_cast<const bf16_t*>(a.q) + pair_rows * D, rbytes);
  x.rk_ = make_rsrc(reinterpret_cast<const bf16_t*>(a.k) + pair_rows * D, rbytes);
  x.rv_ = make_rsrc(reinterpret_cast<const bf16_t*>(a.v) + pair_rows * D, rbytes);
  x.ru_ = make_rsrc(L > 1 ? reinterpret_cast<const bf16_t*>(a.u) + pair_rows * Lm1 * D : a.q, L > 1 ? ubytes_all : 0u);
  x.rg_ = make_rsrc(L > 1 ? reinterpret_cast<const bf16_t*>(a.gamma) + pair_rows * Lm1 * D : a.q,
                    L > 1 ? ubytes_all : 0u);
  x.hist = a.conv_in != nullptr;
  x.rh_ = make_rsrc(x.hist ? reinterpret_cast<const bf16_t*>(a.conv_in) + (size_t)pr * 3 * D : a.q,
                    x.hist ? 3u * D * 2u : 0u);
  x.gg = a.g + pair_rows;
  x.bb = a.beta + pair_rows;
  x.al = L > 1 ? a.alpha + pair_rows * L : nullptr;
  const size_t Tpad = (size_t)a.nch * C;
  x.oloc = reinterpret_cast<bf16_t*>(a.Oloc) + (size_t)pr * Tpad * D;
  x.qhat = reinterpret_cast<bf16_t*>(a.Qhat) + (size_t)pr * Tpad * D;
  x.agg = (w < 4 ? a.Bagg : a.Aagg) + ((size_t)pr * a.nseg + seg) * D * D;

  // conv taps of the half, H^T = 0, A_acc^T = the half's identity columns
  const float* cw = a.conv_w + (size_t)hd * 4 * D;
  for (int i = tid; i < 4 * 64; i += 512) V.sTaps[i] = L > 1 ? cw[(i >> 6) * D + 64 * h + (i & 63)] : 0.f;
  for (int i = tid; i < 64 * D; i += 512) {
    const int r = i / D, c = i % D;
    V.sHt[r * LK + pcol(c)] = (bf16_t)0.f;
    V.sAt[r * LK + pcol(c)] = (bf16_t)(c == 64 * h + r ? 1.f : 0.f);
  }
  __syncthreads();
  // Both roles pass the same barriers in the same order: B0, B1, one per phase
  // P1 .. P_NL and one after the state phase, for every chunk of the segment.
  if (w < 4) sweep128_kwave<LM1S>(x, w);
  else sweep128_qwave<LM1S, NLG, DLT>(x, w - 4);
}

template <int LM1S>
__global__ __launch_bounds__(512, 1) void seg_sweep128_kernel(FwdArgs a) {
  sweep128_run<LM1S, false, false>(a);
}

// the same sweep with the written-correction chain: a.gamma holds the corrections' factors
template <int LM1S>
__global__ __launch_bounds__(512, 1) void seg_sweep128_delta_kernel(FwdArgs a) {
  sweep128_run<LM1S, false, true>(a);
}

// the same sweep with the nonlinear refinement: a.gamma holds the gains p
template <int LM1S>
__global__ __launch_bounds__(512, 1) void seg_sweep128_nl_kernel(FwdArgs a) {
  sweep128_run<LM1S, true, false>(a);
}

}  // namespace prism
