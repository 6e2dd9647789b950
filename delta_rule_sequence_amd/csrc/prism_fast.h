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

// 8 bf16 of a 32-deep MFMA operand from row (r0 + lane%16) of a row-major array (LDS or global):
// slots 0-3 are k0 + 4g .. +3 and slots 4-7 are k0 + 16 + 4g .. +3 (g = lane/16).  The
// same read is the A operand (rows = output rows) and the B operand of a [n][k] array.
__device__ __forceinline__ bf16x8 frag8(const bf16_t* X, int ld, int r0, int k0) {
  const int l = lane_id();
  const bf16_t* p = X + (r0 + (l & 15)) * ld + k0 + 4 * (l >> 4);
  return cat8(*reinterpret_cast<const bf16x4*>(p), *reinterpret_cast<const bf16x4*>(p + 16));
}

// LDS plan of the fast sweep (bytes).
template <int D, int C>
struct FastLds {
  // Row strides of 34 / 10 dwords: the 16 rows an MFMA fragment read touches (and
  // the 16 lanes of a 4x4-block store) land in distinct bank pairs.
  static constexpr int LD = D + 4;    // row stride of [token][d] arrays (bf16)
  static constexpr int LDC = C + 4;   // row stride of [d][token] arrays (bf16)
  static constexpr int LDT = 16 + 4;  // row stride of a 16x16 diagonal inverse block
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
  // V^T with a 4-token halo: element (c, t) at [c][t + 4], t = -4 .. C-1
  static constexpr size_t oV = oTd + (size_t)(C / 16) * 16 * LDT * 2;
  static constexpr size_t oGate = oV + szDT;
  // b, G, D, beta, beta*G [C]; alpha^T [8][C]; conv taps [4][D]
  static constexpr size_t nGate = 5 * C + 8 * C + 4 * D;
  // two slots of (U_l [C][LD], gamma_{l-1}^T [D][LDC], R_l^T [D][LDC], U_l^T [D][LDC]);
  // after the refinement loop the region holds V'^T, Wc, Wc^T and E^T.
  static constexpr size_t oSlot = oGate + nGate * 4;
  static constexpr size_t szSlot = szTD + 3 * szDT;
  static constexpr size_t total = oSlot + 2 * szSlot;
  static_assert(szTD + 2 * szDT <= szSlot, "Wc, Wc^T and E^T must fit one slot");
  static_assert(C + 4 <= LDC, "V^T needs C + 4 token positions");
  static_assert(LD % 4 == 0 && LDC % 4 == 0 && LDT % 4 == 0, "8-byte aligned rows");
  static constexpr bool fits = total <= 160 * 1024;
};

// Input tiles move global -> registers -> LDS in 4-row x 4-column blocks:
// fetch_quads issues the loads (tile row r is global row row0 + r of `src`,
// rows outside [0, hi) read as zero at store time) and store_quads writes them
// to LDS, row-major and / or as the transposed copy; the transposed copy is four
// 8-byte writes (4 consecutive tokens of one column).  Splitting fetch and
// store lets a load be issued a whole phase before its data is needed.
template <int D, int ROWS>
struct QuadRegs {
  static_assert(ROWS % 4 == 0, "rows come in quads");
  static_assert(D == 64, "the block map below assumes 16 column quads");
  static constexpr int RQ = ROWS / 4;
  static constexpr int NB = RQ * 16;
  static constexpr int NIT = (NB + 255) / 256;
  uint2 x[NIT][4];
  int row0, hi;
  // Block b: a wave covers 4 row quads x 16 column quads; each 16-lane group holds a
  // 4 x 4 patch of blocks, so its row-major and its transposed 8-byte stores both hit
  // 32 distinct banks, and a wave's load of one row offset reads 4 whole rows.
  static __device__ __forceinline__ void map(int b, int& rq, int& c4) {
    const int l = b & 63;
    rq = 4 * (b >> 6) + (l & 3);
    c4 = 4 * (4 * (l >> 4) + ((l >> 2) & 3));
  }
};

template <int D, int ROWS>
__device__ __forceinline__ void fetch_quads(QuadRegs<D, ROWS>& R, const bf16_t* src, size_t row_stride, int row0,
                                            int hi) {
  using RR = QuadRegs<D, ROWS>;
  R.row0 = row0;
  R.hi = hi;
#pragma unroll
  for (int it = 0; it < RR::NIT; ++it) {
    const int b = threadIdx.x + 256 * it;
    int rq, c4;
    RR::map(b, rq, c4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gr = row0 + 4 * rq + r;
      const bool ok = rq < RR::RQ && gr >= 0 && gr < hi;
      const size_t rc = ok ? (size_t)gr : 0;
      R.x[it][r] = *reinterpret_cast<const uint2*>(src + rc * row_stride + c4);
    }
  }
}

template <int D, int ROWS, int LD, int LDC>
__device__ __forceinline__ void store_quads(const QuadRegs<D, ROWS>& R, bf16_t* dst, bf16_t* dstT) {
  using RR = QuadRegs<D, ROWS>;
#pragma unroll
  for (int it = 0; it < RR::NIT; ++it) {
    const int b = threadIdx.x + 256 * it;
    int rq, c4;
    RR::map(b, rq, c4);
    if (rq >= RR::RQ) continue;
    bf16x4 rows[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gr = R.row0 + 4 * rq + r;
      const uint2 x = (gr >= 0 && gr < R.hi) ? R.x[it][r] : make_uint2(0, 0);
      rows[r] = __builtin_bit_cast(bf16x4, x);
      if (dst != nullptr) *reinterpret_cast<uint2*>(dst + (4 * rq + r) * LD + c4) = x;
    }
    if (dstT != nullptr) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x4 col = {rows[0][c], rows[1][c], rows[2][c], rows[3][c]};
        *reinterpret_cast<bf16x4*>(dstT + (c4 + c) * LDC + 4 * rq) = col;
      }
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
  bf16_t* sVt0 = reinterpret_cast<bf16_t*>(smem + Ly::oV);  // V^T, token t at position t + 4
  float* sB = reinterpret_cast<float*>(smem + Ly::oGate);
  float* sG = sB + C;
  float* sD = sG + C;
  float* sBeta = sD + C;
  float* sBG = sBeta + C;
  float* sAlphaT = sBG + C;     // [8][C]
  float* sTaps = sAlphaT + 8 * C;  // [4][D]
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

  // conv taps [4][D] (zero when there is no rank injection)
  for (int idx = threadIdx.x; idx < 4 * D; idx += 256) sTaps[idx] = L > 1 ? cw[idx] : 0.f;

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

  // Everything one chunk reads from HBM, held in registers between its fetch (one
  // chunk ahead) and its store into LDS.
  struct ChunkRegs {
    QuadRegs<D, C> q, k, u1, g1;
    QuadRegs<D, C + 4> v;
    float lg, be, al[8];
    bool ok;  // this lane's token of the gates is inside the sequence
  };
  auto fetch_chunk = [&](ChunkRegs& R, int c) {
    const int t0 = c * C, hi = min(T, t0 + C);
    fetch_quads<D, C>(R.q, q, D, t0, hi);
    fetch_quads<D, C>(R.k, k, D, t0, hi);
    fetch_quads<D, C + 4>(R.v, v, D, t0 - 4, hi);
    if (L > 1) {
      fetch_quads<D, C>(R.u1, u, (size_t)Lm1 * D, t0, hi);
      fetch_quads<D, C>(R.g1, gam, (size_t)Lm1 * D, t0, hi);
    }
    if (w == 0) {  // raw loads; padding values are substituted at store time
      R.ok = t0 + l < hi;
      const int tl = R.ok ? t0 + l : 0;
      R.lg = gg[tl];
      R.be = bb[tl];
      if (L > 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) R.al[j] = al[(size_t)tl * L + (j < L ? j : 0)];
      }
    }
  };
  auto store_chunk = [&](const ChunkRegs& R) {
    store_quads<D, C, LD, LDC>(R.q, sQ, nullptr);
    store_quads<D, C, LD, LDC>(R.k, sK, sKt);
    store_quads<D, C + 4, LD, LDC>(R.v, nullptr, sVt0);
    if (L > 1) {
      store_quads<D, C, LD, LDC>(R.u1, reinterpret_cast<bf16_t*>(slot0),
                                 reinterpret_cast<bf16_t*>(slot0 + Ly::szTD + 2 * Ly::szDT));
      store_quads<D, C, LD, LDC>(R.g1, nullptr, reinterpret_cast<bf16_t*>(slot0 + Ly::szTD));
    }
    if (w == 0) {  // gates: b = cumsum(log g) over the chunk, G = exp(b), D = exp(b_last - b)
      float lam = R.ok ? __logf(R.lg) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(lam, off);
        if (l >= off) lam += y;
      }
      const float blast = __shfl(lam, C - 1);
      const float G = __expf(lam);
      sB[l] = lam;
      sG[l] = G;
      sD[l] = __expf(blast - lam);
      const float be = R.ok ? R.be : 0.f;
      sBeta[l] = be;
      sBG[l] = be * G;
#pragma unroll
      for (int j = 0; j < 8; ++j) sAlphaT[j * C + l] = (R.ok && L > 1 && j < L) ? R.al[j] : 0.f;
    }
  };

  ChunkRegs pre;
  if (c_begin < c_end) {
    fetch_chunk(pre, c_begin);
    store_chunk(pre);
  }
  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * C;
    __syncthreads();

    // ---- row-owned prologue: V' = V, residual r0 = V - anchor (tiles: rows 16w.., cols 16vt..)
    const int i0 = 16 * w;
    f32x4 Vp[KT], Oc[KT], Rr[KT];
#pragma unroll
    for (int vt = 0; vt < KT; ++vt) {
      const int col = 16 * vt + li;
      // tokens i0 + g4 - 4 .. i0 + g4 + 3 of column col (positions i0 + g4 .. +7)
      const bf16x4 va = *reinterpret_cast<const bf16x4*>(sVt0 + col * LDC + i0 + g4);
      const bf16x4 vb = *reinterpret_cast<const bf16x4*>(sVt0 + col * LDC + i0 + g4 + 4);
      const float vv[8] = {(float)va[0], (float)va[1], (float)va[2], (float)va[3],
                           (float)vb[0], (float)vb[1], (float)vb[2], (float)vb[3]};
      const float w0 = sTaps[col], w1 = sTaps[D + col], w2 = sTaps[2 * D + col], w3 = sTaps[3 * D + col];
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // token i0 + g4 + r is vv[r + 4]; tap j multiplies token - 3 + j
        const float x = vv[r + 4];
        Vp[vt][r] = x;
        Rr[vt][r] = x - (w0 * vv[r + 1] + w1 * vv[r + 2] + w2 * vv[r + 3] + w3 * vv[r + 4]);
      }
      Oc[vt] = zero4();
    }
    // ---- P(w, j) = lower(Gam * Q K^T) as chained A fragments; M(w, j) -> LDS -------------
    bf16x8 Pa[2];
    float dec[MT][4];
    {
      f32x4 praw[MT], mraw[MT];
#pragma unroll
      for (int jt = 0; jt < MT; ++jt) {
        praw[jt] = zero4();
        mraw[jt] = zero4();
        // all four tiles, masked below: branch-free, and wave 3 needs all four anyway
        mm_ll<bf16_t>(praw[jt], sK, LD, 16 * jt, sQ, LD, i0, D);   // (K_j Q_w^T): [j][i]
        mm_ll<bf16_t>(mraw[jt], sK, LD, 16 * jt, sK, LD, i0, D);   // (K_j K_w^T): [j][i]
      }
      // decay factors Gam(i0 + li, 16 jt + g4 + r), zero above the diagonal; every
      // masked Gram tile of this chunk (P, M, X1, X2) uses this lane layout
      {
        const float bi_lane = sB[i0 + li];
#pragma unroll
        for (int jt = 0; jt < MT; ++jt) {
          const float4 bj = *reinterpret_cast<const float4*>(sB + 16 * jt + g4);
          const float bjr[4] = {bj.x, bj.y, bj.z, bj.w};
#pragma unroll
          for (int r = 0; r < 4; ++r)
            dec[jt][r] = (16 * jt + g4 + r <= i0 + li) ? __expf(bi_lane - bjr[r]) : 0.f;
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) Pa[kb][4 * h + r] = (bf16_t)(dec[2 * kb + h][r] * praw[2 * kb + h][r]);
      // M tiles (row-major [i][j], strict lower, beta_i Gam_ij K_i.K_j)
      const float4 bi4 = *reinterpret_cast<const float4*>(sB + i0 + g4);
      const float4 be4 = *reinterpret_cast<const float4*>(sBeta + i0 + g4);
      const float bir[4] = {bi4.x, bi4.y, bi4.z, bi4.w};
      const float ber[4] = {be4.x, be4.y, be4.z, be4.w};
      const float beil = sBeta[i0 + li];
      {  // lane holds M[i0 + li][16 jt + g4 + r]: four consecutive columns of one row
#pragma unroll
        for (int jt = 0; jt < MT; ++jt) {
          if (jt < w) {
            bf16x4 mv;
#pragma unroll
            for (int r = 0; r < 4; ++r) mv[r] = (bf16_t)(beil * dec[jt][r] * mraw[jt][r]);
            *reinterpret_cast<bf16x4*>(sM + (i0 + li) * LDC + 16 * jt + g4) = mv;
          }
        }
      }
      // diagonal block inverse: Y = -M_ww (and Y^T, from the symmetric raw Gram tile)
      f32x4 Y, Yt;
      {
        const float bl = sB[i0 + li];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float raw = mraw[w][r];
          Y[r] = (li < g4 + r) ? -ber[r] * __expf(bir[r] - bl) * raw : 0.f;
          Yt[r] = (g4 + r < li) ? -beil * dec[w][r] * raw : 0.f;
        }
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
    QuadRegs<D, C> preU, preG;
    for (int lr = 1; lr < L; ++lr) {
      unsigned char* slot = slot0 + (size_t)((lr - 1) & 1) * Ly::szSlot;
      bf16_t* sU = reinterpret_cast<bf16_t*>(slot);
      bf16_t* sGt = reinterpret_cast<bf16_t*>(slot + Ly::szTD);                  // gamma_{l-1}^T
      bf16_t* sRt = reinterpret_cast<bf16_t*>(slot + Ly::szTD + Ly::szDT);       // R_l^T
      bf16_t* sUt = reinterpret_cast<bf16_t*>(slot + Ly::szTD + 2 * Ly::szDT);   // U_l^T
      __syncthreads();  // U_l, gamma_{l-1} of this step are in the slot
      if (lr + 1 < L) {
        const int hi = min(T, t0 + C);
        fetch_quads<D, C>(preU, u + (size_t)lr * D, (size_t)Lm1 * D, t0, hi);
        fetch_quads<D, C>(preG, gam + (size_t)lr * D, (size_t)Lm1 * D, t0, hi);
      }
      // residual step and R_l = alpha_l r_l for rows 16w.., written transposed
      {
        const float4 ap4 = *reinterpret_cast<const float4*>(sAlphaT + (lr - 1) * C + i0 + g4);
        const float4 al4 = *reinterpret_cast<const float4*>(sAlphaT + lr * C + i0 + g4);
        const float ap[4] = {ap4.x, ap4.y, ap4.z, ap4.w}, aw[4] = {al4.x, al4.y, al4.z, al4.w};
        bf16x4 gv[KT];
#pragma unroll
        for (int vt = 0; vt < KT; ++vt)
          gv[vt] = *reinterpret_cast<const bf16x4*>(sGt + (16 * vt + li) * LDC + i0 + g4);
#pragma unroll
        for (int vt = 0; vt < KT; ++vt) {
          bf16x4 rv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = Rr[vt][r] * (1.f - ap[r] * (float)gv[vt][r]);
            Rr[vt][r] = x;
            rv[r] = (bf16_t)(aw[r] * x);
          }
          *reinterpret_cast<bf16x4*>(sRt + (16 * vt + li) * LDC + i0 + g4) = rv;
        }
      }
      __syncthreads();
      // row-owned: X1 = -strict(Gam * K U^T), X2 = lower(Gam * Q U^T) as A fragments
      {
        f32x4 x1raw[MT], x2raw[MT];
#pragma unroll
        for (int jt = 0; jt < MT; ++jt) {
          x1raw[jt] = zero4();
          x2raw[jt] = zero4();
          mm_ll<bf16_t>(x1raw[jt], sU, LD, 16 * jt, sK, LD, i0, D);  // (U_j K_w^T): [j][i]
          mm_ll<bf16_t>(x2raw[jt], sU, LD, 16 * jt, sQ, LD, i0, D);  // (U_j Q_w^T): [j][i]
        }
        bf16x8 X1a[2], X2a[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int jt = 2 * kb + h;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float gm = dec[jt][r];
              X1a[kb][4 * h + r] = (bf16_t)((16 * jt + g4 + r < i0 + li) ? -gm * x1raw[jt][r] : 0.f);
              X2a[kb][4 * h + r] = (bf16_t)(gm * x2raw[jt][r]);
            }
          }
#pragma unroll
        for (int vt = 0; vt < KT; ++vt) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {  // fragments above the diagonal are zero
            const bf16x8 rb = cat8(ldsT_b4(sRt, LDC, 16 * vt, 32 * kb), ldsT_b4(sRt, LDC, 16 * vt, 32 * kb + 16));
            Vp[vt] = mfma(X1a[kb], rb, Vp[vt]);
            Oc[vt] = mfma(X2a[kb], rb, Oc[vt]);
          }
        }
      }
      // column-owned: HB(:, w) += U^T diag(D) R(:, w)  (A from U^T, scaled by D in registers)
      {
        bf16x8 rb[2];  // D (.) R(:, w), the B operand
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const float4 d0 = *reinterpret_cast<const float4*>(sD + 32 * kb + g4);
          const float4 d1 = *reinterpret_cast<const float4*>(sD + 32 * kb + 16 + g4);
          const float dv8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
          const bf16x8 r8 = cat8(ldsT_b4(sRt, LDC, 16 * w, 32 * kb), ldsT_b4(sRt, LDC, 16 * w, 32 * kb + 16));
#pragma unroll
          for (int p = 0; p < 8; ++p) rb[kb][p] = (bf16_t)(dv8[p] * (float)r8[p]);
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 ua = cat8(ldsT_b4(sUt, LDC, 16 * kt, 32 * kb), ldsT_b4(sUt, LDC, 16 * kt, 32 * kb + 16));
            HB[kt] = mfma(ua, rb[kb], HB[kt]);
          }
        }
      }
      if (lr + 1 < L) {  // the other slot was last read before this step's first barrier
        unsigned char* nslot = slot0 + (size_t)(lr & 1) * Ly::szSlot;
        store_quads<D, C, LD, LDC>(preU, reinterpret_cast<bf16_t*>(nslot),
                                   reinterpret_cast<bf16_t*>(nslot + Ly::szTD + 2 * Ly::szDT));
        store_quads<D, C, LD, LDC>(preG, nullptr, reinterpret_cast<bf16_t*>(nslot + Ly::szTD));
      }
    }

    // next chunk's inputs: issued here so their registers are live only through the
    // remaining phases, which still cover the load latency
    if (c + 1 < c_end) fetch_chunk(pre, c + 1);

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
#pragma unroll
      for (int vt = 0; vt < KT; ++vt) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 eb = cat8(ldsT_b4(sEt, LDC, 16 * vt, 32 * kb), ldsT_b4(sEt, LDC, 16 * vt, 32 * kb + 16));
          Oc[vt] = mfma(Pa[kb], eb, Oc[vt]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) oloc[(size_t)(g4 + r) * D + 16 * vt + li] = Oc[vt][r];
      }
    }
    // ---- column-owned: H(:, w) = G_C H + K^T D E + HB;  A_acc(:, w) = G_C A_acc - K^T D WA
    {
      const float GC = sG[C - 1];
      bf16x8 eb[2], wb[2];  // D (.) E(:, w) and D (.) WA(:, w), the B operands
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 d0 = *reinterpret_cast<const float4*>(sD + 32 * kb + g4);
        const float4 d1 = *reinterpret_cast<const float4*>(sD + 32 * kb + 16 + g4);
        const float dv8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          eb[kb][r] = (bf16_t)(dv8[r] * E[2 * kb][r]);
          eb[kb][4 + r] = (bf16_t)(dv8[4 + r] * E[2 * kb + 1][r]);
          wb[kb][r] = (bf16_t)(dv8[r] * WA[2 * kb][r]);
          wb[kb][4 + r] = (bf16_t)(dv8[4 + r] * WA[2 * kb + 1][r]);
        }
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        f32x4 he = zero4(), aw = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kd = cat8(ldsT_b4(sKt, LDC, 16 * kt, 32 * kb), ldsT_b4(sKt, LDC, 16 * kt, 32 * kb + 16));
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
    // new H^T and A_acc^T into LDS for the next chunk, then the prefetched inputs
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      *reinterpret_cast<bf16x4*>(sHt + (16 * w + li) * LD + 16 * kt + g4) = to_bf16x4(Hs[kt]);
      *reinterpret_cast<bf16x4*>(sAt + (16 * w + li) * LD + 16 * kt + g4) = to_bf16x4(As[kt]);
    }
    if (c + 1 < c_end) store_chunk(pre);
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

// Cross-lane moves within 8-lane groups (DPP): lane l reads lane 7 - l of its group of 8,
// 3 - l of its quad, or l ^ 1.
__device__ __forceinline__ float dpp_half_mirror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_rev(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x1B, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_swap(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}

// Inter-segment recurrence H_in(s+1) = A_s H_in(s) + B_s (float32); one workgroup per
// (pair, 4 state columns c0 ..).  Thread t takes state rows i0 = 2 (t / 8), i0 + 1 and the
// contraction slice k = 8 q .. 8 q + 7 (q = t % 8): it keeps those 16 entries of A_s in
// registers (loaded DEPTH steps ahead, so a step never waits on memory), reads rows
// 8 q .. 8 q + 7 of the four H_in(s) columns from LDS (skewed so the eight slices of a
// wave hit distinct banks) and forms 2 x 4 partial sums; three DPP exchange rounds within
// the 8 lanes of the row pair leave lane q with H_in(s+1)[i0 + q / 4][c0 + q % 4].  One
// barrier per step.
template <int DK, int DV>
__global__ __launch_bounds__(256) void seg_scan_fast_kernel(FwdArgs a) {
  static_assert(DK == 64, "the row-pair / k-slice split assumes 64 state rows");
  constexpr int DEPTH = 8;
  constexpr int HS = DK + DK / 8;  // H rows with a one-row skew every 8 rows
  __shared__ __align__(16) float4 sH[2][HS];
  const int tid = threadIdx.x, i0 = 2 * (tid >> 3), q = tid & 7;
  const int pr = blockIdx.x, c0 = 4 * blockIdx.y;
  const int nseg = a.nseg;
  const int orow = i0 + (q >> 2), ocol = c0 + (q & 3);  // the output this lane ends with
  const float* A0 = a.Aagg + (size_t)pr * nseg * DK * DK + (size_t)i0 * DK + 8 * q;
  const float* B0 = a.Bagg + (size_t)pr * nseg * DK * DV + (size_t)orow * DV + ocol;
  // H_in(s) for the output correction: bfloat16, transposed ([column][row], the layout
  // of its MFMA B operand)
  bf16_t* H0 = reinterpret_cast<bf16_t*>(a.Hin) + (size_t)pr * nseg * DK * DV + (size_t)ocol * DK + orow;
  auto hrow = [](int r) { return r + (r >> 3); };
  // ring slot D: the operands of the next step s with s % DEPTH == D (rows i0, i0 + 1 of
  // A_s over the slice, and this lane's entry of B_s)
#define PRISM_DECL(D) float4 R##D##_0, R##D##_1, R##D##_2, R##D##_3; float R##D##_b;
#define PRISM_FETCH(D, S)                                                                     \
  {                                                                                           \
    const size_t sn_ = (size_t)((S) < nseg ? (S) : nseg - 1);                                 \
    const float4* src_ = reinterpret_cast<const float4*>(A0 + sn_ * DK * DK);                \
    R##D##_0 = src_[0];                                                                       \
    R##D##_1 = src_[1];                                                                       \
    R##D##_2 = src_[DK / 4];                                                                  \
    R##D##_3 = src_[DK / 4 + 1];                                                              \
    R##D##_b = B0[sn_ * DK * DV];                                                             \
  }
  PRISM_DECL(0) PRISM_DECL(1) PRISM_DECL(2) PRISM_DECL(3)
  PRISM_DECL(4) PRISM_DECL(5) PRISM_DECL(6) PRISM_DECL(7)
  PRISM_FETCH(0, 0) PRISM_FETCH(1, 1) PRISM_FETCH(2, 2) PRISM_FETCH(3, 3)
  PRISM_FETCH(4, 4) PRISM_FETCH(5, 5) PRISM_FETCH(6, 6) PRISM_FETCH(7, 7)
  float h = 0.f;  // H_in(s)[orow][ocol]
  if (tid < DK) sH[0][hrow(tid)] = make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();
  const bool lo4 = q < 4, lo2 = (q & 2) == 0, lo1 = (q & 1) == 0;
  int cur = 0;
#define PRISM_SCAN_STEP(D, PREFETCH)                                                          \
  {                                                                                           \
    const int s = s0 + (D);                                                                   \
    H0[(size_t)s * DK * DV] = (bf16_t)h;                                                      \
    const float ar0[8] = {R##D##_0.x, R##D##_0.y, R##D##_0.z, R##D##_0.w,                     \
                          R##D##_1.x, R##D##_1.y, R##D##_1.z, R##D##_1.w};                    \
    const float ar1[8] = {R##D##_2.x, R##D##_2.y, R##D##_2.z, R##D##_2.w,                     \
                          R##D##_3.x, R##D##_3.y, R##D##_3.z, R##D##_3.w};                    \
    const float bv = R##D##_b;                                                                \
    if (PREFETCH) PRISM_FETCH(D, s + DEPTH)                                                   \
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}; /* [row][col] */                   \
    _Pragma("unroll") for (int m = 0; m < 8; ++m) {                                           \
      const float4 hv = sH[cur][hrow(8 * q + m)];                                             \
      v[0] += ar0[m] * hv.x;                                                                  \
      v[1] += ar0[m] * hv.y;                                                                  \
      v[2] += ar0[m] * hv.z;                                                                  \
      v[3] += ar0[m] * hv.w;                                                                  \
      v[4] += ar1[m] * hv.x;                                                                  \
      v[5] += ar1[m] * hv.y;                                                                  \
      v[6] += ar1[m] * hv.z;                                                                  \
      v[7] += ar1[m] * hv.w;                                                                  \
    }                                                                                         \
    /* keep row q / 4, then columns (q & 2) .., then column q & 3 */                          \
    float n4[4], n2[2];                                                                       \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                             \
      n4[j] = (lo4 ? v[j] : v[4 + j]) + dpp_half_mirror(lo4 ? v[4 + j] : v[j]);               \
    _Pragma("unroll") for (int j = 0; j < 2; ++j)                                             \
      n2[j] = (lo2 ? n4[j] : n4[2 + j]) + dpp_quad_rev(lo2 ? n4[2 + j] : n4[j]);              \
    h = (lo1 ? n2[0] : n2[1]) + dpp_quad_swap(lo1 ? n2[1] : n2[0]) + bv;                       \
    reinterpret_cast<float*>(&sH[cur ^ 1][hrow(orow)])[q & 3] = h;                            \
    cur ^= 1;                                                                                 \
    __syncthreads();                                                                          \
  }
  // full blocks of DEPTH steps: every step consumes its ring slot and refills it
  // unconditionally, so each slot is loaded straight into its own registers
  int s0 = 0;
  for (; s0 + DEPTH <= nseg; s0 += DEPTH) {
    PRISM_SCAN_STEP(0, true) PRISM_SCAN_STEP(1, true) PRISM_SCAN_STEP(2, true) PRISM_SCAN_STEP(3, true)
    PRISM_SCAN_STEP(4, true) PRISM_SCAN_STEP(5, true) PRISM_SCAN_STEP(6, true) PRISM_SCAN_STEP(7, true)
  }
  // the last nseg % DEPTH steps: their operands are already in the ring
  if (s0 + 0 < nseg) PRISM_SCAN_STEP(0, false)
  if (s0 + 1 < nseg) PRISM_SCAN_STEP(1, false)
  if (s0 + 2 < nseg) PRISM_SCAN_STEP(2, false)
  if (s0 + 3 < nseg) PRISM_SCAN_STEP(3, false)
  if (s0 + 4 < nseg) PRISM_SCAN_STEP(4, false)
  if (s0 + 5 < nseg) PRISM_SCAN_STEP(5, false)
  if (s0 + 6 < nseg) PRISM_SCAN_STEP(6, false)
#undef PRISM_SCAN_STEP
#undef PRISM_FETCH
#undef PRISM_DECL
  a.S_final[(size_t)pr * DK * DV + (size_t)orow * DV + ocol] = h;
}

// Output correction o = O_loc + Qhat H_in(segment) with MFMA; one workgroup per segment
// (4 waves), wave w takes token rows 16 w .. of every chunk of the segment.  Each wave
// holds its B operand, H_in(segment) transposed in bfloat16, in registers for the whole
// segment and streams the chunks: O_loc and Qhat come in the sweep's fragment order (one
// contiguous 8- or 16-byte load per lane and tile), the next chunk's fragments are loaded
// while the current one is finished, and the 16 x 64 output block is staged in the
// wave's own LDS rows for 16-byte row stores (no workgroup barrier).
template <int D, int C>
__global__ __launch_bounds__(256) void seg_fixup_fast_kernel(FwdArgs a) {
  static_assert(D == 64 && C == 64, "fragment order written for 64 x 64 chunks");
  constexpr int LD = D + 8;
  __shared__ __align__(16) bf16_t sO[4][16 * LD];
  const int w = wave_id(), l = lane_id(), g4 = (l >> 4) * 4, li = l & 15;
  const int seg = blockIdx.x, pr = blockIdx.y;
  const int c_begin = seg * a.seg_chunks, c_end = min(a.nch, c_begin + a.seg_chunks);
  const bf16_t* hin = reinterpret_cast<const bf16_t*>(a.Hin) + ((size_t)pr * a.nseg + seg) * D * D;
  bf16x8 hb[4][2];
#pragma unroll
  for (int vt = 0; vt < 4; ++vt)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) hb[vt][kb] = frag8(hin, D, 16 * vt, 32 * kb);
  const size_t gc0 = (size_t)pr * a.nch;
  const bf16_t* qbase = reinterpret_cast<const bf16_t*>(a.Qhat) + (size_t)w * 1024 + l * 8;
  const bf16_t* obase = reinterpret_cast<const bf16_t*>(a.Oloc) + (size_t)w * 1024 + l * 4;
  bf16_t* so = sO[w];
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<bf16_t*>(a.o) + (size_t)pr * a.T * D, (short)0, a.T * D * 2, 0x00020000);
  bf16x8 qf[2];
  bf16x4 of[4];
  auto fetch = [&](int c) {
    const size_t off = (gc0 + c) * 4096;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) qf[kb] = *reinterpret_cast<const bf16x8*>(qbase + off + kb * 512);
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) of[vt] = *reinterpret_cast<const bf16x4*>(obase + off + vt * 256);
  };
  if (c_begin < c_end) fetch(c_begin);
  for (int c = c_begin; c < c_end; ++c) {
    f32x4 acc[4];
    bf16x8 qa[2] = {qf[0], qf[1]};
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[vt][r] = (float)of[vt][r];
    }
    fetch(c + 1 < c_end ? c + 1 : c);  // unconditional: the wait for it stays exact
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) {
      acc[vt] = mfma(qa[0], hb[vt][0], acc[vt]);
      acc[vt] = mfma(qa[1], hb[vt][1], acc[vt]);
#pragma unroll
      for (int r = 0; r < 4; ++r) so[(g4 + r) * LD + 16 * vt + li] = (bf16_t)acc[vt][r];
    }
    __builtin_amdgcn_wave_barrier();  // the wave's LDS writes land before its reads (in order)
    // rows t0 + 16 w .. of the output, 8 lanes per 128-byte row; rows past the sequence
    // end fall outside the pair's buffer and are dropped by the store
    const int t0 = c * C + 16 * w;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int row = 8 * it + (l >> 3), cv = (l & 7) * 8;
      const uint4 x = *reinterpret_cast<const uint4*>(so + row * LD + cv);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, x), orsrc,
                                            ((t0 + row) * D + cv) * 2, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();  // reads done before the next chunk's writes
  }
}

}  // namespace prism
