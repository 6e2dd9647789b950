// prism_sweep8.h - the bfloat16 segment sweep for head dim 64, two waves per SIMD (gfx950).
//
// Same mathematics as seg_local_kernel (prism_kernels.h): per 64-token chunk the
// UT / WY form of the gated delta rule with the rank-L writes folded in
// (PRISM reading notes, sections 2.2-2.3; PRISM summary page, "architecture"
// section), carried across the chunks of one segment together with the
// segment operator A_acc.  Organisation for CDNA4:
//
//   * one workgroup of 8 waves per segment, one segment per CU, so every SIMD
//     runs two waves and one wave's MFMA / LDS latency hides behind the other;
//   * waves 0-3 ("K waves") own the key side of the chunk: the masked Gram
//     tiles K K^T and K U_l^T of token rows 16 (3 - w)..; the corrected values
//     V'; the per-column work Wc = M^-1 diag(beta G) K, Uc = M^-1 beta V', E = Uc - Wc H and the state
//     update of H (columns 16 w..); the rank-L state term sum_l U_l^T D R_l;
//   * waves 4-7 ("Q waves") own the query side: the masked Gram tiles Q K^T and
//     Q U_l^T of token rows 16 (w - 4)..; the chunk output; the inverse M^-1
//     (column block w - 4), the segment operator
//     A_acc and Qhat; they also run the residual chain of the rank-L values;
//   * a K wave and a Q wave on one SIMD take row blocks r and 3 - r, so the
//     triangular Gram work is the same on every SIMD;
//   * (I + M)^-1 is built explicitly: the 16x16 diagonal blocks by the product
//     (I + Y)(I + Y^2)(I + Y^4)(I + Y^8) (Y = -M_ii is nilpotent; bfloat16 products
//     with float32 accumulation), or, when a power of Y grows past 1 (the product then
//     cancels large terms: one key repeated with beta near 1), by float32 forward
//     substitution; the rest by block forward substitution on identity columns,
//     overlapped with the rank-L steps, so the solve that depends on V' is one product;
//   * one barrier per rank-L step plus four per chunk (L + 3 for L >= 4); the
//     inputs of the next step / chunk are loaded one phase ahead into registers.
#pragma once
#include "prism_fast.h"
#include "prism_nl.h"

namespace prism {

// LDS plan (bytes).  Every [64][64] bf16 array has row stride 72 (36 dwords) and its
// columns permuted inside each 32-column block (pcol below), so that a lane's MFMA operand
// (8 values of one row) is 16 contiguous bytes: one ds_read_b128, which on gfx950 moves
// twice the bytes per clock of the 8-byte reads.  With the 36-dword stride the 16 lanes of
// an operand read, and the 16 lanes of a 4x4-block store, touch distinct banks.
struct Sweep8Lds {
  static constexpr int D = 64, C = 64;
  static constexpr int LD = 72;
  static constexpr int LDT = 20;                     // row stride of a 16x16 inverse block
  static constexpr size_t szA = (size_t)64 * LD * 2;  // one array
  static constexpr size_t oQ = 0;                    // Q [token][d]
  static constexpr size_t oK = oQ + szA;             // K [token][d]
  static constexpr size_t oKt = oK + szA;            // K^T [d][token]
  static constexpr size_t oVt = oKt + szA;           // V^T, later (beta V')^T [d][token]
  static constexpr size_t oHt = oVt + szA;           // H^T [dv][dk] (state entering the chunk)
  static constexpr size_t oAt = oHt + szA;           // A_acc^T [dk][dk]
  static constexpr size_t oM = oAt + szA;            // M strict lower [i][j]; later Wc [token][d]
  static constexpr size_t oMinv = oM + szA;          // (I + M)^-1 [i][j]
  static constexpr size_t oWct = oMinv + szA;        // Wc^T [d][token]
  static constexpr size_t oTd = oWct + szA;          // diagonal inverse blocks [4][16][LDT]
  static constexpr size_t oGate = oTd + (size_t)4 * 16 * LDT * 2;
  // b, G, D, beta, beta*G [C]; alpha^T [8][C]; conv taps [4][D]
  static constexpr size_t nGate = 5 * C + 8 * C + 4 * D;
  // each key-side wave's float32 copy of its diagonal block M^T, for the substitution
  static constexpr size_t oMt = oGate + nGate * 4;
  // two slots of (U_l [token][d], U_l^T [d][token], R_l^T [dv][token]); slot 1 holds
  // E^T between the state phase and the output phase
  static constexpr size_t oSlot = oMt + (size_t)4 * 16 * kMtLd * 4;
  static constexpr size_t szSlot = 3 * szA;
  static constexpr size_t total = oSlot + 2 * szSlot;
  static_assert(total <= 160 * 1024, "LDS plan exceeds the 160 KB of a CU");
};

// Two accumulator tiles (rows k0.. and k0+16.. of the contraction) as a 32-deep B
// operand, each element scaled by s[k].
__device__ __forceinline__ bf16x8 scaled_pair(const f32x4& t0, const f32x4& t1, const float* s, int k0) {
  const int g4 = 4 * (lane_id() >> 4);
  const float4 a = *reinterpret_cast<const float4*>(s + k0 + g4);
  const float4 b = *reinterpret_cast<const float4*>(s + k0 + 16 + g4);
  bf16x8 r;
  r[0] = (bf16_t)(t0[0] * a.x);
  r[1] = (bf16_t)(t0[1] * a.y);
  r[2] = (bf16_t)(t0[2] * a.z);
  r[3] = (bf16_t)(t0[3] * a.w);
  r[4] = (bf16_t)(t1[0] * b.x);
  r[5] = (bf16_t)(t1[1] * b.y);
  r[6] = (bf16_t)(t1[2] * b.z);
  r[7] = (bf16_t)(t1[3] * b.w);
  return r;
}

__device__ __forceinline__ bf16x8 pair8(const f32x4& t0, const f32x4& t1) { return cat8(to_bf16x4(t0), to_bf16x4(t1)); }

// Stored position of logical column c of an LDS array: inside each 32-column block,
// column 16 h + 4 g + e (h < 2, g < 4, e < 4) sits at 8 g + 4 h + e, so the two 4-column
// halves of lane group g's 32-deep operand (columns 4 g .. and 16 + 4 g ..) are adjacent.
// Four consecutive columns starting at a multiple of 4 stay consecutive.
__device__ __forceinline__ constexpr int pcol(int c) { return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3); }

// 8 bf16 of a 32-deep MFMA operand from row r0 + lane%16 of a column-permuted LDS array, in
// the k order of frag8 (k0 + 4g .. +3, then k0 + 16 + 4g .. +3; k0 = 0 or 32): one 16-byte read.
__device__ __forceinline__ bf16x8 lfrag(const bf16_t* X, int r0, int k0) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x8*>(X + (r0 + (l & 15)) * Sweep8Lds::LD + k0 + 8 * (l >> 4));
}

// The same operand scaled by s[k] (k in the logical column order).
__device__ __forceinline__ bf16x8 lscaled(const bf16_t* X, int r0, int k0, const float* s) {
  const int g4 = 4 * (lane_id() >> 4);
  const bf16x8 x = lfrag(X, r0, k0);
  const float4 a = *reinterpret_cast<const float4*>(s + k0 + g4);
  const float4 b = *reinterpret_cast<const float4*>(s + k0 + 16 + g4);
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

// ---- global loads -----------------------------------------------------------------------
// Raw buffer loads over one (b, h) pair's slice of an input: a load whose byte offset
// falls outside [0, bytes) returns zero, which is exactly the zero padding the chunk
// needs for tokens before the sequence start and past its end.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferFlags = 0x00020000;  // raw (untyped) access on CDNA

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// The 4x4 blocks of a [64][64] tile dealt to the 256 threads of one role: role thread q
// takes token rows 4 rq .. 4 rq + 3 and columns c4 .. c4 + 3, rq = 4 (q / 64) + q % 4,
// so wave j of a role covers rows 16 j .. 16 j + 15.  A 16-lane group holds a 4 x 4
// patch of blocks: its row-major and its transposed 8-byte stores both hit 32 banks.
__device__ __forceinline__ void quad_map(int q, int& rq, int& c4) {
  const int l = q & 63;
  rq = 4 * (q >> 6) + (l & 3);
  c4 = 4 * (4 * (l >> 4) + ((l >> 2) & 3));
}

// Loads of N rows of 4 columns: row r at byte offset off0 + r * row_bytes.
template <int N>
__device__ __forceinline__ void quad_fetch(uint2* x, rsrc_t r, int off0, int row_bytes) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = bload8(r, off0 + i * row_bytes);
}

// A fetched 4x4 block (rows 4 rq .., columns c4 ..) into LDS, row-major and / or transposed.
__device__ __forceinline__ void quad_store(const uint2* x, bf16_t* dst, bf16_t* dstT, int rq, int c4) {
  constexpr int LD = Sweep8Lds::LD;
  bf16x4 rows[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    rows[r] = __builtin_bit_cast(bf16x4, x[r]);
    if (dst != nullptr) *reinterpret_cast<uint2*>(dst + (4 * rq + r) * LD + pcol(c4)) = x[r];
  }
  if (dstT != nullptr) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x4 col = {rows[0][c], rows[1][c], rows[2][c], rows[3][c]};
      *reinterpret_cast<bf16x4*>(dstT + (c4 + c) * LD + pcol(4 * rq)) = col;
    }
  }
}

// Everything both roles need to know about the workgroup's segment.
struct Sweep8Ctx {
  unsigned char* smem;
  rsrc_t rq_, rk_, rv_, ru_, rg_;  // buffers over the pair's q, k, v, u, gamma
  rsrc_t rh_;                      // buffer over the pair's 3 value rows before the sequence
  bool hist;                       // those rows are given (else they are zero)
  const float *gg, *bb, *al;       // the pair's g, beta, alpha
  float *oloc, *qhat_base, *agg;   // outputs of this pair / segment
  int T, L, Lm1, c_begin, c_end, Tpad, pr, nch;
  int ubytes;                      // bytes per token row of u / gamma
};

// LDS views.
struct Sweep8View {
  bf16_t *sQ, *sK, *sKt, *sVt, *sHt, *sAt, *sM, *sWc, *sMinv, *sWct, *sTd, *sEt;
  float *sB, *sG, *sD, *sBeta, *sBG, *sAlphaT, *sTaps, *sMt;
  unsigned char* slot0;
  __device__ __forceinline__ explicit Sweep8View(unsigned char* smem) {
    using Ly = Sweep8Lds;
    sQ = reinterpret_cast<bf16_t*>(smem + Ly::oQ);
    sK = reinterpret_cast<bf16_t*>(smem + Ly::oK);
    sKt = reinterpret_cast<bf16_t*>(smem + Ly::oKt);
    sVt = reinterpret_cast<bf16_t*>(smem + Ly::oVt);
    sHt = reinterpret_cast<bf16_t*>(smem + Ly::oHt);
    sAt = reinterpret_cast<bf16_t*>(smem + Ly::oAt);
    sM = reinterpret_cast<bf16_t*>(smem + Ly::oM);
    sWc = sM;  // Wc takes M's space once the inverse is built
    sMinv = reinterpret_cast<bf16_t*>(smem + Ly::oMinv);
    sWct = reinterpret_cast<bf16_t*>(smem + Ly::oWct);
    sTd = reinterpret_cast<bf16_t*>(smem + Ly::oTd);
    sB = reinterpret_cast<float*>(smem + Ly::oGate);
    sG = sB + 64;
    sD = sG + 64;
    sBeta = sD + 64;
    sBG = sBeta + 64;
    sAlphaT = sBG + 64;  // [8][64]
    sTaps = sAlphaT + 8 * 64;  // [4][64]
    sMt = reinterpret_cast<float*>(smem + Ly::oMt);  // [4 waves][16][kMtLd]
    slot0 = smem + Ly::oSlot;
    sEt = slotU(1);
  }
  __device__ __forceinline__ bf16_t* slotU(int s) const {
    return reinterpret_cast<bf16_t*>(slot0 + (size_t)s * Sweep8Lds::szSlot);
  }
  __device__ __forceinline__ bf16_t* slotUt(int s) const { return slotU(s) + 64 * Sweep8Lds::LD; }
  __device__ __forceinline__ bf16_t* slotRt(int s) const { return slotU(s) + 2 * 64 * Sweep8Lds::LD; }
};

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8 within each row
// of 16 lanes, then row 15's total into the next row and row 31's into rows 2 and 3 (DPP).
__device__ __forceinline__ float wave_inclusive_sum(float x) {
#define PRISM_ADD_DPP(CTRL, ROWS)                                                              \
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, true));
  PRISM_ADD_DPP(0x111, 0xF)  // row_shr:1
  PRISM_ADD_DPP(0x112, 0xF)  // row_shr:2
  PRISM_ADD_DPP(0x114, 0xF)  // row_shr:4
  PRISM_ADD_DPP(0x118, 0xF)  // row_shr:8
  PRISM_ADD_DPP(0x142, 0xA)  // row_bcast:15 into rows 1 and 3
  PRISM_ADD_DPP(0x143, 0xC)  // row_bcast:31 into rows 2 and 3
#undef PRISM_ADD_DPP
  return x;
}

// Decay factors of the Gram tiles of token row block rb: lane (li, g) of tile jt holds
// Gam(i, j) = exp(b_i - b_j) for i = 16 rb + li, j = 16 jt + 4g + r, zero where j > i
// (or j >= i when strict) and for tiles above the diagonal.
__device__ __forceinline__ void decay_factors(float (&dec)[4][4], const float* sB, int rb, bool strict) {
  const int l = lane_id(), g4 = 4 * (l >> 4), li = l & 15;
  const int i = 16 * rb + li;
  const float bi = sB[i];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const float4 bj = *reinterpret_cast<const float4*>(sB + 16 * jt + g4);
    const float bjr[4] = {bj.x, bj.y, bj.z, bj.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * jt + g4 + r;
      const bool ok = strict ? (j < i) : (j <= i);
      dec[jt][r] = (jt <= rb && ok) ? __expf(bi - bjr[r]) : 0.f;
    }
  }
}

// Masked, decayed Gram rows rb of (X Y^T) as a 64-deep A operand (contraction over the
// token j), from raw tiles [j][i] = Y_j . X_i; `sign` folds a negation in.
__device__ __forceinline__ void gram_rows(bf16x8 (&fa)[2], const bf16_t* sY, const bf16_t* sX, int rb,
                                          const float (&dec)[4][4], float sign) {
  constexpr int LD = Sweep8Lds::LD;
  f32x4 raw[4];
  const bf16x8 x0 = lfrag(sX, 16 * rb, 0), x1 = lfrag(sX, 16 * rb, 32);
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    raw[jt] = zero4();
    if (jt <= rb) {
      raw[jt] = mfma(lfrag(sY, 16 * jt, 0), x0, raw[jt]);
      raw[jt] = mfma(lfrag(sY, 16 * jt, 32), x1, raw[jt]);
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
__device__ __forceinline__ void sweep8_kwave(const Sweep8Ctx& x, int wq) {
  constexpr int LD = Sweep8Lds::LD, LDT = Sweep8Lds::LDT, C = 64;
  const Sweep8View V(x.smem);
  const int l = lane_id(), g4 = 4 * (l >> 4), li = l & 15;
  const int rb = 3 - wq, cb = wq;
  int rq, c4;
  quad_map(threadIdx.x & 255, rq, c4);
  // LM1S >= 0 fixes L - 1 at compile time: the rank-L steps are then unrolled, so the
  // wait for each prefetched operand counts only the loads issued before it.
  const int Lm1 = LM1S >= 0 ? LM1S : x.Lm1;
  const int NL = Lm1 > 3 ? Lm1 : 3, L = Lm1 + 1;

  f32x4 H[4], Vp[4], HB[4], WH[4];
  float dec[4][4];
  uint2 pf[12], lpf[4];
  float glg = 1.f, gbe = 0.f, gal[8];  // wave 0: next chunk's gates for token t0 + lane
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) H[kt] = zero4();
#pragma unroll
  for (int j = 0; j < 8; ++j) gal[j] = 0.f;

  auto fetch_chunk = [&](int c) {
    const int t0 = c * C;
    const int o = (t0 + 4 * rq) * 128 + 2 * c4;
    quad_fetch<4>(pf + 0, x.rq_, o, 128);
    quad_fetch<4>(pf + 4, x.rk_, o, 128);
    if (L > 1) quad_fetch<4>(pf + 8, x.ru_, (t0 + 4 * rq) * x.ubytes + 2 * c4, x.ubytes);
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
    quad_store(pf + 0, V.sQ, nullptr, rq, c4);
    quad_store(pf + 4, V.sK, V.sKt, rq, c4);
    if (L > 1) quad_store(pf + 8, V.slotU(0), V.slotUt(0), rq, c4);
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

    // ---- P0: M[i][j] = beta_i Gam_ij K_i.K_j (j < i) rows rb; diagonal inverse block --
    const int cn = c + 1 < x.c_end ? c + 1 : c;  // next chunk (this one again at the end:
                                                  // unconditional loads keep waits exact)
    {
      // the diagonal tile first (its operands are the row block's own fragments): the
      // inverse of the diagonal block is the longest chain of the phase
      const bf16x8 k0 = lfrag(V.sK, 16 * rb, 0), k1 = lfrag(V.sK, 16 * rb, 32);
      f32x4 draw = mfma(k0, k0, zero4());
      draw = mfma(k1, k1, draw);
      decay_factors(dec, V.sB, rb, true);
      f32x4 mraw[4];
#pragma unroll
      for (int jt = 0; jt < 3; ++jt) {
        mraw[jt] = zero4();
        if (jt < rb) {
          mraw[jt] = mfma(lfrag(V.sK, 16 * jt, 0), k0, mraw[jt]);
          mraw[jt] = mfma(lfrag(V.sK, 16 * jt, 32), k1, mraw[jt]);
        }
      }
      const float beil = V.sBeta[16 * rb + li];
#pragma unroll
      for (int jt = 0; jt < 3; ++jt) {
        if (jt < rb) {
          bf16x4 mv;
#pragma unroll
          for (int r = 0; r < 4; ++r) mv[r] = (bf16_t)(beil * dec[jt][r] * mraw[jt][r]);
          *reinterpret_cast<bf16x4*>(V.sM + (16 * rb + li) * LD + pcol(16 * jt + g4)) = mv;
        }
      }
      // T_rb = (I + M_rb,rb)^-1 = (I + Y)(I + Y^2)(I + Y^4)(I + Y^8), Y = -M_rb,rb (bf16
      // products, float32 sums), unless a power of Y grows past 1: the product then
      // cancels large terms to a bounded inverse, which bf16 cannot resolve, and the wave
      // takes float32 forward substitution instead (one key repeated with beta near 1)
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
        float* Mt = V.sMt + wq * 16 * kMtLd;  // this wave's M^T: Mt[li][g4 + r] = M[g4 + r][li]
        *reinterpret_cast<float4*>(Mt + li * kMtLd + g4) = make_float4(-Y[0], -Y[1], -Y[2], -Y[3]);
        __builtin_amdgcn_wave_barrier();  // the wave's LDS stores land before its reads (in order)
        const f32x4 tc = diag_inverse_subst(Mt);  // T[g4 + r][li]
#pragma unroll
        for (int r = 0; r < 4; ++r) V.sTd[(16 * rb + g4 + r) * LDT + li] = (bf16_t)tc[r];
      }
    }
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) {  // V' starts as V (rows rb); the rank-L state term at zero
      const bf16x4 xv = *reinterpret_cast<const bf16x4*>(V.sVt + (16 * vt + li) * LD + pcol(16 * rb + g4));
#pragma unroll
      for (int r = 0; r < 4; ++r) Vp[vt][r] = (float)xv[r];
      HB[vt] = zero4();
    }
    if (Lm1 >= 2) quad_fetch<4>(lpf, x.ru_, (t0 + 4 * rq) * x.ubytes + 128 + 2 * c4, x.ubytes);  // U_2
    __syncthreads();  // B1: M, diagonal inverse blocks, R_1

    // ---- P1 .. P_NL: rank-L steps ---------------------------------------------------------
    auto level_phase = [&](const int lv) {
      const int s = (lv - 1) & 1;
      if (lv <= Lm1) {
        const bf16_t* sU = V.slotU(s);
        const bf16_t* sUt = V.slotUt(s);
        const bf16_t* sRt = V.slotRt(s);
        bf16x8 xa[2];  // -strict(Gam * K U_l^T) rows rb
        gram_rows(xa, sU, V.sK, rb, dec, -1.f);
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) {  // V' += X1 R_l
          Vp[vt] = mfma(xa[0], lfrag(sRt, 16 * vt, 0), Vp[vt]);
          if (rb >= 2) Vp[vt] = mfma(xa[1], lfrag(sRt, 16 * vt, 32), Vp[vt]);
        }
        // HB(:, cb) += U_l^T diag(D) R_l(:, cb)
        const bf16x8 rd0 = lscaled(sRt, 16 * cb, 0, V.sD);
        const bf16x8 rd1 = lscaled(sRt, 16 * cb, 32, V.sD);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          HB[kt] = mfma(lfrag(sUt, 16 * kt, 0), rd0, HB[kt]);
          HB[kt] = mfma(lfrag(sUt, 16 * kt, 32), rd1, HB[kt]);
        }
      }
      if (lv == 2) {
        // Wc(:, cb) = (I + M)^-1 diag(beta G) K(:, cb), row-major and transposed (the
        // inverse's column blocks come from the Q waves' phase 1)
        const bf16x8 k0 = lscaled(V.sKt, 16 * cb, 0, V.sBG);
        const bf16x8 k1 = lscaled(V.sKt, 16 * cb, 32, V.sBG);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          f32x4 acc = mfma(lfrag(V.sMinv, 16 * it, 0), k0, zero4());
          if (it >= 2) acc = mfma(lfrag(V.sMinv, 16 * it, 32), k1, acc);
          const bf16x4 xv = to_bf16x4(acc);  // Wc[16 it + g4 + r][16 cb + li]
          *reinterpret_cast<bf16x4*>(V.sWct + (16 * cb + li) * LD + pcol(16 * it + g4)) = xv;
#pragma unroll
          for (int r = 0; r < 4; ++r) V.sWc[(16 * it + g4 + r) * LD + pcol(16 * cb + li)] = xv[r];
        }
      }
      if (lv == 3) {  // WH = Wc H(:, cb), Wc from phase 2
        const bf16x8 h0 = pair8(H[0], H[1]), h1 = pair8(H[2], H[3]);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const f32x4 acc = mfma(lfrag(V.sWc, 16 * it, 0), h0, zero4());
          WH[it] = mfma(lfrag(V.sWc, 16 * it, 32), h1, acc);
        }
      }
      if (lv + 1 <= Lm1) {  // U_{lv+1} into the other slot, then fetch U_{lv+2}
        quad_store(lpf, V.slotU(s ^ 1), V.slotUt(s ^ 1), rq, c4);
        if (lv + 2 <= Lm1)
          quad_fetch<4>(lpf, x.ru_, (t0 + 4 * rq) * x.ubytes + (lv + 1) * 128 + 2 * c4, x.ubytes);
      }
      // next chunk's inputs, issued once this chunk's last rank-L prefetch is consumed (the
      // wait for a prefetched operand may cover every load issued before it)
      if (lv == (Lm1 >= 2 ? Lm1 - 1 : 1)) fetch_chunk(cn);
      if (lv == NL) {  // (beta V')^T rows rb for the per-column solve
        const float4 be = *reinterpret_cast<const float4*>(V.sBeta + 16 * rb + g4);
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) {
          const bf16x4 xv = {(bf16_t)(be.x * Vp[vt][0]), (bf16_t)(be.y * Vp[vt][1]), (bf16_t)(be.z * Vp[vt][2]),
                             (bf16_t)(be.w * Vp[vt][3])};
          *reinterpret_cast<bf16x4*>(V.sVt + (16 * vt + li) * LD + pcol(16 * rb + g4)) = xv;
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
      const bf16x8 v0 = lfrag(V.sVt, 16 * cb, 0), v1 = lfrag(V.sVt, 16 * cb, 32);
      f32x4 E[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 acc = mfma(lfrag(V.sMinv, 16 * it, 0), v0, zero4());
        if (it >= 2) acc = mfma(lfrag(V.sMinv, 16 * it, 32), v1, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) E[it][r] = acc[r] - WH[it][r];
        *reinterpret_cast<bf16x4*>(V.sEt + (16 * cb + li) * LD + pcol(16 * it + g4)) = to_bf16x4(E[it]);
      }
      const bf16x8 e0 = scaled_pair(E[0], E[1], V.sD, 0), e1 = scaled_pair(E[2], E[3], V.sD, 32);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        f32x4 he = mfma(lfrag(V.sKt, 16 * kt, 0), e0, zero4());
        he = mfma(lfrag(V.sKt, 16 * kt, 32), e1, he);
#pragma unroll
        for (int r = 0; r < 4; ++r) H[kt][r] = GC * H[kt][r] + he[r] + HB[kt][r];
      }
    }
    __syncthreads();  // E^T in LDS; every read of the old H^T is done

    // ---- P_O: new H^T; next chunk into LDS ---------------------------------------------------
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      *reinterpret_cast<bf16x4*>(V.sHt + (16 * cb + li) * LD + pcol(16 * kt + g4)) = to_bf16x4(H[kt]);
    if (c + 1 < x.c_end) store_chunk(c + 1);
  }
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) x.agg[(16 * kt + g4 + r) * 64 + 16 * cb + li] = H[kt][r];
}

// ---- the Q waves ------------------------------------------------------------------------
// NLG: the chain's factor slots hold gains p and each factor is p Phi(p r) of the running
// residual, rounded to bfloat16 (the nonlinear refinement, as nl_gain_kernel computes it).
// DLT: the written-correction chain (d = gamma r, r <- r - d, written alpha d; the factor
// slots hold the corrections' per-channel factors) in place of r <- r (1 - alpha gamma).
template <int LM1S, bool NLG, bool DLT>
__device__ __forceinline__ void sweep8_qwave(const Sweep8Ctx& x, int wq) {
  constexpr int LD = Sweep8Lds::LD, LDT = Sweep8Lds::LDT, C = 64;
  const Sweep8View V(x.smem);
  const int l = lane_id(), g4 = 4 * (l >> 4), li = l & 15;
  const int rb = wq, cb = wq;
  int rq, c4;
  quad_map(threadIdx.x & 255, rq, c4);
  // LM1S >= 0 fixes L - 1 at compile time: the rank-L steps are then unrolled, so the
  // wait for each prefetched operand counts only the loads issued before it.
  const int Lm1 = LM1S >= 0 ? LM1S : x.Lm1;
  const int NL = Lm1 > 3 ? Lm1 : 3, L = Lm1 + 1;

  f32x4 A[4], O[4], WA[4];
  float rr[4][4];  // residual r_l of this lane's 4x4 block [row][col]
  float dec[4][4];
  bf16x8 Pa[2];
  uint2 pf[12], lpf[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    f32x4 t = zero4();
    if (kt == cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = (g4 + r == li) ? 1.f : 0.f;
    }
    A[kt] = t;
  }

  auto fetch_chunk = [&](int c) {
    const int t0 = c * C;
    // the 4 rows before the block, then the block: a negative base (before the sequence
    // start) only ever occurs for the first of the two, whose rows are then all padding
    quad_fetch<4>(pf + 0, x.rv_, (t0 - 4 + 4 * rq) * 128 + 2 * c4, 128);
    quad_fetch<4>(pf + 4, x.rv_, (t0 + 4 * rq) * 128 + 2 * c4, 128);
    if (L > 1) quad_fetch<4>(pf + 8, x.rg_, (t0 + 4 * rq) * x.ubytes + 2 * c4, x.ubytes);  // gamma_0
  };
  // V^T into LDS (the v rows stay in registers for the anchor)
  auto store_chunk = [&]() {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const bf16x4 col = {__builtin_bit_cast(bf16x4, pf[4])[cc], __builtin_bit_cast(bf16x4, pf[5])[cc],
                          __builtin_bit_cast(bf16x4, pf[6])[cc], __builtin_bit_cast(bf16x4, pf[7])[cc]};
      *reinterpret_cast<bf16x4*>(V.sVt + (c4 + cc) * LD + pcol(4 * rq)) = col;
    }
  };
  // the residual r_0 = v - anchor of the block (anchor_t = sum_j w_j v_{t-3+j})
  auto anchor = [&]() {
    float vv[8][4];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const bf16x4 b4 = __builtin_bit_cast(bf16x4, pf[r]);
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
  // R_lv = alpha_lv r_lv, r_lv = r_{lv-1} (1 - alpha_{lv-1} gamma_{lv-1}), gamma_{lv-1} in gx;
  // written transposed into slot s
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
      *reinterpret_cast<bf16x4*>(dst + (c4 + cc) * LD + pcol(4 * rq)) = col;
    }
  };

  if (x.c_begin < x.c_end) {
    fetch_chunk(x.c_begin);
    if (x.c_begin == 0 && x.hist) {
      // the first chunk of the sequence: tokens -3 .. -1 of the anchor window come from the
      // given history (block row rq = 0 holds tokens -4 .. -1; the other lanes read past
      // the buffer, which returns zero, and keep their rows)
      const int base = rq == 0 ? 2 * c4 : 4096;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const uint2 hv = bload8(x.rh_, base + j * 128);
        pf[1 + j].x |= hv.x;
        pf[1 + j].y |= hv.y;
      }
    }
    store_chunk();
  }
  for (int c = x.c_begin; c < x.c_end; ++c) {
    const int t0 = c * C;
    const int cn = c + 1 < x.c_end ? c + 1 : c;  // next chunk (unconditional loads)
    __syncthreads();  // B0

    // ---- P0: P = lower(Gam * Q K^T) rows rb (registers); r_0 and R_1 ------------------------
    if (L > 1) anchor();
    decay_factors(dec, V.sB, rb, false);
    gram_rows(Pa, V.sK, V.sQ, rb, dec, 1.f);
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) O[vt] = zero4();
    if (Lm1 >= 1) residual_step(pf + 8, 1, 0);
    if (Lm1 >= 2) quad_fetch<4>(lpf, x.rg_, (t0 + 4 * rq) * x.ubytes + 128 + 2 * c4, x.ubytes);  // gamma_1
    __syncthreads();  // B1

    // ---- P1 .. P_NL: rank-L steps; M^-1 (P1), WA and Qhat (P3) -------------------------------
    auto level_phase = [&](const int lv) {
      const int s = (lv - 1) & 1;
      if (lv <= Lm1) {  // O += lower(Gam * Q U_l^T) R_l
        const bf16_t* sU = V.slotU(s);
        const bf16_t* sRt = V.slotRt(s);
        bf16x8 xa[2];
        gram_rows(xa, sU, V.sQ, rb, dec, 1.f);
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) {
          O[vt] = mfma(xa[0], lfrag(sRt, 16 * vt, 0), O[vt]);
          if (rb >= 2) O[vt] = mfma(xa[1], lfrag(sRt, 16 * vt, 32), O[vt]);
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
                const bf16x4 am = *reinterpret_cast<const bf16x4*>(V.sM + (16 * i + li) * LD + pcol(16 * kk + g4));
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
          for (int r = 0; r < 4; ++r) V.sMinv[(16 * i + g4 + r) * LD + pcol(16 * cb + li)] = xv[r];
        }
      } else if (lv == 3) {
        // WA = Wc A_acc(:, cb)
        const bf16x8 a0 = pair8(A[0], A[1]), a1 = pair8(A[2], A[3]);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const f32x4 acc = mfma(lfrag(V.sWc, 16 * it, 0), a0, zero4());
          WA[it] = mfma(lfrag(V.sWc, 16 * it, 32), a1, acc);
        }
        // Qtilde^T = (diag(G) Q)^T - Wc^T P^T (dk rows kt, tokens rb); Qhat^T = A_acc^T Qtilde^T
        const float Gi = V.sG[16 * rb + li];
        f32x4 Qt[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const bf16x4 qv = *reinterpret_cast<const bf16x4*>(V.sQ + (16 * rb + li) * LD + pcol(16 * kt + g4));
          f32x4 pw = mfma(lfrag(V.sWct, 16 * kt, 0), Pa[0], zero4());
          if (rb >= 2) pw = mfma(lfrag(V.sWct, 16 * kt, 32), Pa[1], pw);
#pragma unroll
          for (int r = 0; r < 4; ++r) Qt[kt][r] = Gi * (float)qv[r] - pw[r];
        }
        const bf16x8 q0 = pair8(Qt[0], Qt[1]), q1 = pair8(Qt[2], Qt[3]);
        // lane (li, g) holds Qhat[16 rb + li][16 kt + 4 g + r]: tiles 2 kb and 2 kb + 1 are
        // exactly its 32-deep A operand for k block kb
        bf16_t* qf = reinterpret_cast<bf16_t*>(x.qhat_base) + ((size_t)c * 4 + rb) * 1024 + l * 8;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x4 e0 = mfma(lfrag(V.sAt, 32 * kb, 0), q0, zero4());
          e0 = mfma(lfrag(V.sAt, 32 * kb, 32), q1, e0);
          f32x4 e1 = mfma(lfrag(V.sAt, 32 * kb + 16, 0), q0, zero4());
          e1 = mfma(lfrag(V.sAt, 32 * kb + 16, 32), q1, e1);
          *reinterpret_cast<bf16x8*>(qf + kb * 512) = pair8(e0, e1);
        }
      }
      if (lv + 1 <= Lm1) {  // R_{lv+1} into the other slot, then fetch gamma_{lv+1}
        residual_step(lpf, lv + 1, s ^ 1);
        if (lv + 2 <= Lm1)
          quad_fetch<4>(lpf, x.rg_, (t0 + 4 * rq) * x.ubytes + (lv + 1) * 128 + 2 * c4, x.ubytes);
      }
      // next chunk's inputs, issued once this chunk's last rank-L prefetch is consumed (the
      // wait for a prefetched operand may cover every load issued before it)
      if (lv == (Lm1 >= 2 ? Lm1 - 1 : 1)) fetch_chunk(cn);
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
      const float4 G4 = *reinterpret_cast<const float4*>(V.sG + 16 * rb + g4);
      const float Gr[4] = {G4.x, G4.y, G4.z, G4.w};
      const bf16x8 q0 = lfrag(V.sQ, 16 * rb, 0), q1 = lfrag(V.sQ, 16 * rb, 32);
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) {
        f32x4 qh = mfma(q0, lfrag(V.sHt, 16 * vt, 0), zero4());
        qh = mfma(q1, lfrag(V.sHt, 16 * vt, 32), qh);
#pragma unroll
        for (int r = 0; r < 4; ++r) O[vt][r] += Gr[r] * qh[r];
      }
      const bf16x8 w0 = scaled_pair(WA[0], WA[1], V.sD, 0), w1 = scaled_pair(WA[2], WA[3], V.sD, 32);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        f32x4 aw = mfma(lfrag(V.sKt, 16 * kt, 0), w0, zero4());
        aw = mfma(lfrag(V.sKt, 16 * kt, 32), w1, aw);
#pragma unroll
        for (int r = 0; r < 4; ++r) A[kt][r] = GC * A[kt][r] - aw[r];
        *reinterpret_cast<bf16x4*>(V.sAt + (16 * cb + li) * LD + pcol(16 * kt + g4)) = to_bf16x4(A[kt]);
      }
    }
    __syncthreads();  // E^T in LDS

    // ---- P_O: O += P E, write O_loc; next chunk's V^T and residual ------------------------------
    {
      bf16_t* of = reinterpret_cast<bf16_t*>(x.oloc) + ((size_t)c * 4 + rb) * 1024 + l * 4;
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) {
        O[vt] = mfma(Pa[0], lfrag(V.sEt, 16 * vt, 0), O[vt]);
        if (rb >= 2) O[vt] = mfma(Pa[1], lfrag(V.sEt, 16 * vt, 32), O[vt]);
        *reinterpret_cast<bf16x4*>(of + vt * 256) = to_bf16x4(O[vt]);
      }
    }
    if (c + 1 < x.c_end) store_chunk();
  }
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) x.agg[(16 * kt + g4 + r) * 64 + 16 * cb + li] = A[kt][r];
}

template <int D, int C, int LM1S, bool NLG, bool DLT>
__device__ __forceinline__ void sweep8_run(FwdArgs a) {
  static_assert(D == 64 && C == 64, "the two-wave sweep is written for head dim 64 and 64-token chunks");
  __shared__ __align__(16) unsigned char smem[Sweep8Lds::total];
  const Sweep8View V(smem);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seg = blockIdx.x, pr = blockIdx.y;
  const int hd = pr % a.H;
  const int T = a.T, L = a.L, Lm1 = L - 1;

  Sweep8Ctx x;
  x.smem = smem;
  x.T = T;
  x.L = L;
  x.Lm1 = Lm1;
  x.c_begin = seg * a.seg_chunks;
  x.c_end = min(a.nch, x.c_begin + a.seg_chunks);
  x.Tpad = a.nch * C;
  x.pr = pr;
  x.nch = a.nch;
  x.ubytes = (L > 1 ? Lm1 : 1) * D * 2;
  const size_t pair_rows = (size_t)pr * T;
  const unsigned vbytes = (unsigned)T * D * 2;
  const unsigned ubytes_all = (unsigned)T * (unsigned)x.ubytes;
  x.rq_ = make_rsrc(reinterpret_cast<const bf16_t*>(a.q) + pair_rows * D, vbytes);
  x.rk_ = make_rsrc(reinterpret_cast<const bf16_t*>(a.k) + pair_rows * D, vbytes);
  x.rv_ = make_rsrc(reinterpret_cast<const bf16_t*>(a.v) + pair_rows * D, vbytes);
  x.ru_ = make_rsrc(L > 1 ? reinterpret_cast<const bf16_t*>(a.u) + pair_rows * Lm1 * D : a.q, L > 1 ? ubytes_all : 0u);
  x.rg_ = make_rsrc(L > 1 ? reinterpret_cast<const bf16_t*>(a.gamma) + pair_rows * Lm1 * D : a.q,
                    L > 1 ? ubytes_all : 0u);
  x.hist = a.conv_in != nullptr;
  x.rh_ = make_rsrc(x.hist ? reinterpret_cast<const bf16_t*>(a.conv_in) + (size_t)pr * 3 * D : a.q,
                    x.hist ? 3u * D * 2u : 0u);
  x.gg = a.g + pair_rows;
  x.bb = a.beta + pair_rows;
  x.al = L > 1 ? a.alpha + pair_rows * L : nullptr;
  // O_loc and Qhat in fragment order: per chunk and token row block, the lanes' MFMA
  // tiles back to back (O_loc: 4 value tiles of 64 lanes x 4; Qhat: 2 k blocks of
  // 64 lanes x 8), bfloat16
  x.oloc = reinterpret_cast<float*>(reinterpret_cast<bf16_t*>(a.Oloc) + (size_t)pr * a.nch * 4096);
  x.qhat_base = reinterpret_cast<float*>(reinterpret_cast<bf16_t*>(a.Qhat) + (size_t)pr * a.nch * 4096);
  x.agg = (w < 4 ? a.Bagg : a.Aagg) + ((size_t)pr * a.nseg + seg) * D * D;

  // conv taps, H^T = 0, A_acc^T = I
  const float* cw = a.conv_w + (size_t)hd * 4 * D;
  for (int i = tid; i < 4 * D; i += 512) V.sTaps[i] = L > 1 ? cw[i] : 0.f;
  for (int i = tid; i < D * D; i += 512) {
    const int r = i / D, c = i % D;
    V.sHt[r * Sweep8Lds::LD + pcol(c)] = (bf16_t)0.f;
    V.sAt[r * Sweep8Lds::LD + pcol(c)] = (bf16_t)(r == c ? 1.f : 0.f);
  }
  __syncthreads();
  // Both roles pass the same barriers in the same order: B0, B1, one per phase
  // P1 .. P_NL and one after the state phase, for every chunk of the segment.
  if (w < 4) sweep8_kwave<LM1S>(x, w);
  else sweep8_qwave<LM1S, NLG, DLT>(x, w - 4);
}

template <int D, int C, int LM1S>
__global__ __launch_bounds__(512, 1) void seg_sweep8_kernel(FwdArgs a) {
  sweep8_run<D, C, LM1S, false, false>(a);
}

// the same sweep with the nonlinear refinement: a.gamma holds the gains p
template <int D, int C, int LM1S>
__global__ __launch_bounds__(512, 1) void seg_sweep8_nl_kernel(FwdArgs a) {
  sweep8_run<D, C, LM1S, true, false>(a);
}

// the same sweep with the written-correction chain: a.gamma holds the corrections' factors
template <int D, int C, int LM1S>
__global__ __launch_bounds__(512, 1) void seg_sweep8_delta_kernel(FwdArgs a) {
  sweep8_run<D, C, LM1S, false, true>(a);
}

}  // namespace prism
