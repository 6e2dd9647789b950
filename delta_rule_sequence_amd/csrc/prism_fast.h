// prism_fast.h - the bfloat16, head dim 64 path (gfx950): MFMA helpers shared with the
// two-wave sweep (prism_sweep8.h), the inter-segment scan and the output correction.
//
// The path computes, per (b, h) pair, the segment operators (A_s, B_s) of the chunked
// UT / WY form in the sweep, then H_in(s+1) = A_s H_in(s) + B_s over the segments
// (scan), then o = O_loc + Qhat H_in(segment) (output correction).
#pragma once
#include "prism_kernels.h"

namespace prism {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
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

// Z = A * B for 16x16 tiles held as MFMA accumulators, A given by the tile of A^T and B
// by its own tile: one 16x16x16 MFMA on the bfloat16-rounded operands, float32 sums.
__device__ __forceinline__ f32x4 mm16_bf16(const f32x4& At, const f32x4& Bt) {
  return mfma16(to_bf16x4(At), to_bf16x4(Bt), zero4());
}

// T = (I + M)^-1 of a strictly lower triangular 16 x 16 block M by forward substitution in
// float32.  The 16 lanes c of each lane group g take column c, rows 4 g .. 4 g + 3, and the
// lane holding x_j hands it to the others of its column (one shuffle per step), so a lane
// keeps four unknowns; it returns T[4 g + r][c], r = 0..3.  Mt is M^T in the wave's own LDS
// ([16][kMtLd] floats, Mt[j][r] = M[r][j], zero where r <= j), written by the caller, who
// has also waited for its own stores.  Stable whatever the size of M's entries, where the
// product form (I + Y)(I + Y^2)(I + Y^4)(I + Y^8) with Y = -M sums powers that grow like
// binomial coefficients when |M| is near 1 (one key repeated over the block with beta near
// 1) and cancel to a bounded inverse only in exact arithmetic.
constexpr int kMtLd = 20;  // row stride of Mt (floats)
__device__ __forceinline__ f32x4 diag_inverse_subst(const float* Mt) {
  const int l = lane_id(), c = l & 15, g = l >> 4;
  f32x4 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = 4 * g + e == c ? 1.f : 0.f;
#pragma unroll
  for (int j = 0; j < 15; ++j) {
    const float xj = __shfl(x[j & 3], c + 16 * (j >> 2));  // x_j, final after step j - 1
    const float4 m = *reinterpret_cast<const float4*>(Mt + j * kMtLd + 4 * g);
    const float mv[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * g + e > j) x[e] -= mv[e] * xj;
  }
  return x;
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
// (pair, 2 state columns c0 ..), 256 workgroups at 8 pairs.  Thread t takes state rows
// i0 = 2 (t / 8), i0 + 1 and the contraction slice k = 8 q .. 8 q + 7 (q = t % 8): it keeps
// those 16 entries of A_s in registers (loaded DEPTH steps ahead, so a step never waits on
// memory), reads rows 8 q .. 8 q + 7 of the two H_in(s) columns from LDS (skewed so the
// eight slices of a wave hit distinct banks) and forms 2 x 2 partial sums; three DPP
// exchange rounds within the 8 lanes of the row pair leave lanes q and q ^ 1 with
// H_in(s+1)[i0 + q / 4][c0 + (q / 2) % 2].  One barrier per step.
template <int DK, int DV>
__global__ __launch_bounds__(256) void seg_scan_fast_kernel(FwdArgs a) {
  static_assert(DK == 64, "the row-pair / k-slice split assumes 64 state rows");
  constexpr int DEPTH = 8;
  constexpr int HS = DK + DK / 8;  // H rows with a one-row skew every 8 rows
  __shared__ __align__(16) float2 sH[2][HS];
  const int tid = threadIdx.x, i0 = 2 * (tid >> 3), q = tid & 7;
  const int pr = blockIdx.x, c0 = 2 * blockIdx.y;
  const int nseg = a.nseg;
  const int orow = i0 + (q >> 2), ocol = c0 + ((q >> 1) & 1);  // the output this lane ends with (lanes q, q ^ 1)
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
  // H_in(s)[orow][ocol], from the starting state (zero unless given)
  float h = a.S0 != nullptr ? a.S0[(size_t)pr * DK * DV + (size_t)orow * DV + ocol] : 0.f;
  // the LDS copy of the four columns the products read: row tid of H_in(0)
  if (tid < DK)
    sH[0][hrow(tid)] = a.S0 != nullptr
                           ? *reinterpret_cast<const float2*>(a.S0 + (size_t)pr * DK * DV + (size_t)tid * DV + c0)
                           : make_float2(0.f, 0.f);
  __syncthreads();
  const bool lo4 = q < 4, lo2 = (q & 2) == 0;
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
    float v[4] = {0.f, 0.f, 0.f, 0.f}; /* [row][col] */                                       \
    _Pragma("unroll") for (int m = 0; m < 8; ++m) {                                           \
      const float2 hv = sH[cur][hrow(8 * q + m)];                                             \
      v[0] += ar0[m] * hv.x;                                                                  \
      v[1] += ar0[m] * hv.y;                                                                  \
      v[2] += ar1[m] * hv.x;                                                                  \
      v[3] += ar1[m] * hv.y;                                                                  \
    }                                                                                         \
    /* refill the slot after the products: the loads queue while the exchanges run */         \
    if (PREFETCH) PRISM_FETCH(D, s + DEPTH)                                                   \
    /* keep row q / 4, then columns (q & 2) .., then column q & 3 */                          \
    float n2[2];                                                                              \
    _Pragma("unroll") for (int j = 0; j < 2; ++j)                                             \
      n2[j] = (lo4 ? v[j] : v[2 + j]) + dpp_half_mirror(lo4 ? v[2 + j] : v[j]);               \
    const float n1 = (lo2 ? n2[0] : n2[1]) + dpp_quad_rev(lo2 ? n2[1] : n2[0]);               \
    h = n1 + dpp_quad_swap(n1) + bv;                                                          \
    reinterpret_cast<float*>(&sH[cur ^ 1][hrow(orow)])[(q >> 1) & 1] = h;                     \
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
