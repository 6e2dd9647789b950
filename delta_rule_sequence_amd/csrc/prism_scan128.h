// prism_scan128.h - the inter-segment scan after the d = 128 half-split sweep, on bfloat16
// MFMA with float32-like accuracy (gfx950).
//
// The segments of one (b, h) pair compose associatively (PRISM reading notes, section 2.1:
// each token's step is affine in the state, so a run of steps is one affine map): the state
// entering segment s + 1 is H_in(s+1) = A_s H_in(s) + B_s, with A_s the segment's operator
// and B_s its end state from a zero start, both [128][128] from the sweep.
//
// Each float x of A_s and H_in(s) enters as two bfloat16 terms, hi = bf16(x) and
// lo = bf16(x - hi), and the product is A_hi H_hi + A_hi H_lo + A_lo H_hi with float32
// accumulation: the dropped A_lo H_lo and the terms' own rounding leave a relative error of
// about 2^-16 per step, where float32 MFMA (v_mfma_f32_16x16x4f32) would take ~8 times the
// matrix-pipe cycles.  Each lane splits its operator rows as it uses them, and H_in as it
// forms it.
//
// One workgroup takes NC state columns of one pair (grid (P, 128 / NC), 8 waves); wave w
// owns state rows 16 w .. 16 w + 15.  In k block kb (0 .. 3) lane (li, g) feeds
// A_s[16 w + li][32 kb + 8 g .. + 7] (two 16-byte loads) and H_in(s)[32 kb + 8 g ..
// + 7][column li] (one 16-byte read per term from the LDS copy of H_in(s)^T).  The operator
// rows come through a ring of DEPTH steps' registers, so a step waits only on its own loads.
// One barrier per step.
//
// Outputs: H_in(s) for every segment in bfloat16 (its hi term), [column][k'] with k
// permuted inside each 32-block (the operand layout of seg_fixup_mfma_kernel), and the
// final state in float32.
#pragma once
#include "prism_kernels.h"

namespace prism {

template <int NC>
__global__ __launch_bounds__(512) void seg_scan128_mfma_kernel(FwdArgs a) {
  constexpr int D = 128, NT = NC / 16;
  constexpr int LH = D + 8;  // row stride of the H_in^T terms in LDS (bf16)
  constexpr int DEPTH = NT == 1 ? 3 : 2;  // steps of operators in flight
  static_assert(NC == 16 || NC == 32, "16 or 32 state columns per workgroup");
  // [buffer][term hi / lo][column][k]
  __shared__ __align__(16) bf16_t sHt[2][2][NC * LH];
  const int w = wave_id(), l = lane_id(), g = l >> 4, li = l & 15;
  const int pr = blockIdx.x, c0 = NC * blockIdx.y;
  const int nseg = a.nseg;
  const int row0 = 16 * w + 4 * g;  // this lane's accumulator rows row0 .. row0 + 3
  const float* Arow = a.Aagg + (size_t)pr * nseg * D * D + (size_t)(16 * w + li) * D + 8 * g;
  const float* Bpt = a.Bagg + (size_t)pr * nseg * D * D + (size_t)row0 * D + c0 + li;
  // rows row0 .. row0 + 3 land on four consecutive permuted positions (row0 % 4 == 0)
  const int ip0 = (row0 & ~31) | ((row0 & 12) << 1) | ((row0 & 16) >> 2);
  bf16_t* Hb = reinterpret_cast<bf16_t*>(a.Hin) + (size_t)pr * nseg * D * D + (size_t)(c0 + li) * D + ip0;

  f32x4 h[NT];  // H_in(s)[row0 + r][c0 + 16 nt + li], float32
  bf16x4 hhi[NT];
  // the two terms of H_in(s) into LDS buffer b; hhi keeps the hi terms
  auto put_h = [&](int b) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bf16x4 lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hhi[nt][r] = (bf16_t)h[nt][r];
        lo[r] = (bf16_t)(h[nt][r] - (float)hhi[nt][r]);
      }
      *reinterpret_cast<bf16x4*>(&sHt[b][0][(16 * nt + li) * LH + row0]) = hhi[nt];
      *reinterpret_cast<bf16x4*>(&sHt[b][1][(16 * nt + li) * LH + row0]) = lo;
    }
  };
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      h[nt][r] = a.S0 != nullptr ? a.S0[(size_t)pr * D * D + (size_t)(row0 + r) * D + c0 + 16 * nt + li] : 0.f;
  put_h(0);

  // ring slot d: the operator rows (k block kb in float4s 2 kb, 2 kb + 1) and this lane's
  // entries of B_s for the next step s with s % DEPTH == d
  float4 ring[DEPTH][8];
  float bring[DEPTH][NT][4];
  auto fetch = [&](float4 (&x)[8], float (&b)[NT][4], int s) {
    const size_t sn = (size_t)(s < nseg ? s : nseg - 1);
    const float* src = Arow + sn * D * D;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      x[2 * kb] = *reinterpret_cast<const float4*>(src + 32 * kb);
      x[2 * kb + 1] = *reinterpret_cast<const float4*>(src + 32 * kb + 4);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) b[nt][r] = Bpt[sn * D * D + (size_t)r * D + 16 * nt];
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) fetch(ring[d], bring[d], d);
  __syncthreads();
  int cur = 0;
  // one step from ring slot d; `refill` loads the slot with step s + DEPTH
  auto step = [&](const int d, const int s, const bool refill) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)  // H_in(s) for the output correction
      *reinterpret_cast<bf16x4*>(Hb + (size_t)s * D * D + (size_t)16 * nt * D) = hhi[nt];
    f32x4 acc[NT][3];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 3; ++j) acc[nt][j] = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float av[8] = {ring[d][2 * kb].x,     ring[d][2 * kb].y,     ring[d][2 * kb].z,     ring[d][2 * kb].w,
                           ring[d][2 * kb + 1].x, ring[d][2 * kb + 1].y, ring[d][2 * kb + 1].z, ring[d][2 * kb + 1].w};
      bf16x8 ah, al;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        ah[p] = (bf16_t)av[p];
        al[p] = (bf16_t)(av[p] - (float)ah[p]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int at = (16 * nt + li) * LH + 32 * kb + 8 * g;
        const bf16x8 hh = *reinterpret_cast<const bf16x8*>(&sHt[cur][0][at]);
        const bf16x8 hl = *reinterpret_cast<const bf16x8*>(&sHt[cur][1][at]);
        acc[nt][0] = mfma(ah, hh, acc[nt][0]);
        acc[nt][1] = mfma(ah, hl, acc[nt][1]);
        acc[nt][2] = mfma(al, hh, acc[nt][2]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) h[nt][r] = bring[d][nt][r] + acc[nt][0][r] + (acc[nt][1][r] + acc[nt][2][r]);
    if (refill) fetch(ring[d], bring[d], s + DEPTH);  // past the end: the last operator again
    put_h(cur ^ 1);
    cur ^= 1;
    __syncthreads();  // H_in(s+1) complete; every read of H_in(s) done
  };
  // whole blocks of DEPTH steps refill unconditionally (so each wait counts only the loads
  // issued before its own slot); the last nseg % DEPTH steps find their operands loaded
  int s0 = 0;
  for (; s0 + DEPTH <= nseg; s0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) step(d, s0 + d, true);
  }
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d)
    if (s0 + d < nseg) step(d, s0 + d, false);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) a.S_final[(size_t)pr * D * D + (size_t)(row0 + r) * D + c0 + 16 * nt + li] = h[nt][r];
}

}  // namespace prism
