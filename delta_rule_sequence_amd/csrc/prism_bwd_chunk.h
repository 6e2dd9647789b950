// prism_bwd_chunk.h - the backward in chunked (UT / WY) form on MFMA: bfloat16 inputs,
// dk = dv = 64, chunks of 64 tokens (gfx950).
//
// The forward per chunk, with H = S^T (dk x dv) its start state, b = cumsum(log g),
// G = exp(b), D_j = exp(b_C - b_j), Gam_ij = exp(b_i - b_j) (j <= i), T = (I + A)^-1 with
// A = strict(diag(beta) (Gam * K K^T)), N_l = strict(Gam * K U_l^T), P = lower(Gam * Q K^T),
// PU_l = lower(Gam * Q U_l^T), R_l = alpha_l r_l the written values of the residual chain:
//   V' = V - sum_l N_l R_l,  Uc = T diag(beta) V',  Wc = T diag(beta G) K,  E = Uc - Wc H
//   O  = diag(G) Q H + P E + sum_l PU_l R_l
//   H' = G_C H + K^T diag(D) E + sum_l U_l^T diag(D) R_l
// (the UT transform of the delta rule's chunked form with PRISM's rank-L writes: PRISM
// reading notes, sections 2.1-2.3; Tencent / PKU article, sections 01-三 and 03-三).  Every
// step is a matrix product, so its adjoint is a handful of products too.  Given d_o and the
// adjoint dH' of the chunk's end state:
//   dE  = P^T dO + diag(D) K dH'             dX1 = T^T dE,  dVp = diag(beta) dX1
//   dWc = -dE H^T,  dX2 = T^T dWc            dA  = strict(-T^T (dE Uc^T + dWc Wc^T))
//   dQ  = diag(G) dO H^T + (Gam*dP) K + sum_l (Gam*dPU_l) U_l,  dP = lower(dO E^T), dPU_l = lower(dO R_l^T)
//   dK  = diag(D) E dH'^T + (Gam*dP)^T Q + diag(beta G) dX2 + Z K + Z^T K + sum_l (Gam*dN_l) U_l
//         with Z = diag(beta) Gam * dA and dN_l = strict(-dVp R_l^T)
//   dU_l = diag(D) R_l dH'^T + (Gam*dPU_l)^T Q + (Gam*dN_l)^T K
//   dR_l = diag(D) U_l dH' + PU_l^T dO - N_l^T dVp   (then back through the residual chain)
//   dbeta = rowsum(V' * dX1) + G rowsum(K * dX2) + rowsum(dA * Gam * K K^T)
//   d log g_s = sum_{t >= s} dG_t G_t (+ dG_C G_C) + sum_{t < s} dD_t D_t
//         + sum_{i >= s > j} dlG_ij, dlG the elementwise sum of dX * X over the decayed
//         matrices: every term carries g_s, so a token with a tiny gate gets a tiny sum (the
//         same quantity as a reverse cumsum of dG G - dD D + rowsum(dlG) - colsum(dlG), which
//         cancels large terms there before the division by g)
// and the adjoint of the start state is dH = Qt^T dO + Acc^T dH' with Qt = diag(G) Q - P Wc,
// Acc = G_C I - K^T diag(D) Wc.  Two kernels:
//   * bwdc_local_kernel: per chunk, the operator Acc and its transpose, the end state from
//     zero HB = K^T D Uc + sum U_l^T D R_l and the local adjoint ell = Qt^T dO (H layout),
//     and T, Uc, Wc, V' for the gradient pass (bfloat16);
//   * bwdc_scan_kernel: the two scans over a pair's chunks, giving each chunk its start
//     state and the adjoint of its end state (stored in the S layout, S = H^T);
//   * bwdc_grad_kernel: per chunk, from those, every gradient (the state-independent part
//     of the chunk is not formed again).
// One workgroup of 8 waves per chunk.  Every 64 x 64 product is 16 output tiles of
// v_mfma_f32_16x16x32_bf16; wave w computes the tiles (w / 2, 2 (w % 2) + {0, 1}) of each,
// its operands read from LDS (16-byte row reads, or gfx950's transposing reads for a
// transposed operand), accumulating in float32.  Lane (i, g) = (lane % 16, lane / 16) holds
// out[m0 + i][n0 + 4 g + r], r = 0..3 (the product's operands are passed to the MFMA
// swapped, which yields the transposed tile): a lane's four values are consecutive columns
// of one row.  The unit lower triangular inverse is a float32 forward substitution.
#pragma once
#include "prism_bwd_args.h"
#include "prism_tile.h"

namespace prism {
namespace bwdc {

constexpr int C = 64;        // tokens per chunk
constexpr int D = 64;        // dk = dv
constexpr int LDM = 72;      // bf16 row stride of an LDS matrix (144 bytes, rows 16-byte aligned)
constexpr int MB = C * LDM;  // bf16 elements per LDS matrix
constexpr int LDF = 68;      // float32 row stride of an LDS matrix
constexpr int NT = 512;      // threads per workgroup
constexpr int kMaxL = 8;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// LDS plan (bytes): sixteen bf16 64 x 64 matrices M0 .. M15, then per-token float32
// arrays.  The float32 matrices overlay pairs of bf16 ones (a 64 x 68 float32 matrix
// takes 17 408 of their 18 432 bytes).
struct Lds {
  static constexpr int kMat = MB * 2;  // 9216 bytes
  static constexpr int oM = 0;
  static constexpr int oTok = 16 * kMat;          // per-token arrays
  // per-token float32 arrays (64 each)
  static constexpr int nTok = 5 + kMaxL + 12;     // b, G, D, beta, g, alpha[8], partials
  static constexpr int oVx = oTok + nTok * 64 * 4 + 4 * 64 * 4;  // after the dlG column partials [4][64]
  static constexpr int total = oVx + 67 * 64 * 2;  // value rows t0 - 3 .. t0 + 63, bf16, unpadded
};
static_assert(Lds::total <= 163840, "LDS plan exceeds 160 KiB");

// Per-token arrays, offsets in floats from Lds::oTok.
enum : int {
  kB = 0, kG = 64, kDd = 128, kBeta = 192, kGg = 256, kAl = 320,       // alpha: [l][64], l < 8
  kRowBeta = 320 + 512,       // dbeta partials [2 halves][64]
  kRowGv = kRowBeta + 128,    // dG partials
  kRowDd = kRowGv + 128,      // dD partials
  kRowLg = kRowDd + 128,      // (unused)
  kMisc = kRowLg + 128,       // [0..15]: dG_C partials of the 8 waves etc.
  kColLg = kMisc + 128,       // [64]: sum_{i >= s > j} dlG[i][j] for each token s
};

__device__ __forceinline__ bf16x8 rfrag(const bf16_t* X, int r0, int k0) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x8*>(X + (r0 + (l & 15)) * LDM + k0 + 8 * (l >> 4));
}

// The operand slots of column m0 + lane % 16 of a row-major matrix X, rows k0 + 8 g .. +7:
// two transposing reads.  In each 16-lane group, lane 4 a + b names row k0 + 8 g + a (+4),
// columns m0 + 4 b .. +3, and receives column m0 + lane % 16 of the 4 rows.
__device__ __forceinline__ bf16x8 tfrag(const bf16_t* X, int m0, int k0) {
  const int l = lane_id(), g = l >> 4, i = l & 15;
  const bf16_t* s = X + (k0 + 8 * g + (i >> 2)) * LDM + m0 + 4 * (i & 3);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<bf16_t*>(s)));
  const s16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<bf16_t*>(s + 4 * LDM)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
}

// operand slots k0 + 8 g + p scaled by sc[k0 + 8 g + p]
__device__ __forceinline__ bf16x8 scale8(const bf16x8& x, const float* sc, int k0) {
  const int g8 = 8 * (lane_id() >> 4);
  const float4 a = *reinterpret_cast<const float4*>(sc + k0 + g8);
  const float4 b = *reinterpret_cast<const float4*>(sc + k0 + g8 + 4);
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

// acc += A B over k = 0 .. 63 for the output tile (m0, n0).  TA: A(m, k) = XA[k][m], else
// XA[m][k]; TB: B(k, n) = XB[k][n], else XB[n][k].  bsc (optional): B's row k scaled by bsc[k].
template <bool TA, bool TB>
__device__ __forceinline__ f32x4 mm(f32x4 acc, const bf16_t* XA, const bf16_t* XB, int m0, int n0,
                                    const float* bsc = nullptr) {
#pragma unroll
  for (int k0 = 0; k0 < 64; k0 += 32) {
    const bf16x8 a = TA ? tfrag(XA, m0, k0) : rfrag(XA, m0, k0);
    bf16x8 b = TB ? tfrag(XB, n0, k0) : rfrag(XB, n0, k0);
    if (bsc != nullptr) b = scale8(b, bsc, k0);
    acc = mfma(b, a, acc);
  }
  return acc;
}

// Both of a wave's output tiles (m0, n0) and (m0, n0 + 16) of one product, the A operand
// read once per k block.
template <bool TA, bool TB>
__device__ __forceinline__ void mm2(f32x4 (&acc)[2], const bf16_t* XA, const bf16_t* XB, int m0, int n0) {
#pragma unroll
  for (int k0 = 0; k0 < 64; k0 += 32) {
    const bf16x8 a = TA ? tfrag(XA, m0, k0) : rfrag(XA, m0, k0);
    const bf16x8 b0 = TB ? tfrag(XB, n0, k0) : rfrag(XB, n0, k0);
    const bf16x8 b1 = TB ? tfrag(XB, n0 + 16, k0) : rfrag(XB, n0 + 16, k0);
    acc[0] = mfma(b0, a, acc[0]);
    acc[1] = mfma(b1, a, acc[1]);
  }
}

// Two products with the same B operand, XA1 B and XA2 B, on both of a wave's tiles: each
// operand fragment read once per k block.
template <bool TA, bool TB>
__device__ __forceinline__ void mm2b(f32x4 (&acc1)[2], f32x4 (&acc2)[2], const bf16_t* XA1, const bf16_t* XA2,
                                     const bf16_t* XB, int m0, int n0) {
#pragma unroll
  for (int k0 = 0; k0 < 64; k0 += 32) {
    const bf16x8 a1 = TA ? tfrag(XA1, m0, k0) : rfrag(XA1, m0, k0);
    const bf16x8 a2 = TA ? tfrag(XA2, m0, k0) : rfrag(XA2, m0, k0);
    const bf16x8 b0 = TB ? tfrag(XB, n0, k0) : rfrag(XB, n0, k0);
    const bf16x8 b1 = TB ? tfrag(XB, n0 + 16, k0) : rfrag(XB, n0 + 16, k0);
    acc1[0] = mfma(b0, a1, acc1[0]);
    acc1[1] = mfma(b1, a1, acc1[1]);
    acc2[0] = mfma(b0, a2, acc2[0]);
    acc2[1] = mfma(b1, a2, acc2[1]);
  }
}

__device__ __forceinline__ void put_bf16(bf16_t* X, int row, int col, const f32x4& v) {
  bf16x4 y;
#pragma unroll
  for (int r = 0; r < 4; ++r) y[r] = (bf16_t)v[r];
  *reinterpret_cast<bf16x4*>(X + row * LDM + col) = y;
}

__device__ __forceinline__ f32x4 get_bf16(const bf16_t* X, int row, int col) {
  const bf16x4 y = *reinterpret_cast<const bf16x4*>(X + row * LDM + col);
  f32x4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = (float)y[r];
  return v;
}

// Sum over the 8 consecutive lanes of a group (every lane ends with the total).
__device__ __forceinline__ float sum8(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  return x;
}

// Sum over the four lane groups g of a wave (lanes i, i + 16, i + 32, i + 48).
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Sum over the 16 lanes i of a lane group (every lane ends with the total).
__device__ __forceinline__ float sum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

// The chunk's view: pointers into LDS and the global inputs of pair pr, chunk c.
struct Chunk {
  const BwdArgs* a;
  int pr, c, t0, nt;  // nt: tokens of the chunk inside the sequence
  int L;
  char* lds;
  float* tok;
  __device__ bf16_t* m(int i) const { return reinterpret_cast<bf16_t*>(lds + i * Lds::kMat); }
  __device__ float* mf(int i) const { return reinterpret_cast<float*>(lds + i * Lds::kMat); }
};

// Matrix slots.
enum : int { mQ = 0, mK = 1, mdO = 2, mT = 3, mU = 4, mR = 5, mN = 6, mX1 = 7, mX2 = 8, mUc = 9, mWc = 10,
             mS = 11, mLam = 12, m13 = 13, m14 = 14, m15 = 15 };

// 64 rows x 64 bf16 of a token-major global array (row stride rs elements, rows >= nt zero)
// into LDS matrix X: 16 bytes per thread.
__device__ __forceinline__ void load_rows(bf16_t* X, const bf16_t* src, size_t rs, int nt) {
  const int tid = threadIdx.x, row = tid >> 3, col = 8 * (tid & 7);
  uint4 v = {0u, 0u, 0u, 0u};
  if (row < nt) v = *reinterpret_cast<const uint4*>(src + (size_t)row * rs + col);
  *reinterpret_cast<uint4*>(X + row * LDM + col) = v;
}

// Token scalars: b = cumsum(log g) (wave 0, one token per lane), G, D, beta, g, alpha.
__device__ __forceinline__ void load_scalars(const Chunk& x) {
  const BwdArgs& a = *x.a;
  const int tid = threadIdx.x;
  float* tk = x.tok;
  if (tid < 64) {
    const size_t gi = (size_t)x.pr * a.T + x.t0 + tid;
    const bool in = tid < x.nt;
    const float gv = in ? a.g[gi] : 1.f;
    float s = __logf(gv);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(s, o);
      if (tid >= o) s += y;
    }
    const float bl = __shfl(s, 63);
    tk[kB + tid] = s;
    tk[kG + tid] = __expf(s);
    tk[kDd + tid] = __expf(bl - s);
    tk[kBeta + tid] = in ? a.beta[gi] : 0.f;
    tk[kGg + tid] = gv;
  }
  if (x.L > 1) {
    for (int e = tid; e < 64 * x.L; e += NT) {
      const int t = e / x.L, l = e % x.L;
      tk[kAl + l * 64 + t] = t < x.nt ? a.alpha[((size_t)x.pr * a.T + x.t0 + t) * x.L + l] : 0.f;
    }
  }
}

// The residual chain of thread (t, 8 channels ch0 ..): r_0 = v - anchor for its channels.
struct ChainLane {
  int t, ch0;
  float r0[8];
};

__device__ __forceinline__ void load_bf16x8(float (&y)[8], const bf16_t* p) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (float)v[e];
}

__device__ __forceinline__ void chain_start(const Chunk& x, ChainLane& cl) {
  const BwdArgs& a = *x.a;
  cl.t = threadIdx.x >> 3;
  cl.ch0 = 8 * (threadIdx.x & 7);
  const bf16_t* v = static_cast<const bf16_t*>(a.v) + (size_t)x.pr * a.T * D;
  const float* w = a.conv_w + (size_t)(x.pr % a.H) * 4 * D + cl.ch0;
#pragma unroll
  for (int e = 0; e < 8; ++e) cl.r0[e] = 0.f;
  if (cl.t >= x.nt) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tg = x.t0 + cl.t - 3 + j;
    if (tg < 0) continue;
    float y[8];
    load_bf16x8(y, v + (size_t)tg * D + cl.ch0);
    const float4 w0 = *reinterpret_cast<const float4*>(w + j * D);
    const float4 w1 = *reinterpret_cast<const float4*>(w + j * D + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) cl.r0[e] += (j == 3 ? y[e] : 0.f) - wv[e] * y[e];
  }
}

// factor 1 - alpha_{t,l} gamma_{t,l} of the thread's channels (gamma slot l), and gamma itself
__device__ __forceinline__ void chain_factor(const Chunk& x, const ChainLane& cl, int l, float (&f)[8],
                                             float (&gm)[8]) {
  const BwdArgs& a = *x.a;
  if (cl.t >= x.nt) {  // past the sequence end: alpha is zero, nothing is read
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[e] = 1.f;
      gm[e] = 0.f;
    }
    return;
  }
  load_bf16x8(gm, static_cast<const bf16_t*>(a.gamma) +
                      (((size_t)x.pr * a.T + x.t0 + cl.t) * (x.L - 1) + l) * D + cl.ch0);
  const float al = x.tok[kAl + l * 64 + cl.t];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = 1.f - al * gm[e];
}
__device__ __forceinline__ void chain_factor(const Chunk& x, const ChainLane& cl, int l, float (&f)[8]) {
  float gm[8];
  chain_factor(x, cl, l, f, gm);
}

// R_l = alpha_l r_l into X (bf16 rows t)
__device__ __forceinline__ void put_written(const Chunk& x, const ChainLane& cl, bf16_t* X, int l, const float (&r)[8]) {
  const float al = x.tok[kAl + l * 64 + cl.t];
  bf16x8 y;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (bf16_t)(al * r[e]);
  *reinterpret_cast<bf16x8*>(X + cl.t * LDM + cl.ch0) = y;
}

// T = (I + A)^-1 for A strictly lower triangular (float32 A, row-major, stride LDF), in
// float32 by 16 x 16 blocks, as five steps each followed by a barrier (the caller's, so that
// other work shares the intervals):
//   step 0: diagonal blocks: wave 0, lane 16 b + c walks column c of block b down its rows
//           (right-looking substitution, x_r -= A_rj x_j);
//   steps 1..3: off-diagonal blocks at block distance d = step (block (j + d, j) on wave j):
//           T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, two float32 MFMA products
//           (v_mfma_f32_16x16x4_f32), the sum's tile fed straight back as the B operand of
//           the second;
//   step 4: the result into Tb in bf16 (zero above the diagonal blocks), every thread.
// Tf (float32, stride LDF) is scratch.
__device__ __forceinline__ void inverse_step(int step, const float* A, float* Tf, bf16_t* Tb) {
  const int w = wave_id(), l = lane_id(), i = l & 15, g = l >> 4;
  if (step == 0) {
    if (w == 0) {
      const int o = 16 * g, c = i;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = r == c ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < 15; ++j) {
#pragma unroll
        for (int r = j + 1; r < 16; ++r) x[r] -= A[(o + r) * LDF + o + j] * x[j];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Tf[(o + r) * LDF + o + c] = x[r];
    }
  } else if (step < 4) {
    const int d = step;
    if (w < 4 - d) {
      const int bj = w, bi = w + d;
      f32x4 xs = zero4();
      for (int bk = bj; bk < bi; ++bk) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          xs = mfma(A[(16 * bi + i) * LDF + 16 * bk + 4 * kb + g], Tf[(16 * bk + 4 * kb + g) * LDF + 16 * bj + i], xs);
      }
      // xs[r] = X[4 g + r][i]; the next product contracts over k = 4 g + r
      f32x4 t = zero4();
#pragma unroll
      for (int r = 0; r < 4; ++r) t = mfma(Tf[(16 * bi + i) * LDF + 16 * bi + 4 * g + r], xs[r], t);
#pragma unroll
      for (int r = 0; r < 4; ++r) Tf[(16 * bi + 4 * g + r) * LDF + 16 * bj + i] = -t[r];
    }
  } else {
    for (int e = threadIdx.x; e < 64 * 16; e += NT) {
      const int row = e >> 4, c4 = 4 * (e & 15);
      const bool keep = (c4 >> 4) <= (row >> 4);
      const float4 v = *reinterpret_cast<const float4*>(Tf + row * LDF + c4);
      bf16x4 y;
      y[0] = keep ? (bf16_t)v.x : (bf16_t)0.f;
      y[1] = keep ? (bf16_t)v.y : (bf16_t)0.f;
      y[2] = keep ? (bf16_t)v.z : (bf16_t)0.f;
      y[3] = keep ? (bf16_t)v.w : (bf16_t)0.f;
      *reinterpret_cast<bf16x4*>(Tb + row * LDM + c4) = y;
    }
  }
}

// A row-lane tile (lane: out[row][col .. col + 3]) stored transposed into a float32 matrix.
__device__ __forceinline__ void store_tile_t(float* dst, int row, int col, const f32x4& v) {
#pragma unroll
  for (int r = 0; r < 4; ++r) dst[(size_t)(col + r) * D + row] = v[r];
}

// lower(Gam) at the lane's four entries (row, col .. col + 3) of a 64 x 64 tile.
__device__ __forceinline__ f32x4 gam_tile(const float* tk, int row, int col) {
  const float b_i = tk[kB + row];
  const float4 bj = *reinterpret_cast<const float4*>(tk + kB + col);
  f32x4 gm;
  gm[0] = col + 0 <= row ? __expf(b_i - bj.x) : 0.f;
  gm[1] = col + 1 <= row ? __expf(b_i - bj.y) : 0.f;
  gm[2] = col + 2 <= row ? __expf(b_i - bj.z) : 0.f;
  gm[3] = col + 3 <= row ? __expf(b_i - bj.w) : 0.f;
  return gm;
}

// The state-independent part of a chunk, shared by both kernels.  On return (after a
// barrier): sT, sUc, sWc filled; vp = V' tiles and uc = Uc tiles of the wave (float32).
// With HB, hb accumulates sum_l U_l^T diag(D) R_l (H layout).
struct Fwd {
  f32x4 vp[2], uc[2];
};

template <bool HB>
__device__ __forceinline__ void chunk_forward(const Chunk& x, ChainLane& cl, Fwd& f, f32x4 (&hb)[2]) {
  const BwdArgs& a = *x.a;
  const int w = wave_id(), l = lane_id(), i = l & 15, g = l >> 4;
  const int mt = w >> 1, nt0 = 2 * (w & 1), row = 16 * mt + i;
  const float* tk = x.tok;
  bf16_t *sK = x.m(mK), *sT = x.m(mT), *sU = x.m(mU), *sR = x.m(mR), *sN = x.m(mN);
  bf16_t *sX1 = x.m(mX1), *sX2 = x.m(mX2), *sUc = x.m(mUc), *sWc = x.m(mWc);
  float* sAf = x.mf(m13);
  const float beta_i = tk[kBeta + row], G_i = tk[kG + row];
  // F1: A = strict(diag(beta) Gam * K K^T) (float32); with HB also P = lower(Gam * Q K^T)
  // into slot 15 for the local pass's Qt
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n0 = 16 * (nt0 + h), col = n0 + 4 * g;
    const f32x4 kk = mm<false, false>(zero4(), sK, sK, 16 * mt, n0);
    const f32x4 gm = gam_tile(tk, row, col);
    f32x4 av;
#pragma unroll
    for (int r = 0; r < 4; ++r) av[r] = col + r < row ? beta_i * gm[r] * kk[r] : 0.f;
    *reinterpret_cast<f32x4*>(sAf + row * LDF + col) = av;
    if constexpr (HB) {
      f32x4 p = mm<false, false>(zero4(), x.m(mQ), sK, 16 * mt, n0);
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] *= gm[r];
      put_bf16(x.m(m15), row, col, p);
    }
  }
  __syncthreads();
  // V' = V - sum_l N_l R_l: V's tiles straight from memory
  const bf16_t* vg = static_cast<const bf16_t*>(a.v) + ((size_t)x.pr * a.T + x.t0) * D;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = 16 * (nt0 + h) + 4 * g;
    f.vp[h] = zero4();
    if (row < x.nt) {
      const bf16x4 y = *reinterpret_cast<const bf16x4*>(vg + (size_t)row * D + col);
#pragma unroll
      for (int r = 0; r < 4; ++r) f.vp[h][r] = (float)y[r];
    }
  }
  // The inverse (five steps, T not needed before F4) and the rank slots (F3, ascending) share
  // barrier intervals.  Slot l's phases: A_l writes U_l and R_l (alternating between two LDS
  // slot pairs, the u rows and gamma loaded one slot ahead; r_{l-1} goes to the chunk's
  // matrices for the gradient pass), B_l forms N_l = strict(Gam * K U_l^T) (and hb), C_l
  // subtracts N_l R_l from V'.  Interval k holds inverse step k (k < 5) and, for k = 2 m, C_m
  // and A_{m+1}, for k = 2 m + 1, B_{m+1}.
  bf16_t* sUb[2] = {sU, x.m(mS)};
  bf16_t* sRb[2] = {sR, x.m(mLam)};
  float* sTf = x.mf(mUc);
  const int tid = threadIdx.x, trow = tid >> 3, tc8 = 8 * (tid & 7);
  const bool tin = trow < x.nt;
  const bf16_t* ug = static_cast<const bf16_t*>(a.u) + ((size_t)x.pr * a.T + x.t0) * (x.L - 1) * D;
  const bf16_t* gg = static_cast<const bf16_t*>(a.gamma) + ((size_t)x.pr * a.T + x.t0) * (x.L - 1) * D;
  bf16_t* rout = static_cast<bf16_t*>(a.chunk_mats) + ((size_t)x.pr * a.nseg + x.c) * (4 + x.L - 1) * 4096 +
                 4 * 4096;
  uint4 pu = {0u, 0u, 0u, 0u}, pg = {0u, 0u, 0u, 0u};
  if (x.L > 1 && tin) {
    pu = *reinterpret_cast<const uint4*>(ug + (size_t)trow * (x.L - 1) * D + tc8);
    pg = *reinterpret_cast<const uint4*>(gg + (size_t)trow * (x.L - 1) * D + tc8);
  }
  float rc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) rc[e] = cl.r0[e];
  constexpr int kSteps = 5;
  const int nk = (2 * (x.L - 1) + 1 > kSteps) ? 2 * (x.L - 1) + 1 : kSteps;
#pragma unroll
  for (int k = 0; k < nk; ++k) {
    if (k < kSteps) inverse_step(k, sAf, sTf, sT);
    const int m = k >> 1;
    if ((k & 1) == 0) {
      if (m >= 1 && m <= x.L - 1) {
        // C_m: V' -= N_m R_m
        const int b = (m - 1) & 1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4 t = mm<false, true>(zero4(), sN, sRb[b], 16 * mt, 16 * (nt0 + h));
#pragma unroll
          for (int r = 0; r < 4; ++r) f.vp[h][r] -= t[r];
        }
      }
      if (m + 1 <= x.L - 1) {
        // A_{m+1}: U and R of slot lv = m + 1
        const int lv = m + 1, b = (lv - 1) & 1;
        *reinterpret_cast<uint4*>(sUb[b] + trow * LDM + tc8) = pu;
        bf16x8 rb;
#pragma unroll
        for (int e = 0; e < 8; ++e) rb[e] = (bf16_t)rc[e];
        *reinterpret_cast<bf16x8*>(rout + (size_t)(lv - 1) * 4096 + trow * 64 + tc8) = rb;
        const bf16x8 gv = __builtin_bit_cast(bf16x8, pg);
        const float al = tk[kAl + (lv - 1) * 64 + trow];
#pragma unroll
        for (int e = 0; e < 8; ++e) rc[e] *= 1.f - al * (float)gv[e];
        put_written(x, cl, sRb[b], lv, rc);
      }
    } else if (m + 1 <= x.L - 1) {
      // B_{m+1}: N_{m+1} (and hb); the next slot's u rows and gamma from memory
      const int lv = m + 1, b = (lv - 1) & 1;
      if (lv + 1 < x.L && tin) {
        pu = *reinterpret_cast<const uint4*>(ug + (size_t)trow * (x.L - 1) * D + (size_t)lv * D + tc8);
        pg = *reinterpret_cast<const uint4*>(gg + (size_t)trow * (x.L - 1) * D + (size_t)lv * D + tc8);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n0 = 16 * (nt0 + h), col = n0 + 4 * g;
        f32x4 nr = mm<false, false>(zero4(), sK, sUb[b], 16 * mt, n0);
        const f32x4 gm = gam_tile(tk, row, col);
#pragma unroll
        for (int r = 0; r < 4; ++r) nr[r] = col + r < row ? gm[r] * nr[r] : 0.f;
        put_bf16(sN, row, col, nr);
        if constexpr (HB) hb[h] = mm<true, true>(hb[h], sUb[b], sRb[b], 16 * mt, n0, tk + kDd);
      }
    }
    if (k + 1 < nk) __syncthreads();
  }
  // F4: X1 = diag(beta) V', X2 = diag(beta G) K; Uc = T X1, Wc = T X2
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = 16 * (nt0 + h) + 4 * g;
    f32x4 x1, x2 = get_bf16(sK, row, col);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x1[r] = beta_i * f.vp[h][r];
      x2[r] *= beta_i * G_i;
    }
    put_bf16(sX1, row, col, x1);
    put_bf16(sX2, row, col, x2);
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n0 = 16 * (nt0 + h), col = n0 + 4 * g;
    f.uc[h] = mm<false, true>(zero4(), sT, sX1, 16 * mt, n0);
    const f32x4 wc = mm<false, true>(zero4(), sT, sX2, 16 * mt, n0);
    put_bf16(sUc, row, col, f.uc[h]);
    put_bf16(sWc, row, col, wc);
  }
  __syncthreads();
}

__device__ __forceinline__ void load_chunk_inputs(const Chunk& x) {
  const BwdArgs& a = *x.a;
  const size_t r0 = ((size_t)x.pr * a.T + x.t0) * D;
  load_rows(x.m(mQ), static_cast<const bf16_t*>(a.q) + r0, D, x.nt);
  load_rows(x.m(mK), static_cast<const bf16_t*>(a.k) + r0, D, x.nt);
  load_rows(x.m(mdO), static_cast<const bf16_t*>(a.d_o) + r0, D, x.nt);
  load_scalars(x);
}

// Segment-form operands of each chunk (segments of one chunk: a.nseg == chunks per pair).
// NL = L - 1 rank slots, fixed at compile time so that the rank loops unroll.
template <int NL>
__global__ __launch_bounds__(NT) void bwdc_local_kernel(BwdArgs a) {
  __shared__ __align__(16) char lds[Lds::total];
  Chunk x;
  x.a = &a;
  x.c = blockIdx.x;
  x.pr = blockIdx.y;
  x.t0 = x.c * C;
  x.nt = min(C, a.T - x.t0);
  x.L = NL + 1;
  x.lds = lds;
  x.tok = reinterpret_cast<float*>(lds + Lds::oTok);
  const int w = wave_id(), l = lane_id(), i = l & 15, g = l >> 4;
  const int mt = w >> 1, nt0 = 2 * (w & 1), row = 16 * mt + i;
  load_chunk_inputs(x);
  ChainLane cl;
  if (x.L > 1) chain_start(x, cl);
  __syncthreads();
  Fwd f;
  f32x4 hb[2] = {zero4(), zero4()};
  chunk_forward<true>(x, cl, f, hb);
  const float* tk = x.tok;
  bf16_t *sQ = x.m(mQ), *sK = x.m(mK), *sdO = x.m(mdO), *sUc = x.m(mUc), *sWc = x.m(mWc);
  bf16_t *sP = x.m(m15), *sQt = x.m(mX2);
  {
    // T, Uc, Wc and V' for the gradient pass (bf16, row-major 64 x 64 each)
    bf16_t* cm = static_cast<bf16_t*>(a.chunk_mats) + ((size_t)x.pr * a.nseg + x.c) * (4 + x.L - 1) * 4096;
    const int tid = threadIdx.x, r = tid >> 3, c8 = 8 * (tid & 7);
    *reinterpret_cast<uint4*>(cm + r * 64 + c8) = *reinterpret_cast<const uint4*>(x.m(mT) + r * LDM + c8);
    *reinterpret_cast<uint4*>(cm + 4096 + r * 64 + c8) = *reinterpret_cast<const uint4*>(sUc + r * LDM + c8);
    *reinterpret_cast<uint4*>(cm + 8192 + r * 64 + c8) = *reinterpret_cast<const uint4*>(sWc + r * LDM + c8);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x4 y;
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = (bf16_t)f.vp[h][q];
      *reinterpret_cast<bf16x4*>(cm + 12288 + row * 64 + 16 * (nt0 + h) + 4 * g) = y;
    }
  }
  // Qt = diag(G) Q - P Wc (P formed in F1); Acc = G_C I - K^T D Wc (bf16: it is only ever
  // an MFMA operand); HB = hb + K^T D Uc
  const float GC = tk[kG + 63];
  const size_t so = ((size_t)x.pr * a.nseg + x.c) * D * D;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n0 = 16 * (nt0 + h), col = n0 + 4 * g;
    f32x4 qt = get_bf16(sQ, row, col);
    const f32x4 pw = mm<false, true>(zero4(), sP, sWc, 16 * mt, n0);
    const float G_i = tk[kG + row];
#pragma unroll
    for (int r = 0; r < 4; ++r) qt[r] = G_i * qt[r] - pw[r];
    put_bf16(sQt, row, col, qt);
    f32x4 ac = mm<true, true>(zero4(), sK, sWc, 16 * mt, n0, tk + kDd);
#pragma unroll
    for (int r = 0; r < 4; ++r) ac[r] = (col + r == row ? GC : 0.f) - ac[r];
    {
      bf16x4 y;
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = (bf16_t)ac[r];
      *reinterpret_cast<bf16x4*>(static_cast<bf16_t*>(a.c_Acc) + so + (size_t)row * D + col) = y;
    }
    const f32x4 bb = mm<true, true>(hb[h], sK, sUc, 16 * mt, n0, tk + kDd);
    *reinterpret_cast<f32x4*>(a.seg_B + so + (size_t)row * D + col) = bb;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n0 = 16 * (nt0 + h), col = n0 + 4 * g;
    const f32x4 el = mm<true, true>(zero4(), sQt, sdO, 16 * mt, n0);
    *reinterpret_cast<f32x4*>(a.seg_ell + so + (size_t)row * D + col) = el;
  }
}

// The two scans over a pair's groups of chunks, on columns c0 .. c0 + 3 of the carried
// 64 x 64 matrix (H layout): forwards (blockIdx.z = 0) X_0 = 0, X_{g+1} = Acc_g X_g + HB_g,
// storing S_in(g) = X_g^T; backwards (blockIdx.z = 1) X_{ngrp-1} = dS_final (zero if
// absent), X_{g-1} = Acc_g^T X_g + ell_g, storing Lambda_g = X_g^T.  Thread t takes rows
// i0 = 2 (t / 8), i0 + 1 and the contraction slice k = 8 q .. 8 q + 7 (q = t % 8): it keeps
// those 16 entries of the step's operator in registers (loaded DEPTH steps ahead, so a step
// never waits on memory), reads rows 8 q .. 8 q + 7 of the four carried columns from LDS
// (one 16-byte read each, rows skewed so the eight slices hit distinct banks) and forms
// 2 x 4 partial sums; three DPP exchange rounds within the 8 lanes of the row pair (the
// rows, then halves of the columns, then single columns) leave lane q with
// X_new[i0 + q / 4][c0 + q % 4].  Four columns per workgroup (16 per pair and direction,
// 256 workgroups at 8 pairs) keep each step's chain to 64 multiply-adds per thread.  One
// barrier per step.
__device__ __forceinline__ float dpp_mirror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_rev4(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x1B, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_swap2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}

constexpr int kScanCols = 4;
__device__ __forceinline__ int scan_row(int r) { return 4 * r + 4 * (r >> 3); }  // float offset of carried row r

__global__ __launch_bounds__(256) void bwdc_scan_kernel(BwdArgs a) {
  constexpr int DEPTH = 4;
  __shared__ __align__(16) float sH[2][64 * 4 + 8 * 4];
  const int tid = threadIdx.x, i0 = 2 * (tid >> 3), q = tid & 7;
  const int pr = blockIdx.x, c0 = kScanCols * blockIdx.y;
  const bool rev = blockIdx.z == 1;
  const int n = a.ngrp;
  const int orow = i0 + (q >> 2), ocol = c0 + (q & 3);  // the entry this lane ends with
  const size_t base = (size_t)pr * n * D * D;
  const float* A0 = (rev ? a.grp_Phi : a.grp_Acc) + base + (size_t)i0 * D + 8 * q;
  const float* B0 = (rev ? a.grp_ell : a.grp_B) + base + (size_t)orow * D + ocol;
  float* O0 = (rev ? a.grp_Lam : a.grp_Sin) + base + (size_t)ocol * D + orow;
  auto chunk_of = [&](int s) { return rev ? n - 1 - s : s; };
#define PRISM_DECL(D_) float4 R##D_##_0, R##D_##_1, R##D_##_2, R##D_##_3; float R##D_##_b;
#define PRISM_FETCH(D_, S)                                                                    \
  {                                                                                           \
    const size_t cn_ = (size_t)chunk_of((S) < n ? (S) : n - 1);                               \
    const float4* src_ = reinterpret_cast<const float4*>(A0 + cn_ * D * D);                  \
    R##D_##_0 = src_[0];                                                                      \
    R##D_##_1 = src_[1];                                                                      \
    R##D_##_2 = src_[D / 4];                                                                  \
    R##D_##_3 = src_[D / 4 + 1];                                                              \
    R##D_##_b = B0[cn_ * D * D];                                                              \
  }
  PRISM_DECL(0) PRISM_DECL(1) PRISM_DECL(2) PRISM_DECL(3)
  PRISM_FETCH(0, 0) PRISM_FETCH(1, 1) PRISM_FETCH(2, 2) PRISM_FETCH(3, 3)
  const float* X0 = rev ? a.dS_final : nullptr;
  const float* xs = X0 != nullptr ? X0 + (size_t)pr * D * D : nullptr;
  float h = xs != nullptr ? xs[(size_t)orow * D + ocol] : 0.f;
  if (tid < 64)
    *reinterpret_cast<float4*>(&sH[0][scan_row(tid)]) =
        xs != nullptr ? *reinterpret_cast<const float4*>(xs + (size_t)tid * D + c0) : make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();
  const bool lo4 = q < 4, lo2 = (q & 2) == 0, lo1 = (q & 1) == 0;
  int cur = 0;
#define PRISM_SCAN_STEP(D_, PREFETCH)                                                         \
  {                                                                                           \
    const int s = s0 + (D_);                                                                  \
    O0[(size_t)chunk_of(s) * D * D] = h;                                                      \
    const float ar0[8] = {R##D_##_0.x, R##D_##_0.y, R##D_##_0.z, R##D_##_0.w,                 \
                          R##D_##_1.x, R##D_##_1.y, R##D_##_1.z, R##D_##_1.w};                \
    const float ar1[8] = {R##D_##_2.x, R##D_##_2.y, R##D_##_2.z, R##D_##_2.w,                 \
                          R##D_##_3.x, R##D_##_3.y, R##D_##_3.z, R##D_##_3.w};                \
    const float bv = R##D_##_b;                                                               \
    float v0[4], v1[4]; /* rows i0, i0 + 1; columns c0 .. c0 + 3 */                          \
    _Pragma("unroll") for (int c = 0; c < 4; ++c) { v0[c] = 0.f; v1[c] = 0.f; }              \
    _Pragma("unroll") for (int m = 0; m < 8; ++m) {                                           \
      const float4 xa = *reinterpret_cast<const float4*>(&sH[cur][scan_row(8 * q + m)]);      \
      const float xv[4] = {xa.x, xa.y, xa.z, xa.w};                                           \
      _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                         \
        v0[c] += ar0[m] * xv[c];                                                              \
        v1[c] += ar1[m] * xv[c];                                                              \
      }                                                                                       \
    }                                                                                         \
    if (PREFETCH) PRISM_FETCH(D_, s + DEPTH)                                                  \
    /* the rows, then halves of the columns, then single columns */                          \
    float k[4];                                                                               \
    _Pragma("unroll") for (int c = 0; c < 4; ++c)                                             \
      k[c] = (lo4 ? v0[c] : v1[c]) + dpp_mirror8(lo4 ? v1[c] : v0[c]);                        \
    float j[2];                                                                               \
    _Pragma("unroll") for (int c = 0; c < 2; ++c)                                             \
      j[c] = (lo2 ? k[c] : k[2 + c]) + dpp_rev4(lo2 ? k[2 + c] : k[c]);                        \
    h = (lo1 ? j[0] : j[1]) + dpp_swap2(lo1 ? j[1] : j[0]) + bv;                              \
    sH[cur ^ 1][scan_row(orow) + (q & 3)] = h;                                                \
    cur ^= 1;                                                                                 \
    __syncthreads();                                                                          \
  }
  int s0 = 0;
  for (; s0 + DEPTH <= n; s0 += DEPTH) {
    PRISM_SCAN_STEP(0, true) PRISM_SCAN_STEP(1, true) PRISM_SCAN_STEP(2, true) PRISM_SCAN_STEP(3, true)
  }
  if (s0 + 0 < n) PRISM_SCAN_STEP(0, false)
  if (s0 + 1 < n) PRISM_SCAN_STEP(1, false)
  if (s0 + 2 < n) PRISM_SCAN_STEP(2, false)
#undef PRISM_SCAN_STEP
#undef PRISM_FETCH
#undef PRISM_DECL
}

// A bf16 64 x 64 matrix (row-major, unpadded) in two steps: this thread's 8 entries from
// memory, then into an LDS matrix.
__device__ __forceinline__ uint4 fetch8b(const bf16_t* src) {
  const int tid = threadIdx.x;
  return *reinterpret_cast<const uint4*>(src + (tid >> 3) * D + 8 * (tid & 7));
}
__device__ __forceinline__ void put8b(bf16_t* X, const uint4& v) {
  const int tid = threadIdx.x;
  *reinterpret_cast<uint4*>(X + (tid >> 3) * LDM + 8 * (tid & 7)) = v;
}

// A float32 64 x 64 matrix (row-major) in two steps: this thread's 8 entries from memory,
// then into LDS as bf16.
struct F32Row8 {
  float4 u, v;
};
__device__ __forceinline__ F32Row8 fetch8(const float* src) {
  const int tid = threadIdx.x, row = tid >> 3, col = 8 * (tid & 7);
  return {*reinterpret_cast<const float4*>(src + row * D + col), *reinterpret_cast<const float4*>(src + row * D + col + 4)};
}
__device__ __forceinline__ void put8(bf16_t* X, const F32Row8& f) {
  const int tid = threadIdx.x, row = tid >> 3, col = 8 * (tid & 7);
  bf16x8 y;
  y[0] = (bf16_t)f.u.x; y[1] = (bf16_t)f.u.y; y[2] = (bf16_t)f.u.z; y[3] = (bf16_t)f.u.w;
  y[4] = (bf16_t)f.v.x; y[5] = (bf16_t)f.v.y; y[6] = (bf16_t)f.v.z; y[7] = (bf16_t)f.v.w;
  *reinterpret_cast<bf16x8*>(X + row * LDM + col) = y;
}

// Group operators of the two-level scan, one workgroup per group of up to kBwdGroup chunks
// (c0 .. c0 + G - 1): with Pre_i = Acc_{c0+i-1} .. Acc_{c0} (Pre_0 = I),
//   Acc_g = Pre_G,  HB_g = sum_i Acc_{c0+G-1} .. Acc_{c0+i+1} HB_{c0+i},  ell_g = sum_i Pre_i^T ell_{c0+i}
// (the state after the group from a zero start, and the adjoint at its start from its own
// outputs), formed one chunk at a time: ell_g += M^T ell_i, M <- Acc_i M, HB_g <- Acc_i HB_g +
// HB_i.  Products on bf16 MFMA operands (the running matrices kept in float32); the next
// chunk's operands are loaded while the current chunk's products run.
__global__ __launch_bounds__(NT) void bwdc_compose_kernel(BwdArgs a) {
  __shared__ __align__(16) bf16_t sm[4][MB];
  bf16_t *sA = sm[0], *sE = sm[1], *sM = sm[2], *sHg = sm[3];
  const int w = wave_id(), l = lane_id(), i = l & 15, g = l >> 4;
  const int mt = w >> 1, nt0 = 2 * (w & 1), row = 16 * mt + i;
  const int grp = blockIdx.x, pr = blockIdx.y;
  const int c0 = grp * kBwdGroup, G = min(kBwdGroup, a.nseg - c0);
  f32x4 M[2], Hg[2], Eg[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = 16 * (nt0 + h) + 4 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) M[h][r] = col + r == row ? 1.f : 0.f;
    Hg[h] = zero4();
    Eg[h] = zero4();
  }
  auto so_of = [&](int it) { return ((size_t)pr * a.nseg + c0 + it) * D * D; };
  const bf16_t* cacc = static_cast<const bf16_t*>(a.c_Acc);
  uint4 fa = fetch8b(cacc + so_of(0));
  F32Row8 fe = fetch8(a.seg_ell + so_of(0));
  f32x4 hb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    hb[h] = *reinterpret_cast<const f32x4*>(a.seg_B + so_of(0) + (size_t)row * D + 16 * (nt0 + h) + 4 * g);
  for (int it = 0; it < G; ++it) {
    put8b(sA, fa);
    put8(sE, fe);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = 16 * (nt0 + h) + 4 * g;
      put_bf16(sM, row, col, M[h]);
      put_bf16(sHg, row, col, Hg[h]);
    }
    __syncthreads();
    const f32x4 hc[2] = {hb[0], hb[1]};
    if (it + 1 < G) {
      fa = fetch8b(cacc + so_of(it + 1));
      fe = fetch8(a.seg_ell + so_of(it + 1));
#pragma unroll
      for (int h = 0; h < 2; ++h)
        hb[h] = *reinterpret_cast<const f32x4*>(a.seg_B + so_of(it + 1) + (size_t)row * D + 16 * (nt0 + h) + 4 * g);
    }
    mm2<true, true>(Eg, sM, sE, 16 * mt, 16 * nt0);
    M[0] = zero4();
    M[1] = zero4();
    mm2<false, true>(M, sA, sM, 16 * mt, 16 * nt0);
    Hg[0] = hc[0];
    Hg[1] = hc[1];
    mm2<false, true>(Hg, sA, sHg, 16 * mt, 16 * nt0);
    __syncthreads();
  }
  const size_t go = ((size_t)pr * a.ngrp + grp) * D * D;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = 16 * (nt0 + h) + 4 * g;
    *reinterpret_cast<f32x4*>(a.grp_Acc + go + (size_t)row * D + col) = M[h];
    store_tile_t(a.grp_Phi + go, row, col, M[h]);
    *reinterpret_cast<f32x4*>(a.grp_B + go + (size_t)row * D + col) = Hg[h];
    *reinterpret_cast<f32x4*>(a.grp_ell + go + (size_t)row * D + col) = Eg[h];
  }
}

// Each chunk's entering state and arriving adjoint from its group's (S layout, stored in
// bf16, the gradient pass's operand type): forwards (blockIdx.z = 0) X_{c0} = X_g,
// X_{c+1} = Acc_c X_c + HB_c; backwards (blockIdx.z = 1) Y_{c0+G-1} = Y_g, Y_{c-1} =
// Acc_c^T Y_c + ell_c.  The carried matrix is the B operand of the next product in its S
// layout (B(k, n) = X[k][n] = S[n][k]); bf16 operands, float32 sums; the next step's
// operator is loaded while the current step's product runs.
__global__ __launch_bounds__(NT) void bwdc_expand_kernel(BwdArgs a) {
  __shared__ __align__(16) bf16_t sm[2][MB];
  bf16_t *sA = sm[0], *sS = sm[1];
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), i = l & 15, g = l >> 4;
  const int mt = w >> 1, nt0 = 2 * (w & 1), row = 16 * mt + i;
  const int grp = blockIdx.x, pr = blockIdx.y;
  const bool rev = blockIdx.z == 1;
  const int c0 = grp * kBwdGroup, G = min(kBwdGroup, a.nseg - c0);
  const size_t go = ((size_t)pr * a.ngrp + grp) * D * D;
  const float* xg = (rev ? a.grp_Lam : a.grp_Sin) + go;
  bf16_t* outb = static_cast<bf16_t*>(rev ? a.c_Lam : a.c_Sin);
  const bf16_t* cacc = static_cast<const bf16_t*>(a.c_Acc);
  const float* addb = rev ? a.seg_ell : a.seg_B;
  auto src_of = [&](int it) { return rev ? c0 + G - it : c0 + it - 1; };  // the chunk whose operator applies
  auto so_of = [&](int c) { return ((size_t)pr * a.nseg + c) * D * D; };
  const int r8 = tid >> 3, c8 = 8 * (tid & 7);
  uint4 fa = {0u, 0u, 0u, 0u};
  f32x4 ad[2] = {zero4(), zero4()};
  if (G > 1) {
    fa = fetch8b(cacc + so_of(src_of(1)));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      ad[h] = *reinterpret_cast<const f32x4*>(addb + so_of(src_of(1)) + (size_t)row * D + 16 * (nt0 + h) + 4 * g);
  }
  // the group's own entry: into bf16, staged for the first product and stored for its chunk
  {
    const int c = rev ? c0 + G - 1 : c0;
    put8(sS, fetch8(xg));
    __syncthreads();
    *reinterpret_cast<uint4*>(outb + so_of(c) + r8 * D + c8) = *reinterpret_cast<const uint4*>(sS + r8 * LDM + c8);
  }
  for (int it = 1; it < G; ++it) {
    const int cd = rev ? src_of(it) - 1 : src_of(it) + 1;  // the chunk that receives the result
    put8b(sA, fa);
    __syncthreads();
    f32x4 x[2] = {ad[0], ad[1]};
    if (it + 1 < G) {
      fa = fetch8b(cacc + so_of(src_of(it + 1)));
#pragma unroll
      for (int h = 0; h < 2; ++h)
        ad[h] = *reinterpret_cast<const f32x4*>(addb + so_of(src_of(it + 1)) + (size_t)row * D + 16 * (nt0 + h) + 4 * g);
    }
    if (rev) mm2<true, false>(x, sA, sS, 16 * mt, 16 * nt0);
    else mm2<false, false>(x, sA, sS, 16 * mt, 16 * nt0);
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = 16 * (nt0 + h) + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) sS[(col + r) * LDM + row] = (bf16_t)x[h][r];
    }
    __syncthreads();
    *reinterpret_cast<uint4*>(outb + so_of(cd) + r8 * D + c8) = *reinterpret_cast<const uint4*>(sS + r8 * LDM + c8);
  }
}

// dconv_w[h] = sum over the batch and the chunks of the per-chunk shares [B][H][nch][4][64]:
// workgroup (h, block of 64 entries) of 1024 threads; thread (q, e) sums the shares
// x = q, q + 16, .. of entry e (eight loads in flight, eight accumulators), then the 16
// partial sums are added in a fixed order (deterministic).
__global__ __launch_bounds__(1024) void bwdc_conv_reduce_kernel(const float* part, float* dconv_w, int B, int H,
                                                                int nch) {
  __shared__ float ps[16][64];
  const int h = blockIdx.x, q = threadIdx.x >> 6, e = threadIdx.x & 63, idx = 64 * blockIdx.y + e;
  const int n = B * nch;
  // eight shares in flight per round (independent loads), eight accumulators
  float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int x0 = q; x0 < n; x0 += 16 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int x = x0 + 16 * u;
      v[u] = x < n ? part[(((size_t)(x / nch) * H + h) * nch + x % nch) * 4 * D + idx] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) s8[u] += v[u];
  }
  ps[q][e] = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
  __syncthreads();
  if (q == 0) {
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) t += ps[r][e];
    dconv_w[(size_t)h * 4 * D + idx] = t;
  }
}

// Every gradient of chunk (blockIdx.x, pair blockIdx.y) from its start state (c_Sin) and
// the adjoint of its end state (c_Lam).  NL = L - 1 rank slots, fixed at compile time.
template <int NL>
__global__ __launch_bounds__(NT) void bwdc_grad_kernel(BwdArgs a) {
  __shared__ __align__(16) char lds[Lds::total];
  Chunk x;
  x.a = &a;
  x.c = blockIdx.x;
  x.pr = blockIdx.y;
  x.t0 = x.c * C;
  x.nt = min(C, a.T - x.t0);
  x.L = NL + 1;
  x.lds = lds;
  x.tok = reinterpret_cast<float*>(lds + Lds::oTok);
  float* tk = x.tok;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), i = l & 15, g = l >> 4;
  const int mt = w >> 1, nt0 = 2 * (w & 1), row = 16 * mt + i, half = w & 1;
  const size_t so = ((size_t)x.pr * a.nseg + x.c) * D * D;
  load_chunk_inputs(x);
  {
    // the entering state and the arriving adjoint (bf16, S layout); <dH', H> (the end
    // state's factor G_C): this thread's 8 entries, then the wave's sum
    const uint4 su = fetch8b(static_cast<const bf16_t*>(a.c_Sin) + so);
    const uint4 lu = fetch8b(static_cast<const bf16_t*>(a.c_Lam) + so);
    put8b(x.m(mS), su);
    put8b(x.m(mLam), lu);
    const bf16x8 sv = __builtin_bit_cast(bf16x8, su), lv8 = __builtin_bit_cast(bf16x8, lu);
    float gc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) gc += (float)sv[e] * (float)lv8[e];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) gc += __shfl_xor(gc, o);
    if (l == 0) tk[kMisc + w] = gc;
  }
  // T, Uc, Wc (LDS) and V' (this lane's tiles) as the chunk's local pass formed them
  const bf16_t* cm = static_cast<const bf16_t*>(a.chunk_mats) + ((size_t)x.pr * a.nseg + x.c) * (4 + x.L - 1) * 4096;
  load_rows(x.m(mT), cm, 64, 64);
  load_rows(x.m(mUc), cm + 4096, 64, 64);
  load_rows(x.m(mWc), cm + 8192, 64, 64);
  f32x4 vp[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16x4 y = *reinterpret_cast<const bf16x4*>(cm + 12288 + row * 64 + 16 * (nt0 + h) + 4 * g);
#pragma unroll
    for (int q = 0; q < 4; ++q) vp[h][q] = (float)y[q];
  }
  bf16_t* sVx = reinterpret_cast<bf16_t*>(lds + Lds::oVx);  // value rows t0 - 3 .. t0 + 63
  if (x.L > 1) {
    const bf16_t* vg = static_cast<const bf16_t*>(a.v) + (size_t)x.pr * a.T * D;
    for (int e = tid; e < 67 * 8; e += NT) {
      const int r = e >> 3, c8 = 8 * (e & 7), tv = x.t0 - 3 + r;
      uint4 y = {0u, 0u, 0u, 0u};
      if (tv >= 0 && tv < a.T) y = *reinterpret_cast<const uint4*>(vg + (size_t)tv * D + c8);
      *reinterpret_cast<uint4*>(sVx + r * 64 + c8) = y;
    }
  }
  __syncthreads();
  bf16_t *sQ = x.m(mQ), *sK = x.m(mK), *sdO = x.m(mdO), *sT = x.m(mT), *sU = x.m(mU), *sR = x.m(mR);
  bf16_t *sS = x.m(mS), *sLam = x.m(mLam), *sUc = x.m(mUc), *sWc = x.m(mWc);
  bf16_t *sE = x.m(mX1), *sP = x.m(mX2), *sZ = x.m(mN), *sdE = x.m(m13), *sdVp = x.m(m14), *sdWc = x.m(m15);
  const float beta_i = tk[kBeta + row], G_i = tk[kG + row], D_i = tk[kDd + row];
  const bool in_i = row < x.nt;
  const size_t grow = (size_t)x.pr * a.T + x.t0 + row;  // global token row of this lane
  f32x4 dq[2], dk[2], dlg[2], p[2];
  float rb_beta = 0.f, rb_gv = 0.f, rb_dd = 0.f;  // this lane's row partials (4 columns x 2 tiles)
  const int n0w = 16 * nt0;  // the wave's first output column
  // B0: E = Uc - Wc H; P = lower(Gam * Q K^T)
  {
    f32x4 e[2] = {zero4(), zero4()};
    p[0] = zero4();
    p[1] = zero4();
    mm2<false, false>(e, sWc, sS, 16 * mt, n0w);
    mm2<false, false>(p, sQ, sK, 16 * mt, n0w);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = n0w + 16 * h + 4 * g;
      const f32x4 ucv = get_bf16(sUc, row, col);
#pragma unroll
      for (int r = 0; r < 4; ++r) e[h][r] = ucv[r] - e[h][r];
      put_bf16(sE, row, col, e[h]);
      const f32x4 gm = gam_tile(tk, row, col);
#pragma unroll
      for (int r = 0; r < 4; ++r) p[h][r] *= gm[r];
      put_bf16(sP, row, col, p[h]);
      dlg[h] = zero4();
    }
  }
  __syncthreads();
  // B1: dE = P^T dO + D (K dH'); dP = lower(dO E^T) -> Zp = Gam * dP; dG from Q H;
  //     dQ = G dO H^T; E dH'^T -> dK, dD
  {
    f32x4 a1[2] = {zero4(), zero4()}, a2[2] = {zero4(), zero4()};
    mm2<true, true>(a1, sP, sdO, 16 * mt, n0w);
    mm2<false, false>(a2, sK, sLam, 16 * mt, n0w);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 de;
#pragma unroll
      for (int r = 0; r < 4; ++r) de[r] = a1[h][r] + D_i * a2[h][r];
      put_bf16(sdE, row, n0w + 16 * h + 4 * g, de);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    f32x4 dp[2] = {zero4(), zero4()}, qh[2] = {zero4(), zero4()};
    mm2<false, false>(dp, sdO, sE, 16 * mt, n0w);
    mm2<false, false>(qh, sQ, sS, 16 * mt, n0w);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = n0w + 16 * h + 4 * g;
      const f32x4 gm = gam_tile(tk, row, col);
      const f32x4 dov = get_bf16(sdO, row, col);
      f32x4 zp;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d = col + r <= row ? dp[h][r] : 0.f;
        dlg[h][r] += d * p[h][r];
        zp[r] = gm[r] * d;
        rb_gv += dov[r] * qh[h][r];
      }
      put_bf16(sZ, row, col, zp);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    dq[0] = zero4();
    dq[1] = zero4();
    mm2<false, true>(dq, sdO, sS, 16 * mt, n0w);
    f32x4 edh[2] = {zero4(), zero4()};
    mm2<false, true>(edh, sE, sLam, 16 * mt, n0w);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 kv = get_bf16(sK, row, n0w + 16 * h + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dq[h][r] *= G_i;
        dk[h][r] = D_i * edh[h][r];
        rb_dd += kv[r] * edh[h][r];
      }
    }
  }
  __syncthreads();
  // B2: dX1 = T^T dE -> dVp (LDS, and dv's direct part), dbeta; dWc = -dE H^T;
  //     dQ += Zp K; dK += Zp^T Q
  float* dvg = a.dv + grow * D;
  {
    f32x4 dx1[2] = {zero4(), zero4()}, dwc[2] = {zero4(), zero4()};
    mm2<true, true>(dx1, sT, sdE, 16 * mt, n0w);
    mm2<false, true>(dwc, sdE, sS, 16 * mt, n0w);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = n0w + 16 * h + 4 * g;
      f32x4 dvp;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dvp[r] = beta_i * dx1[h][r];
        rb_beta += vp[h][r] * dx1[h][r];
        dwc[h][r] = -dwc[h][r];
      }
      put_bf16(sdVp, row, col, dvp);
      if (in_i) *reinterpret_cast<f32x4*>(dvg + col) = dvp;
      put_bf16(sdWc, row, col, dwc[h]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  mm2<false, true>(dq, sZ, sK, 16 * mt, n0w);
  mm2<true, true>(dk, sZ, sQ, 16 * mt, n0w);
  __syncthreads();
  // B3: dX2 = T^T dWc -> dK, dbeta, dG; Y = dE Uc^T + dWc Wc^T (into E's slot)
  bf16_t* sY = sE;
  {
    f32x4 dx2[2] = {zero4(), zero4()};
    mm2<true, true>(dx2, sT, sdWc, 16 * mt, n0w);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 kv = get_bf16(sK, row, n0w + 16 * h + 4 * g);
      float rk = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rk += kv[r] * dx2[h][r];
        dk[h][r] += beta_i * G_i * dx2[h][r];
      }
      rb_beta += G_i * rk;
      rb_gv += beta_i * rk;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    f32x4 y[2] = {zero4(), zero4()};
    mm2<false, false>(y, sdE, sUc, 16 * mt, n0w);
    mm2<false, false>(y, sdWc, sWc, 16 * mt, n0w);
#pragma unroll
    for (int h = 0; h < 2; ++h) put_bf16(sY, row, n0w + 16 * h + 4 * g, y[h]);
  }
  __syncthreads();
  // B4: dA = strict(-T^T Y) -> dbeta, dlG, Z = diag(beta) Gam * dA (into P's slot)
  bf16_t* sZ2 = sP;
  {
    f32x4 t[2] = {zero4(), zero4()}, kk[2] = {zero4(), zero4()};
    mm2<true, true>(t, sT, sY, 16 * mt, n0w);
    mm2<false, false>(kk, sK, sK, 16 * mt, n0w);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = n0w + 16 * h + 4 * g;
      const f32x4 gm = gam_tile(tk, row, col);
      f32x4 z;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float da = col + r < row ? -t[h][r] : 0.f;
        const float gk = gm[r] * kk[h][r];
        rb_beta += da * gk;
        dlg[h][r] += da * beta_i * gk;
        z[r] = beta_i * gm[r] * da;
      }
      put_bf16(sZ2, row, col, z);
    }
  }
  __syncthreads();
  // B5: dK += Z K + Z^T K
  mm2<false, true>(dk, sZ2, sK, 16 * mt, n0w);
  mm2<true, true>(dk, sZ2, sK, 16 * mt, n0w);
  // B6: rank slots, descending
  bf16_t *sN = x.m(mN), *sPU = x.m(mT), *sZpu = x.m(mX1), *sZn = x.m(mX2);
  float* sdR = x.mf(mUc);
  float dr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) dr[e] = 0.f;
  float da_carry = 0.f;
  // thread (ct, 8 channels cc ..) of the chain: u rows, r_{l-1} (as the local pass formed it)
  // and gamma_{l-1} of the next slot are loaded one slot ahead
  const int ct = tid >> 3, cc = 8 * (tid & 7);
  const bool in_t = x.L > 1 && ct < x.nt;
  const size_t tg = (size_t)x.pr * a.T + x.t0 + ct;
  const bf16_t* ug = static_cast<const bf16_t*>(a.u) + ((size_t)x.pr * a.T + x.t0) * (x.L - 1) * D;
  const bf16_t* gg = static_cast<const bf16_t*>(a.gamma) + ((size_t)x.pr * a.T + x.t0) * (x.L - 1) * D;
  const bf16_t* rin = cm + 4 * 4096;
  uint4 pu = {0u, 0u, 0u, 0u}, pr_ = {0u, 0u, 0u, 0u}, pg = {0u, 0u, 0u, 0u};
  if (x.L > 1) {
    if (in_t) {
      pu = *reinterpret_cast<const uint4*>(ug + (size_t)ct * (x.L - 1) * D + (size_t)(x.L - 2) * D + cc);
      pg = *reinterpret_cast<const uint4*>(gg + (size_t)ct * (x.L - 1) * D + (size_t)(x.L - 2) * D + cc);
    }
    pr_ = *reinterpret_cast<const uint4*>(rin + (size_t)(x.L - 2) * 4096 + ct * 64 + cc);
  }
#pragma unroll 1
  for (int lv = x.L - 1; lv >= 1; --lv) {
    // slot lv: U_lv, R_lv = alpha_lv r_lv with r_lv = r_{lv-1} (1 - alpha_{lv-1} gamma_{lv-1})
    *reinterpret_cast<uint4*>(sU + ct * LDM + cc) = pu;
    const uint4 cr = pr_, cgv = pg;  // this slot's r_{lv-1} and gamma_{lv-1}, kept packed
    {
      const bf16x8 rv = __builtin_bit_cast(bf16x8, cr), gv = __builtin_bit_cast(bf16x8, cgv);
      const float alm = tk[kAl + (lv - 1) * 64 + ct], al = tk[kAl + lv * 64 + ct];
      bf16x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (bf16_t)(al * ((float)rv[e] * (1.f - alm * (float)gv[e])));
      *reinterpret_cast<bf16x8*>(sR + ct * LDM + cc) = y;
    }
    __syncthreads();
    if (lv > 1) {
      if (in_t) {
        pu = *reinterpret_cast<const uint4*>(ug + (size_t)ct * (x.L - 1) * D + (size_t)(lv - 2) * D + cc);
        pg = *reinterpret_cast<const uint4*>(gg + (size_t)ct * (x.L - 1) * D + (size_t)(lv - 2) * D + cc);
      }
      pr_ = *reinterpret_cast<const uint4*>(rin + (size_t)(lv - 2) * 4096 + ct * 64 + cc);
    }
    {
      const int n0 = 16 * nt0;
      f32x4 n[2] = {zero4(), zero4()}, pu[2] = {zero4(), zero4()};
      mm2b<false, false>(n, pu, sK, sQ, sU, 16 * mt, n0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = n0 + 16 * h + 4 * g;
        const f32x4 gm = gam_tile(tk, row, col);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          n[h][r] = col + r < row ? gm[r] * n[h][r] : 0.f;
          pu[h][r] = gm[r] * pu[h][r];
        }
        put_bf16(sN, row, col, n[h]);
        put_bf16(sPU, row, col, pu[h]);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4 dpu[2] = {zero4(), zero4()}, dn[2] = {zero4(), zero4()};
      mm2b<false, false>(dpu, dn, sdO, sdVp, sR, 16 * mt, n0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = n0 + 16 * h + 4 * g;
        const f32x4 gm = gam_tile(tk, row, col);
        f32x4 zpu, zn;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool lo = col + r <= row, st = col + r < row;
          const float dp = lo ? dpu[h][r] : 0.f, dq_ = st ? -dn[h][r] : 0.f;
          dlg[h][r] += dp * pu[h][r] + dq_ * n[h][r];
          zpu[r] = gm[r] * dp;
          zn[r] = gm[r] * dq_;
        }
        put_bf16(sZpu, row, col, zpu);
        put_bf16(sZn, row, col, zn);
      }
    }
    __syncthreads();
    float* dug = a.du + (grow * (x.L - 1) + lv - 1) * D;
    {
      // groups of products sharing their A operand across the wave's two tiles, fenced so
      // that one group's temporaries are live at a time (register budget)
      const int n0 = 16 * nt0;
      {
        f32x4 udh[2] = {zero4(), zero4()}, drt[2] = {zero4(), zero4()};
        mm2<false, false>(udh, sU, sLam, 16 * mt, n0);
        mm2<true, true>(drt, sPU, sdO, 16 * mt, n0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) drt[h][r] += D_i * udh[h][r];
        f32x4 ndv[2] = {zero4(), zero4()};
        mm2<true, true>(ndv, sN, sdVp, 16 * mt, n0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int r = 0; r < 4; ++r) drt[h][r] -= ndv[h][r];
          *reinterpret_cast<f32x4*>(sdR + row * LDF + n0 + 16 * h + 4 * g) = drt[h];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        f32x4 rdh[2] = {zero4(), zero4()}, du[2] = {zero4(), zero4()};
        mm2<false, true>(rdh, sR, sLam, 16 * mt, n0);
        mm2<true, true>(du, sZpu, sQ, 16 * mt, n0);
        mm2<true, true>(du, sZn, sK, 16 * mt, n0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = n0 + 16 * h + 4 * g;
          const f32x4 uv = get_bf16(sU, row, col);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            rb_dd += uv[r] * rdh[h][r];
            du[h][r] += D_i * rdh[h][r];
          }
          if (in_i) *reinterpret_cast<f32x4*>(dug + col) = du[h];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      mm2b<false, true>(dq, dk, sZpu, sZn, sU, 16 * mt, n0);
    }
    __syncthreads();
    // the chain's adjoint for slot lv
    {
      const float4 d0 = *reinterpret_cast<const float4*>(sdR + ct * LDF + cc);
      const float4 d1 = *reinterpret_cast<const float4*>(sdR + ct * LDF + cc + 4);
      const float dR[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      const bf16x8 rv = __builtin_bit_cast(bf16x8, cr), gv = __builtin_bit_cast(bf16x8, cgv);
      const float al = tk[kAl + lv * 64 + ct], alm = tk[kAl + (lv - 1) * 64 + ct];
      float s = 0.f, s2 = 0.f;
      float dgm[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float rp = (float)rv[e], gm = (float)gv[e], fl = 1.f - alm * gm;
        s += dR[e] * (rp * fl);
        dr[e] += al * dR[e];
        s2 += dr[e] * gm * rp;
        dgm[e] = -dr[e] * alm * rp;
        dr[e] *= fl;
      }
      s = sum8(s) + da_carry;
      da_carry = -sum8(s2);
      if (in_t) {
        if ((tid & 7) == 0) a.dalpha[tg * x.L + lv] = s;
        float* dgp = a.dgamma + (tg * (x.L - 1) + lv - 1) * D + cc;
        *reinterpret_cast<float4*>(dgp) = make_float4(dgm[0], dgm[1], dgm[2], dgm[3]);
        *reinterpret_cast<float4*>(dgp + 4) = make_float4(dgm[4], dgm[5], dgm[6], dgm[7]);
      }
    }
  }
  // the direct part of dv (stored by this workgroup in B2), for the anchor terms at the end
  float dvd[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (in_t) {
    const float4 d0 = *reinterpret_cast<const float4*>(a.dv + tg * D + cc);
    const float4 d1 = *reinterpret_cast<const float4*>(a.dv + tg * D + cc + 4);
    dvd[0] = d0.x; dvd[1] = d0.y; dvd[2] = d0.z; dvd[3] = d0.w;
    dvd[4] = d1.x; dvd[5] = d1.y; dvd[6] = d1.z; dvd[7] = d1.w;
  }
  // row partials of this lane's row over the wave's 32 columns; the decay-weighted adjoint
  // W = dlG (W_ij = Gam_ij dL/dGam_ij, lower triangular) into LDS for its rectangle sums
  float* sWl = x.mf(mQ);  // float32 [64][LDF] over slots Q and K (free after the rank loop)
  {
    const float s_beta = sum_groups(rb_beta), s_gv = sum_groups(rb_gv), s_dd = sum_groups(rb_dd);
    if (g == 0) {
      tk[kRowBeta + half * 64 + row] = s_beta;
      tk[kRowGv + half * 64 + row] = s_gv;
      tk[kRowDd + half * 64 + row] = s_dd;
    }
    __syncthreads();  // every product that read slots Q and K is done
#pragma unroll
    for (int h = 0; h < 2; ++h) *reinterpret_cast<f32x4*>(sWl + row * LDF + 16 * (nt0 + h) + 4 * g) = dlg[h];
  }
  float* sW = x.mf(mT);  // the head's conv taps [4][64] (slot T is free after the rank loop)
  if (x.L > 1) {
    // d r_0 of the chain, for the anchor's terms
#pragma unroll
    for (int e = 0; e < 8; e += 4)
      *reinterpret_cast<float4*>(sdR + ct * LDF + cc + e) = make_float4(dr[e], dr[e + 1], dr[e + 2], dr[e + 3]);
    if ((tid & 7) == 0 && in_t) a.dalpha[tg * x.L] = da_carry;
    if (tid < 4 * D) sW[tid] = a.conv_w[(size_t)(x.pr % a.H) * 4 * D + tid];
  }
  __syncthreads();
  {
    // E[i][s] = sum_{j < s} W[i][j], in place: eight threads per row, eight columns each
    const int ri = tid >> 3, seg = tid & 7;
    float* wr = sWl + ri * LDF + 8 * seg;
    const float4 w0 = *reinterpret_cast<const float4*>(wr), w1 = *reinterpret_cast<const float4*>(wr + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float tot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) tot += wv[e];
    // the totals of the row's earlier column blocks (lanes seg' < seg of the same 8)
    float off = 0.f;
#pragma unroll
    for (int o = 1; o < 8; ++o) {
      const float y = __shfl(tot, (lane_id() & ~7) + ((seg - o) & 7));
      if (seg - o >= 0) off += y;
    }
    float ex[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ex[e] = off;
      off += wv[e];
    }
    *reinterpret_cast<float4*>(wr) = make_float4(ex[0], ex[1], ex[2], ex[3]);
    *reinterpret_cast<float4*>(wr + 4) = make_float4(ex[4], ex[5], ex[6], ex[7]);
  }
  __syncthreads();
  {
    // C(s) = sum_{i >= s} E[i][s] = sum_{i >= s > j} W[i][j]: eight threads per s, rows
    // part, part + 8, ...; only entries whose decay spans token s enter, so a token with a
    // tiny gate gets a tiny sum instead of a difference of two large ones
    const int sc = tid >> 3, part = tid & 7;
    float cs = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int ri = part + 8 * k;
      if (ri >= sc) cs += sWl[ri * LDF + sc];
    }
    cs += __shfl_xor(cs, 1);
    cs += __shfl_xor(cs, 2);
    cs += __shfl_xor(cs, 4);
    if (part == 0) tk[kColLg + sc] = cs;
  }
  __syncthreads();
  {
    float* dqg = a.dq + grow * D;
    float* dkg = a.dk + grow * D;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = 16 * (nt0 + h) + 4 * g;
      if (in_i) {
        *reinterpret_cast<f32x4*>(dqg + col) = dq[h];
        *reinterpret_cast<f32x4*>(dkg + col) = dk[h];
      }
    }
  }
  if (tid < 64) {
    // d log g_s = sum_{t >= s} G_t dL/dG_t (+ G_C dL/dG_C) + sum_{t < s} D_t dL/dD_t
    // + C(s), each a sum of terms that carry g_s (G_t = prod_{u <= t} g_u, D_t =
    // prod_{u > t} g_u); dg = d log g / g.  dbeta (wave 0, one token per lane).
    const int t = tid;
    const float Gt = tk[kG + t], Dt = tk[kDd + t];
    const float dD = tk[kRowDd + t] + tk[kRowDd + 64 + t];
    const float dGv = tk[kRowGv + t] + tk[kRowGv + 64 + t];
    float gsum = dGv * Gt;
    if (t == 63) {
      float dGC = 0.f;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) dGC += tk[kMisc + ww];
      gsum += dGC * Gt;
    }
    // suffix sum of the G terms over lanes t .. 63
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_down(gsum, o);
      if (t + o < 64) gsum += y;
    }
    // exclusive prefix sum of the D terms over lanes 0 .. t - 1
    const float dterm = dD * Dt;
    float dsum = __shfl_up(dterm, 1);
    if (t == 0) dsum = 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(dsum, o);
      if (t >= o) dsum += y;
    }
    const float dlog = gsum + dsum + tk[kColLg + t];
    if (t < x.nt) {
      const size_t gi = (size_t)x.pr * a.T + x.t0 + t;
      a.dg[gi] = dlog / tk[kGg + t];
      a.dbeta[gi] = tk[kRowBeta + t] + tk[kRowBeta + 64 + t];
    }
  }
  if (x.L > 1) {
    const size_t ps = (size_t)x.pr * a.nseg + x.c;
    const float* w = sW;
    // dv += d r_0 - sum_j w_j d r_0(t + 3 - j) over the chunk's anchors that read v_t
    if (in_t) {
      float out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ch = cc + e;
        float s = dvd[e] + sdR[ct * LDF + ch];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ta = ct + 3 - j;
          if (ta < C) s -= w[j * D + ch] * sdR[ta * LDF + ch];
        }
        out[e] = s;
      }
      float* dvp = a.dv + tg * D + cc;
      *reinterpret_cast<float4*>(dvp) = make_float4(out[0], out[1], out[2], out[3]);
      *reinterpret_cast<float4*>(dvp + 4) = make_float4(out[4], out[5], out[6], out[7]);
    }
    if (tid < 3 * D) {
      // the terms owed to tokens t0 - 1 - jj of the previous chunk
      const int jj = tid / D, ch = tid % D;
      float s = 0.f;
      for (int t = 0; t <= 2 - jj; ++t) s -= w[(2 - jj - t) * D + ch] * sdR[t * LDF + ch];
      a.carry[(ps * 3 + jj) * D + ch] = s;
    }
    // dconv_w share: dw_j = -sum_t d r_0(t) v_{t-3+j}, each (tap, channel) over two halves of
    // the tokens (threads tid and tid + 256), four independent partial sums per half
    float* sPart = x.mf(mU);  // [2][256] (slot U is free after the rank loop)
    {
      const int hf = tid >> 8, j = (tid & 255) >> 6, ch = tid & 63;
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int t = 32 * hf; t < 32 * hf + 32; ++t) s4[t & 3] -= sdR[t * LDF + ch] * (float)sVx[(t + j) * 64 + ch];
      sPart[tid] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    __syncthreads();
    if (tid < 256) a.dconv_part[ps * 4 * D + tid] = sPart[tid] + sPart[256 + tid];
  }
}

}  // namespace bwdc
}  // namespace prism
