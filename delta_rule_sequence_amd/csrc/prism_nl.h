// prism_nl.h - PRISM's nonlinear residual refinement as per-channel chain factors (gfx950).
//
// In the nonlinear form each refinement layer subtracts a correction formed by a GELU of
// the gain-modulated residual, p ⊙ r ("PRISM" reading notes, section 2.3: greedy residual
// subtraction).  The Tencent Ads article (section 03-三) folds that GELU into precomputed
// scaling factors, which leaves an element-wise linear chain.  For the exact erf GELU the
// fold is exact: GELU(z) = z Phi(z), so
//
//   alpha GELU(p r) = alpha (p Phi(p r)) r,   i.e.  gamma = p Phi(p r),
//
// evaluated on the chain's own residuals.  nl_gain_kernel walks the chain once per token
// and channel and writes those factors; the linear forward (any of its entry points) run
// with them is the nonlinear forward.  Each factor is rounded to the I/O type before the
// chain moves on with it, exactly as the forward's chain will use it, so both evaluate the
// same residuals.  nl_pred_gain_kernel does the same with gains predicted from the anchor;
// the bf16 d = 64 sweep (prism_sweep8.h) evaluates the factors in its own chain with
// std_normal_cdf below.
//
// nl_gain_kernel: one thread per (pair, token, 4 value channels), element-wise and
// HBM-bound: per token-head it reads v (and the three earlier rows, from cache), L - 1 gain
// rows and L step sizes, and writes L - 1 factor rows.
#pragma once
#include "prism_kernels.h"

namespace prism {

struct NlArgs {
  const void* v;        // [P][T][dv]
  const float* alpha;   // [P][T][L]
  const void* p;        // [P][T][L-1][dv]
  const float* conv_w;  // [H][4][dv]
  const void* conv_in;  // [P][3][dv] values of the three tokens before the sequence, or null
  void* gamma;          // out [P][T][L-1][dv]
  int H, T, L, dv;
  int lognc;            // log2(dv / 4): a pair's T * dv / 4 groups are token-major
};

// Standard normal CDF Phi(z) = erfc(-z / sqrt 2) / 2, erfc by the rational approximation of
// Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26 (after
// Hastings): for x >= 0, erfc(x) = t (a1 + a2 t + a3 t^2 + a4 t^3 + a5 t^4) exp(-x^2),
// t = 1 / (1 + p x), with absolute error below 1.5e-7.  One reciprocal, one exponential
// and five multiply-adds, against several times that for a full-accuracy erfc: the factor
// kernel would otherwise be bound by this function, not by memory.
__device__ __forceinline__ float std_normal_cdf(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(1.f + 0.3275911f * x);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float half_erfc = 0.5f * poly * __expf(-x * x);
  return z >= 0.f ? 1.f - half_erfc : half_erfc;
}

template <class E> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ float4 load(const float* x) { return *reinterpret_cast<const float4*>(x); }
  static __device__ __forceinline__ void store(float* x, const float4& y) { *reinterpret_cast<float4*>(x) = y; }
};
template <> struct Vec4<bf16_t> {
  typedef bf16_t b4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ float4 load(const bf16_t* x) {
    const b4 y = *reinterpret_cast<const b4*>(x);
    return make_float4((float)y[0], (float)y[1], (float)y[2], (float)y[3]);
  }
  static __device__ __forceinline__ void store(bf16_t* x, const float4& y) {
    const b4 z = {(bf16_t)y.x, (bf16_t)y.y, (bf16_t)y.z, (bf16_t)y.w};
    *reinterpret_cast<b4*>(x) = z;
  }
};

__device__ __forceinline__ float f4get(const float4& x, int i) { return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w; }

// grid (ceil(T * dv / 4 / 256), P): 32-bit indexing inside a pair, no division.
// DLT: the written-correction chain (notes, section 2.3: the correction GELU(p r) is
// subtracted as it is and written): r <- r - f r with the rounded factor f, alpha unread.
template <class E, bool DLT>
__global__ __launch_bounds__(256) void nl_gain_kernel(NlArgs a) {
  const unsigned j = blockIdx.x * 256u + threadIdx.x;
  const int L = a.L, Lm1 = L - 1, dv = a.dv;
  if (j >= ((unsigned)a.T << a.lognc)) return;
  const int c4 = 4 * (int)(j & ((1u << a.lognc) - 1));
  const int t = (int)(j >> a.lognc);
  const int pri = blockIdx.y;
  const int hd = pri % a.H;
  const size_t pr = (size_t)pri;
  const size_t pt = pr * a.T + t;
  const E* v = reinterpret_cast<const E*>(a.v) + (size_t)pr * a.T * dv;
  const E* ci = a.conv_in != nullptr ? reinterpret_cast<const E*>(a.conv_in) + (size_t)pr * 3 * dv : nullptr;
  // value rows t-3 .. t; rows before the sequence come from the given history, else zero
  float4 x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = t - 3 + j;
    if (s >= 0)
      x[j] = Vec4<E>::load(v + (size_t)s * dv + c4);
    else if (ci != nullptr)
      x[j] = Vec4<E>::load(ci + (size_t)(s + 3) * dv + c4);
    else
      x[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float* w = a.conv_w + (size_t)hd * 4 * dv + c4;
  const float4 w0 = *reinterpret_cast<const float4*>(w), w1 = *reinterpret_cast<const float4*>(w + dv);
  const float4 w2 = *reinterpret_cast<const float4*>(w + 2 * dv), w3 = *reinterpret_cast<const float4*>(w + 3 * dv);
  float r[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    r[c] = f4get(x[3], c) - (f4get(w0, c) * f4get(x[0], c) + f4get(w1, c) * f4get(x[1], c) +
                             f4get(w2, c) * f4get(x[2], c) + f4get(w3, c) * f4get(x[3], c));
  const float* al = DLT ? nullptr : a.alpha + (size_t)pt * L;
  const E* pg = reinterpret_cast<const E*>(a.p) + (size_t)pt * Lm1 * dv + c4;
  E* gm = reinterpret_cast<E*>(a.gamma) + (size_t)pt * Lm1 * dv + c4;
  for (int l = 0; l < Lm1; ++l) {
    const float4 pv = Vec4<E>::load(pg + (size_t)l * dv);
    const float at = DLT ? 1.f : al[l];
    float f[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float pc = f4get(pv, c);
      f[c] = pc * std_normal_cdf(pc * r[c]);
    }
    Vec4<E>::store(gm + (size_t)l * dv, make_float4(f[0], f[1], f[2], f[3]));
    // move on with the stored (rounded) factor, as the forward's chain will
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (DLT) {
        const float d = to_f(from_f<E>(f[c])) * r[c];
        r[c] -= d;
      } else {
        r[c] = r[c] * (1.f - at * to_f(from_f<E>(f[c])));
      }
    }
  }
}

// Gains from a linear predictor on the anchor, fused with the factor pass ("PRISM" notes,
// section 2.3: the gains come from predictors that read the ShortConv anchor):
//   p_{t,l} = W_p[h][l] anchor_t    (W_p [H][L-1][D][D], (out, in) layout, bfloat16)
// then the factors as in nl_gain_kernel.  The gains never touch memory: per token-head the
// pass reads v and the step sizes and writes the factors (W_p, D x D per level and head,
// stays in cache).  One workgroup of 4 waves per 4 x 16 TPW tokens of a pair; wave w takes
// 16 TPW consecutive tokens on its own:
//   * its value window (3 rows of halo) and step sizes are staged in LDS;
//   * per 16-token tile the anchor, rounded to bfloat16, is the A operand of 16x16x32
//     MFMAs (lane: token li, channels 32 kb + 8 g .. + 7, from 16-byte LDS reads); the B
//     operand of output tile nt in lane li is row NT li + nt of W_p (one 16-byte load), so
//     lane (li, g) ends with p for tokens 4 g + rr and the NT adjacent channels NT li ..:
//   * the residual chain runs in that layout (r from 8-byte window reads, in the
//     forward's order of operations) and each token's NT factors leave as one vector store.
// Ruled out at the 16K shape: one 16-token tile per wave re-read each level's weights for
// every 16 tokens (46-51 us, whatever the LDS layout or occupancy).
struct NlPredArgs {
  const void* v;        // [P][T][D] bf16
  const float* alpha;   // [P][T][L] (the linear chain's step sizes; unread by the front end)
  const void* W_p;      // [H][L-1][D][D] bf16
  const float* conv_w;  // [H][4][D]
  const void* conv_in;  // [P][3][D] bf16, or null
  void* gamma;          // out [P][T][L-1][D] bf16
  // the front end only: key and gate predictors and their outputs
  const void* W_k;      // [H][L-1][D][D] bf16 ((out, in): key channel, anchor channel)
  const void* W_b;      // [H][L][D] bf16
  void* u;              // out [P][T][L-1][D] bf16: unit keys
  float* alpha_out;     // out [P][T][L]: gates
  int H, T, L;
};

// N adjacent bfloat16 values as one LDS / global access (N = 2, 4, 8)
template <int N> struct BfN;
template <> struct BfN<2> { typedef unsigned raw; };
template <> struct BfN<4> { typedef uint2 raw; };
template <> struct BfN<8> { typedef uint4 raw; };
template <int N>
__device__ __forceinline__ void bf_load(const bf16_t* p, float (&x)[N]) {
  const typename BfN<N>::raw r = *reinterpret_cast<const typename BfN<N>::raw*>(p);
  const bf16_t* b = reinterpret_cast<const bf16_t*>(&r);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = (float)b[i];
}
template <int N>
__device__ __forceinline__ void bf_store(bf16_t* p, const bf16_t (&x)[N]) {
  typename BfN<N>::raw r;
  bf16_t* b = reinterpret_cast<bf16_t*>(&r);
#pragma unroll
  for (int i = 0; i < N; ++i) b[i] = x[i];
  *reinterpret_cast<typename BfN<N>::raw*>(p) = r;
}

// Wave w of a workgroup takes TPW consecutive 16-token tiles (TPW = 4 for d = 64, so each
// level's W_p fragments are loaded once for 64 tokens: the weights' cache traffic is a
// quarter of one tile per wave; 243 VGPRs, two waves per SIMD, no spills).
//
// DLT: the written-correction chain, r <- r - f r (notes, section 2.3: greedy residual
// subtraction without a step size).  FRONT (with DLT): the whole predictor front end of
// the notes' Phase 1 from the same anchor operands: per level the keys W_k[h, l] anchor,
// normalised over their channels (a 16-lane sum of squares), and once per tile the gates
// sigmoid(W_b[h, l] . anchor) for l < L as one more MFMA tile (output column l = gate l).
template <int D, bool DLT, bool FRONT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1)))
void nl_pred_gain_kernel(NlPredArgs a) {
  static_assert(D == 32 || D == 64 || D == 128, "32-deep MFMA contraction over the channels");
  static_assert(!FRONT || DLT, "the front end feeds the written-correction chain");
  constexpr int TPW = D == 64 ? 4 : 1;
  constexpr int ROWS = 16 * TPW + 3;  // a wave's value window
  constexpr int LDV = D + 8;          // LDS row stride (bf16)
  constexpr int KB = D / 32, NT = D / 16, PIECES = D / 8;
  __shared__ __align__(16) bf16_t sV[4][ROWS * LDV];  // per wave: value rows tw-3 .. tw+16 TPW-1
  __shared__ float sA[4][16 * TPW * 8];               // per wave: step sizes [token][level]
  const int w = wave_id(), l = lane_id(), li = l & 15, g = l >> 4;
  const int pr = blockIdx.y, hd = pr % a.H, T = a.T, L = a.L, Lm1 = L - 1;
  const int tw = (blockIdx.x * 4 + w) * 16 * TPW;
  const bf16_t* v = reinterpret_cast<const bf16_t*>(a.v) + (size_t)pr * T * D;
  const bf16_t* ci = a.conv_in != nullptr ? reinterpret_cast<const bf16_t*>(a.conv_in) + (size_t)pr * 3 * D : nullptr;
  bf16_t* sv = sV[w];
  // rows before the sequence come from the history (else zero); rows past its end are zero
  for (int i = l; i < ROWS * PIECES; i += 64) {
    const int rr = i / PIECES, cv = (i % PIECES) * 8;
    const int s = tw - 3 + rr;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (s >= 0 && s < T)
      x = *reinterpret_cast<const uint4*>(v + (size_t)s * D + cv);
    else if (s < 0 && ci != nullptr)
      x = *reinterpret_cast<const uint4*>(ci + (size_t)(s + 3) * D + cv);
    *reinterpret_cast<uint4*>(sv + rr * LDV + cv) = x;
  }
  if constexpr (!DLT) {
    const float* al = a.alpha + (size_t)pr * T * L;
    for (int i = l; i < 16 * TPW * L; i += 64) {
      const int tok = tw + i / L;
      sA[w][i] = tok < T ? al[(size_t)tok * L + i % L] : 0.f;
    }
  }
  __syncthreads();
  const float* cw = a.conv_w + (size_t)hd * 4 * D;
  // A operands: anchor of token 16 j + li, channels 32 kb + 8 g .. + 7
  bf16x8 an[TPW][KB];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int c0 = 32 * kb + 8 * g;
      float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        float x[8];
        bf_load<8>(sv + (16 * j + li + jt) * LDV + c0, x);
        const float4 wa = *reinterpret_cast<const float4*>(cw + jt * D + c0);
        const float4 wb = *reinterpret_cast<const float4*>(cw + jt * D + c0 + 4);
        const float wt[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) s8[q] += wt[q] * x[q];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) an[j][kb][q] = (bf16_t)s8[q];
    }
  // residuals of tokens 16 j + 4 g + rr, channels NT li + nt
  const int cl = NT * li;
  float r[TPW][4][NT];
  {
    float wt[4][NT];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) wt[jt][nt] = cw[jt * D + cl + nt];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int tok = 16 * j + 4 * g + rr;  // window rows tok .. tok + 3, the token itself last
        float x0[NT], x1[NT], x2[NT], x3[NT];
        bf_load<NT>(sv + tok * LDV + cl, x0);
        bf_load<NT>(sv + (tok + 1) * LDV + cl, x1);
        bf_load<NT>(sv + (tok + 2) * LDV + cl, x2);
        bf_load<NT>(sv + (tok + 3) * LDV + cl, x3);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          r[j][rr][nt] = x3[nt] - (wt[0][nt] * x0[nt] + wt[1][nt] * x1[nt] + wt[2][nt] * x2[nt] + wt[3][nt] * x3[nt]);
      }
  }
  const bf16_t* Wh = reinterpret_cast<const bf16_t*>(a.W_p) + (size_t)hd * Lm1 * D * D;
  bf16_t* gout = reinterpret_cast<bf16_t*>(a.gamma) + (size_t)pr * T * Lm1 * D;
  for (int lv = 0; lv < Lm1; ++lv) {
    // this level's weight fragments, loaded once for the wave's TPW tiles
    const bf16_t* W = Wh + (size_t)lv * D * D;
    bf16x8 wf[NT][KB];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        wf[nt][kb] = *reinterpret_cast<const bf16x8*>(W + (size_t)(cl + nt) * D + 32 * kb + 8 * g);
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      bf16_t fb[4][NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = mfma(an[j][kb], wf[nt][kb], acc);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float pv = acc[rr];
          fb[rr][nt] = (bf16_t)(pv * std_normal_cdf(pv * r[j][rr][nt]));
        }
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int tl = 16 * j + 4 * g + rr, tok = tw + tl;
        if constexpr (DLT) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float d = (float)fb[rr][nt] * r[j][rr][nt];
            r[j][rr][nt] -= d;
          }
        } else {
          const float at = sA[w][tl * L + lv];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) r[j][rr][nt] = r[j][rr][nt] * (1.f - at * (float)fb[rr][nt]);
        }
        if (tok < T) bf_store<NT>(gout + ((size_t)tok * Lm1 + lv) * D + cl, fb[rr]);
      }
    }
    if constexpr (FRONT) {
      // keys u_{t, lv+1} = W_k[h, lv] anchor_t / |W_k[h, lv] anchor_t|, tokens 16 j + 4 g + rr,
      // channels NT li ..: the weight fragments take wf's registers
      const bf16_t* Wkl = reinterpret_cast<const bf16_t*>(a.W_k) + ((size_t)hd * Lm1 + lv) * D * D;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          wf[nt][kb] = *reinterpret_cast<const bf16x8*>(Wkl + (size_t)(cl + nt) * D + 32 * kb + 8 * g);
      bf16_t* uout = reinterpret_cast<bf16_t*>(a.u) + (size_t)pr * T * Lm1 * D;
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        float kv[4][NT], ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) acc = mfma(an[j][kb], wf[nt][kb], acc);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            kv[rr][nt] = acc[rr];
            ss[rr] += acc[rr] * acc[rr];
          }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          // a token's channels sit in the 16 lanes of its lane group g
#pragma unroll
          for (int m = 1; m < 16; m <<= 1) ss[rr] += __shfl_xor(ss[rr], m, 16);
          const float inv = 1.f / sqrtf(ss[rr]);
          const int tok = tw + 16 * j + 4 * g + rr;
          bf16_t kb16[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) kb16[nt] = (bf16_t)(kv[rr][nt] * inv);
          if (tok < T) bf_store<NT>(uout + ((size_t)tok * Lm1 + lv) * D + cl, kb16);
        }
      }
    }
  }
  if constexpr (FRONT) {
    // gates alpha_{t, l} = sigmoid(W_b[h, l] . anchor_t): B operand row li = W_b[h, li]
    // (zero for li >= L), so lane (li, g) ends with gate li of tokens 16 j + 4 g + rr
    const bf16_t* Wb = reinterpret_cast<const bf16_t*>(a.W_b) + (size_t)hd * L * D;
    bf16x8 bfr[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (li < L) {
        bfr[kb] = *reinterpret_cast<const bf16x8*>(Wb + (size_t)li * D + 32 * kb + 8 * g);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) bfr[kb][q] = (bf16_t)0.f;
      }
    }
    float* aout = a.alpha_out + (size_t)pr * T * L;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = mfma(an[j][kb], bfr[kb], acc);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int tok = tw + 16 * j + 4 * g + rr;
        if (li < L && tok < T) aout[(size_t)tok * L + li] = 1.f / (1.f + __expf(-acc[rr]));
      }
    }
  }
}

// The d = 128 gains-only pass (linear chain) with the weights shared through LDS: a
// workgroup of 4 waves (one per SIMD, the registers of two) takes 128 consecutive tokens
// (wave w: two 16-token tiles, its value window and step sizes in LDS as above), and each
// level's W_p[h, l] (32 KB) is copied from memory into LDS once per workgroup, the next
// level's while the current one is used (two buffers, one barrier per level);
// nl_pred_gain_kernel at d = 128 reads a level's weights once per 16-token tile and wave.
// The anchors, residuals, products and chain are those of nl_pred_gain_kernel<128, false,
// false>.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void nl_pred_gain_lds_kernel(NlPredArgs a) {
  static_assert(D == 128, "the weights of one level fill 32 KB of LDS at d = 128");
  constexpr int NW = 4, TPW = 2, ROWS = 16 * TPW + 3, LDV = D + 8, LDW = D + 8;
  constexpr int KB = D / 32, NT = D / 16, PIECES = D / 8;
  __shared__ __align__(16) bf16_t sV[NW][ROWS * LDV];  // per wave: value rows tw-3 .. tw+31
  __shared__ float sA[NW][16 * TPW * 8];               // per wave: step sizes [token][level]
  __shared__ __align__(16) bf16_t sW[2][D * LDW];     // the current and the next level's W_p
  const int w = wave_id(), l = lane_id(), li = l & 15, g = l >> 4, tid = threadIdx.x;
  const int pr = blockIdx.y, hd = pr % a.H, T = a.T, L = a.L, Lm1 = L - 1;
  const int tw = (blockIdx.x * NW + w) * 16 * TPW;
  const bf16_t* v = reinterpret_cast<const bf16_t*>(a.v) + (size_t)pr * T * D;
  const bf16_t* ci = a.conv_in != nullptr ? reinterpret_cast<const bf16_t*>(a.conv_in) + (size_t)pr * 3 * D : nullptr;
  const bf16_t* Wh = reinterpret_cast<const bf16_t*>(a.W_p) + (size_t)hd * Lm1 * D * D;
  bf16_t* sv = sV[w];
  // rows before the sequence come from the history (else zero); rows past its end are zero
  for (int i = l; i < ROWS * PIECES; i += 64) {
    const int rr = i / PIECES, cv = (i % PIECES) * 8;
    const int s = tw - 3 + rr;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (s >= 0 && s < T)
      x = *reinterpret_cast<const uint4*>(v + (size_t)s * D + cv);
    else if (s < 0 && ci != nullptr)
      x = *reinterpret_cast<const uint4*>(ci + (size_t)(s + 3) * D + cv);
    *reinterpret_cast<uint4*>(sv + rr * LDV + cv) = x;
  }
  {
    const float* al = a.alpha + (size_t)pr * T * L;
    for (int i = l; i < 16 * TPW * L; i += 64) {
      const int tok = tw + i / L;
      sA[w][i] = tok < T ? al[(size_t)tok * L + i % L] : 0.f;
    }
  }
  // level 0's weights: 2048 16-byte pieces, eight per thread
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = tid + 64 * NW * q, row = i / PIECES, c8 = (i % PIECES) * 8;
    *reinterpret_cast<uint4*>(sW[0] + row * LDW + c8) = *reinterpret_cast<const uint4*>(Wh + (size_t)row * D + c8);
  }
  __syncthreads();
  const float* cw = a.conv_w + (size_t)hd * 4 * D;
  // A operands: anchor of token 16 j + li, channels 32 kb + 8 g .. + 7
  bf16x8 an[TPW][KB];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int c0 = 32 * kb + 8 * g;
      float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        float x[8];
        bf_load<8>(sv + (16 * j + li + jt) * LDV + c0, x);
        const float4 wa = *reinterpret_cast<const float4*>(cw + jt * D + c0);
        const float4 wb = *reinterpret_cast<const float4*>(cw + jt * D + c0 + 4);
        const float wt[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) s8[q] += wt[q] * x[q];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) an[j][kb][q] = (bf16_t)s8[q];
    }
  // residuals of tokens 16 j + 4 g + rr, channels NT li + nt
  const int cl = NT * li;
  float r[TPW][4][NT];
  {
    float wt[4][NT];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) wt[jt][nt] = cw[jt * D + cl + nt];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int tok = 16 * j + 4 * g + rr;  // window rows tok .. tok + 3, the token itself last
        float x0[NT], x1[NT], x2[NT], x3[NT];
        bf_load<NT>(sv + tok * LDV + cl, x0);
        bf_load<NT>(sv + (tok + 1) * LDV + cl, x1);
        bf_load<NT>(sv + (tok + 2) * LDV + cl, x2);
        bf_load<NT>(sv + (tok + 3) * LDV + cl, x3);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          r[j][rr][nt] = x3[nt] - (wt[0][nt] * x0[nt] + wt[1][nt] * x1[nt] + wt[2][nt] * x2[nt] + wt[3][nt] * x3[nt]);
      }
  }
  bf16_t* gout = reinterpret_cast<bf16_t*>(a.gamma) + (size_t)pr * T * Lm1 * D;
  for (int lv = 0; lv < Lm1; ++lv) {
    // the next level's weights into registers while this level's are used
    const bool more = lv + 1 < Lm1;
    uint4 wn[8];
    if (more) {
      const bf16_t* Wn = Wh + (size_t)(lv + 1) * D * D;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = tid + 64 * NW * q;
        wn[q] = *reinterpret_cast<const uint4*>(Wn + (size_t)(i / PIECES) * D + (i % PIECES) * 8);
      }
    }
    const bf16_t* sw = sW[lv & 1];
    bf16_t fb[TPW][4][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // B operand of output tile nt: row NT li + nt of W_p, so lane (li, g) ends with p for
      // tokens 4 g + rr and the NT adjacent channels NT li ..
      bf16x8 wf[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) wf[kb] = *reinterpret_cast<const bf16x8*>(sw + (cl + nt) * LDW + 32 * kb + 8 * g);
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = mfma(an[j][kb], wf[kb], acc);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float pv = acc[rr];
          fb[j][rr][nt] = (bf16_t)(pv * std_normal_cdf(pv * r[j][rr][nt]));
        }
      }
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int tl = 16 * j + 4 * g + rr, tok = tw + tl;
        const float at = sA[w][tl * L + lv];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) r[j][rr][nt] = r[j][rr][nt] * (1.f - at * (float)fb[j][rr][nt]);
        if (tok < T) bf_store<NT>(gout + ((size_t)tok * Lm1 + lv) * D + cl, fb[j][rr]);
      }
    if (more) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = tid + 64 * NW * q;
        *reinterpret_cast<uint4*>(sW[(lv + 1) & 1] + (i / PIECES) * LDW + (i % PIECES) * 8) = wn[q];
      }
    }
    __syncthreads();
  }
}

}  // namespace prism
