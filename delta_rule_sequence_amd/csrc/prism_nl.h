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
// evaluated on the chain's own residuals.  This kernel walks the chain once per token and
// channel and writes those factors; the linear forward (any of its entry points) run with
// them is the nonlinear forward.  Each factor is rounded to the I/O type before the chain
// moves on with it, exactly as the forward's chain will use it, so both evaluate the same
// residuals.
//
// Work: one thread per (pair, token, 4 value channels), element-wise and HBM-bound: per
// token-head it reads v (and the three earlier rows, from cache), L - 1 gain rows and L
// step sizes, and writes L - 1 factor rows.
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

// grid (ceil(T * dv / 4 / 256), P): 32-bit indexing inside a pair, no division
template <class E>
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
  const float* al = a.alpha + (size_t)pt * L;
  const E* pg = reinterpret_cast<const E*>(a.p) + (size_t)pt * Lm1 * dv + c4;
  E* gm = reinterpret_cast<E*>(a.gamma) + (size_t)pt * Lm1 * dv + c4;
  for (int l = 0; l < Lm1; ++l) {
    const float4 pv = Vec4<E>::load(pg + (size_t)l * dv);
    const float at = al[l];
    float f[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float pc = f4get(pv, c);
      f[c] = pc * std_normal_cdf(pc * r[c]);
    }
    Vec4<E>::store(gm + (size_t)l * dv, make_float4(f[0], f[1], f[2], f[3]));
    // move on with the stored (rounded) factor, as the forward's chain will
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = r[c] * (1.f - at * to_f(from_f<E>(f[c])));
  }
}

}  // namespace prism
