// prism_decode.h - streaming pieces of the PRISM forward (gfx950):
//
//   conv_tail_kernel : the ShortConv window a continuation needs - the values of the last
//                      three tokens of [history; v] - written after a forward call;
//   decode_kernel    : one token for every (b, h) pair, updating the state and the window
//                      in place, for token-by-token generation or serving.
//
// The fixed-size state is all the linear recurrence carries from one token to the next
// (Tencent Ads article, section 01-二; "PRISM" reading notes, section 2.1), and the anchor
// only looks three tokens back (notes, section 2.3), so (state, window) resumes a sequence
// exactly.  The decode step is memory-bound: it reads and writes the dk x dv float32
// state once (2 x 16 KB per pair at d = 64) and touches a few vectors.
#pragma once
#include "prism_kernels.h"

namespace prism {

// conv_out[pr][r][:] = row T - 3 + r of [conv_in (or zeros); v] for pair pr.  Each thread
// reads its column's three rows before writing them, so conv_out may alias conv_in.
template <class E>
__global__ __launch_bounds__(128) void conv_tail_kernel(FwdArgs a, int dv) {
  const int pr = blockIdx.x;
  const E* v = reinterpret_cast<const E*>(a.v) + (size_t)pr * a.T * dv;
  const E* h = a.conv_in != nullptr ? reinterpret_cast<const E*>(a.conv_in) + (size_t)pr * 3 * dv : nullptr;
  E* out = reinterpret_cast<E*>(a.conv_out) + (size_t)pr * 3 * dv;
  for (int col = threadIdx.x; col < dv; col += blockDim.x) {
    E x[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int src = a.T - 3 + r;
      x[r] = src >= 0 ? v[(size_t)src * dv + col] : (h != nullptr ? h[(src + 3) * dv + col] : from_f<E>(0.f));
    }
#pragma unroll
    for (int r = 0; r < 3; ++r) out[r * dv + col] = x[r];
  }
}

struct DecodeArgs {
  const void* q;       // [P][dk]
  const void* k;       // [P][dk]
  const void* v;       // [P][dv]
  const float* g;      // [P]
  const float* beta;   // [P]
  const void* u;       // [P][L-1][dk]
  const float* alpha;  // [P][L]
  const void* gamma;   // [P][L-1][dv]
  const float* conv_w; // [H][4][dv]
  float* S;            // [P][dk][dv] in / out (the S_final layout, H = S^T)
  void* conv_state;    // [P][3][dv] in / out, or null (L == 1)
  void* o;             // [P][dv]
  int H, L;
};

// One workgroup of 256 threads per (b, h) pair.  Thread (rg, j) = (tid / D, tid % D) owns
// column j of H = S^T over the rows rg * RPT .. rg * RPT + RPT - 1, with the RG row groups'
// partial sums of k^T H and q^T H' combined through LDS.
//   H' = g (H - beta k (k^T H)) + beta k v^T + sum_l u_l W_l^T,  o = H'^T q,
// W_l = alpha_l r_l from the anchor and the residual chain of the token.
template <class E, int D>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int RG = 256 / D;   // row groups
  constexpr int RPT = D / RG;   // rows per thread
  __shared__ float sk[D], sq[D], sv[D], su[7][D], sw[7][D], sx[RG][D], so[RG][D];
  const int pr = blockIdx.x, tid = threadIdx.x, j = tid % D, rg = tid / D;
  const int L = a.L, hd = pr % a.H;
  const E* q = reinterpret_cast<const E*>(a.q) + (size_t)pr * D;
  const E* k = reinterpret_cast<const E*>(a.k) + (size_t)pr * D;
  const E* v = reinterpret_cast<const E*>(a.v) + (size_t)pr * D;
  for (int i = tid; i < D; i += 256) {
    sq[i] = to_f(q[i]);
    sk[i] = to_f(k[i]);
    sv[i] = to_f(v[i]);
  }
  if (L > 1) {
    const E* u = reinterpret_cast<const E*>(a.u) + (size_t)pr * (L - 1) * D;
    for (int i = tid; i < (L - 1) * D; i += 256) su[i / D][i % D] = to_f(u[i]);
  }
  if (tid < D) {
    // the value window (t-3, t-2, t-1, t); the residual chain; the window moves on by one
    E* cs = a.conv_state != nullptr ? reinterpret_cast<E*>(a.conv_state) + (size_t)pr * 3 * D : nullptr;
    const float h0 = cs != nullptr ? to_f(cs[j]) : 0.f;
    const float h1 = cs != nullptr ? to_f(cs[D + j]) : 0.f;
    const float h2 = cs != nullptr ? to_f(cs[2 * D + j]) : 0.f;
    const float vj = to_f(v[j]);
    if (L > 1) {
      const float* w = a.conv_w + (size_t)hd * 4 * D;
      float r = vj - (w[j] * h0 + w[D + j] * h1 + w[2 * D + j] * h2 + w[3 * D + j] * vj);
      const float* al = a.alpha + (size_t)pr * L;
      const E* ga = reinterpret_cast<const E*>(a.gamma) + (size_t)pr * (L - 1) * D;
      for (int l = 1; l < L; ++l) {
        r = r * (1.f - al[l - 1] * to_f(ga[(l - 1) * D + j]));
        sw[l - 1][j] = al[l] * r;
      }
    }
    if (cs != nullptr) {
      cs[j] = from_f<E>(h1);
      cs[D + j] = from_f<E>(h2);
      cs[2 * D + j] = v[j];
    }
  }
  float* S = a.S + (size_t)pr * D * D;
  float hv[RPT];
  __syncthreads();
  float x = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    hv[i] = S[(size_t)row * D + j];
    x += sk[row] * hv[i];
  }
  sx[rg][j] = x;
  __syncthreads();
  float kh = 0.f;
#pragma unroll
  for (int r = 0; r < RG; ++r) kh += sx[r][j];
  const float g = a.g[pr], be = a.beta[pr];
  float oacc = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    float hn = g * (hv[i] - be * sk[row] * kh) + be * sk[row] * sv[j];
    for (int l = 1; l < L; ++l) hn += su[l - 1][row] * sw[l - 1][j];
    S[(size_t)row * D + j] = hn;
    oacc += sq[row] * hn;
  }
  so[rg][j] = oacc;
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) o += so[r][tid];
    reinterpret_cast<E*>(a.o)[(size_t)pr * D + tid] = from_f<E>(o);
  }
}

}  // namespace prism
