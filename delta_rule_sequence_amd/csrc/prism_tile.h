// prism_tile.h - wave-level 16x16 MFMA tile primitives for gfx950 (CDNA4).
//
// Every product in the chunked forward is built from 16x16 output tiles held
// as MFMA accumulators (f32x4 per lane).  Lane l of a wave holds, for a tile
// X, the elements X[4*(l/16) + r][l%16], r = 0..3 (the MFMA "D" layout).
//
// Two MFMA flavours share one interface:
//   bf16: v_mfma_f32_16x16x32_bf16 - one instruction per 32-deep k block; lane
//         group g = l/16 feeds 8 k values;
//   f32:  v_mfma_f32_16x16x4f32    - four instructions per 16-deep k block; lane
//         group g feeds 1 k value per instruction.
// The k order inside a block is chosen so that an accumulator tile can be fed
// straight back as the B operand of a product that contracts over the tile's
// rows:  bf16 slot p of group g is k = 16*(p/4) + 4*g + p%4 (so slots 0..3
// come from row tile 2i and slots 4..7 from row tile 2i+1), f32 instruction r of
// group g is k = 4*g + r.  Operands read from LDS use the same order.
#pragma once
#include <hip/hip_runtime.h>
#include <type_traits>

namespace prism {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

template <class E> struct Mma;

template <> struct Mma<bf16_t> {
  static constexpr int KB = 32;  // k per block
  // k offset (within a block) of slot p for lane group g
  static __device__ __forceinline__ int koff(int g, int p) { return ((p >> 2) << 4) + (g << 2) + (p & 3); }
};
template <> struct Mma<float> {
  static constexpr int KB = 16;
  static __device__ __forceinline__ int koff(int g, int r) { return (g << 2) + r; }
};

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

template <class E> __device__ __forceinline__ float to_f(E x) { return (float)x; }
template <class E> __device__ __forceinline__ E from_f(float x) { return (E)x; }

// ----------------------------------------------------------------------------
// acc += A[m0:m0+16, 0:K] * B[0:K, n0:n0+16]
// A row-major in LDS with row stride lda (k contiguous);
// B stored as [n][k] in LDS with row stride ldb (k contiguous).
// K is a multiple of 16; for bf16 a trailing half block (K % 32 == 16) is padded
// with zeros.
template <class E>
__device__ __forceinline__ void mm_ll(f32x4& acc, const E* A, int lda, int m0,
                                      const E* B, int ldb, int n0, int K) {
  const int l = lane_id(), g = l >> 4, i = l & 15;
  const E* a = A + (m0 + i) * lda;
  const E* b = B + (n0 + i) * ldb;
  if constexpr (std::is_same<E, bf16_t>::value) {
    for (int k0 = 0; k0 < K; k0 += 32) {
      bf16x8 fa, fb;
      bf16x4 a0 = *reinterpret_cast<const bf16x4*>(a + k0 + 4 * g);
      bf16x4 b0 = *reinterpret_cast<const bf16x4*>(b + k0 + 4 * g);
      bf16x4 a1, b1;
      if (k0 + 16 < K) {
        a1 = *reinterpret_cast<const bf16x4*>(a + k0 + 16 + 4 * g);
        b1 = *reinterpret_cast<const bf16x4*>(b + k0 + 16 + 4 * g);
      } else {
        a1 = bf16x4{0, 0, 0, 0};
        b1 = bf16x4{0, 0, 0, 0};
      }
      fa = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      fb = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
      acc = mfma(fa, fb, acc);
    }
  } else {
    for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mfma(a[k0 + 4 * g + r], b[k0 + 4 * g + r], acc);
    }
  }
}

// acc += A[m0:m0+16, 0:K] * Bt, where Bt is given as accumulator tiles:
// Bt[kt] is the 16x16 tile holding rows 16*kt..16*kt+15 (k) of B and the
// 16 columns of the output.  Each B element is multiplied by bscale[k] (if not
// null) before rounding to E.  A row-major in LDS (k contiguous).
template <class E, int NKT>
__device__ __forceinline__ void mm_lt(f32x4& acc, const E* A, int lda, int m0,
                                      const f32x4 (&Bt)[NKT], const float* bscale, int K) {
  const int l = lane_id(), g = l >> 4, i = l & 15;
  const E* a = A + (m0 + i) * lda;
  if constexpr (std::is_same<E, bf16_t>::value) {
#pragma unroll
    for (int kb = 0; kb < (NKT + 1) / 2; ++kb) {
      const int k0 = kb * 32;
      if (k0 >= K) break;
      bf16x8 fa, fb;
      bf16x4 a0 = *reinterpret_cast<const bf16x4*>(a + k0 + 4 * g);
      bf16x4 a1 = bf16x4{0, 0, 0, 0};
      const bool hi = (2 * kb + 1 < NKT) && (k0 + 16 < K);
      if (hi) a1 = *reinterpret_cast<const bf16x4*>(a + k0 + 16 + 4 * g);
      fa = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float s0 = bscale ? bscale[k0 + 4 * g + p] : 1.f;
        fb[p] = (bf16_t)(Bt[2 * kb][p] * s0);
        if (2 * kb + 1 < NKT) {
          float s1 = (hi && bscale) ? bscale[k0 + 16 + 4 * g + p] : 1.f;
          fb[4 + p] = hi ? (bf16_t)(Bt[2 * kb + 1][p] * s1) : (bf16_t)0.f;
        } else {
          fb[4 + p] = (bf16_t)0.f;
        }
      }
      acc = mfma(fa, fb, acc);
    }
  } else {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const int k0 = kt * 16;
      if (k0 >= K) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = bscale ? bscale[k0 + 4 * g + r] : 1.f;
        acc = mfma(a[k0 + 4 * g + r], Bt[kt][r] * s, acc);
      }
    }
  }
}

// acc += A * Bt with A(m, k) = ascale[k] * S[k * lds + m0 + m]: a scaled transpose of a
// row-major LDS array S whose rows are indexed by k.  bfloat16: the A operand comes from
// gfx950's transposing LDS read (ds_read_b64_tr_b16: in each group of 16 lanes, lane
// 4 r + c supplies row r, columns 4 c .. 4 c + 3 of a 4 x 16 block and lane j receives its
// column j), two reads per 32-deep block; the scale moves onto the B operand's k rows
// (ascale[k] multiplies the same products).  float32: element-wise.
template <class E, int NKT>
__device__ __forceinline__ void mm_tt(f32x4& acc, const E* S, int lds, int m0, const float* ascale,
                                      const f32x4 (&Bt)[NKT], int K) {
  const int l = lane_id(), g = l >> 4, i = l & 15;
  if constexpr (std::is_same<E, bf16_t>::value) {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
    const E* s = S + (i >> 2) * lds + m0 + 4 * (i & 3);
#pragma unroll
    for (int kb = 0; kb < (NKT + 1) / 2; ++kb) {
      const int k0 = kb * 32;
      if (k0 >= K) break;
      const bool hi = (2 * kb + 1 < NKT) && (k0 + 16 < K);
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(const_cast<E*>(s + (k0 + 4 * g) * lds)));
      s16x4_t up = {0, 0, 0, 0};
      if (hi) up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<E*>(s + (k0 + 16 + 4 * g) * lds)));
      const bf16x8 fa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
      bf16x8 fb;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        fb[p] = (bf16_t)(Bt[2 * kb][p] * ascale[k0 + 4 * g + p]);
        fb[4 + p] = hi ? (bf16_t)(Bt[2 * kb + 1][p] * ascale[k0 + 16 + 4 * g + p]) : (bf16_t)0.f;
      }
      acc = mfma(fa, fb, acc);
    }
  } else {
    const E* s = S + m0 + i;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const int k0 = kt * 16;
      if (k0 >= K) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ka = k0 + 4 * g + r;
        acc = mfma(s[ka * lds] * ascale[ka], Bt[kt][r], acc);
      }
    }
  }
}

// acc += A * B with A row-major in LDS (k contiguous) and B(k, n) =
// bscale[k] * S[k * lds + n0 + n] read element-wise from a row-major LDS array.
template <class E>
__device__ __forceinline__ void mm_ls(f32x4& acc, const E* A, int lda, int m0,
                                      const E* S, int lds, int n0, const float* bscale, int K) {
  const int l = lane_id(), g = l >> 4, i = l & 15;
  const E* a = A + (m0 + i) * lda;
  const E* s = S + n0 + i;
  if constexpr (std::is_same<E, bf16_t>::value) {
    for (int k0 = 0; k0 < K; k0 += 32) {
      const bool hi = k0 + 16 < K;
      bf16x8 fa, fb;
      bf16x4 a0 = *reinterpret_cast<const bf16x4*>(a + k0 + 4 * g);
      bf16x4 a1 = bf16x4{0, 0, 0, 0};
      if (hi) a1 = *reinterpret_cast<const bf16x4*>(a + k0 + 16 + 4 * g);
      fa = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int kb0 = k0 + 4 * g + p;
        fb[p] = (bf16_t)(to_f(s[kb0 * lds]) * bscale[kb0]);
        fb[4 + p] = hi ? (bf16_t)(to_f(s[(kb0 + 16) * lds]) * bscale[kb0 + 16]) : (bf16_t)0.f;
      }
      acc = mfma(fa, fb, acc);
    }
  } else {
    for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = k0 + 4 * g + r;
        acc = mfma(a[kk], s[kk * lds] * bscale[kk], acc);
      }
    }
  }
}

}  // namespace prism
