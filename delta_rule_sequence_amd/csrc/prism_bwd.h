// prism_bwd.h - gradients of the PRISM rank-L gated delta-rule forward (gfx950).
//
// The forward, per (b, h) pair with S_0 = 0 (S is dv x dk):
//   anchor_t = sum_j w_j v_{t-3+j};  r_{t,0} = v_t - anchor_t;
//   r_{t,l} = r_{t,l-1} (1 - alpha_{t,l-1} gamma_{t,l-1});  W_{t,l} = alpha_{t,l} r_{t,l}
//   S_t = g_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T + sum_l W_{t,l} u_{t,l}^T
//   o_t = S_t q_t
// (PRISM reading notes, sections 2.1-2.3; Tencent / PKU article, sections 01-四 and 03-三).
// The pages train the layer end to end (their throughput figures are training
// throughput, reading notes section 3.3); this is the reverse-mode derivative of that
// recurrence, token by token, in float32:
//   dS_t += do_t q_t^T;  dq_t = S_t^T do_t;  p = S_{t-1} k_t;  e = dS_t k_t
//   dk_t = dS_t^T (beta v_t - g beta p) - g beta S_{t-1}^T e
//   dv_t = beta e + (1 - w_3) dr_0 + later tokens' anchor terms;  du_{t,l} = dS_t^T W_{t,l}
//   dg_t = <dS_t, S_{t-1}> - beta p.e;  dbeta_t = e.(v_t - g p)
//   dW_{t,l} = dS_t u_{t,l}, then back through the residual chain to alpha, gamma, v, w
//   dS_{t-1} = g (dS_t - beta e k_t^T) = dS_t A_t      (A_t = g (I - beta k k^T) is symmetric)
//
// The rows of S and dS evolve independently (the recurrence acts on the right), so a
// state's D rows are split over NSP workgroups of 256 threads; thread (rb, cb) =
// (tid / 16, tid % 16) of workgroup sp owns rows RW (16 sp + rb) .. + RW - 1 and columns
// cb R .. (R = D / 16).  Sums over a row run through the 16 lanes of the thread's row
// group (DPP butterfly); sums over a column through an LDS table with one slot per token
// of a group of KR tokens, indexed by row block and reduced once per group (two barriers
// per group), then, with NSP > 1, over the workgroups in bwd_part_reduce_kernel.
//
// Two organisations of the same per-token steps:
//   * sequential (bwd_pair_kernel, the low-memory form): one state per pair walks the
//     whole sequence; pass 1 keeps the state entering every block of kBwdBlock tokens,
//     pass 2 walks the blocks backwards, re-runs each block's forward into a scratch and
//     then the adjoint steps of the block in reverse order;
//   * segment-parallel (bwd_seg_*): the sequence is cut into segments of seg_len tokens.
//     Because both recurrences are affine in their carried matrix,
//        S_end = S_in Phi_s + B_s,   Lambda_{s-1} = Lambda_s Phi_s^T + ell_s,
//     with Phi_s = A_{t0} .. A_{t1-1} the segment operator (associativity of the
//     recurrence: reading notes section 2.1; article section 01-二), one parallel pass
//     forms (B_s, Phi_s, ell_s) per segment, two short scans give every segment its
//     entering state S_in and the adjoint Lambda arriving at its last state, and a second
//     parallel pass runs the token steps of every segment from those, exactly as the
//     sequential form does; anchor terms that cross a segment start are added afterwards.
#pragma once
#include "prism_bwd_args.h"
#include "prism_tile.h"

namespace prism {

// One token's inputs as seen by thread (rb, cb): key-side entries of its columns,
// value-side entries of its rows (NR rank slots).
template <int R, int NR, int RW>
struct BwdTok {
  float k[R], q[R], u[NR][R];
  float v[RW], dO[RW], gm[NR][RW], vh[3][RW];  // vh: v_{t-3}, v_{t-2}, v_{t-1}
  float g, beta, al[NR + 1];
};

// The inputs of the adjoint's own recurrence: q, k of the thread's columns, d_o of its rows.
template <int R, int RW>
struct BwdAdjTok {
  float k[R], q[R], dO[RW];
  float g, beta;
};

// Sum over the 16 lanes of a row (DPP butterfly): swap neighbours, swap pairs, mirror
// the halves of each 8 lanes, mirror the row; every lane ends with the row's total.
__device__ __forceinline__ float row16_sum(float x) {
#define PRISM_DPP_ADD(CTRL) x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
  PRISM_DPP_ADD(0xB1)   // quad_perm [1, 0, 3, 2]
  PRISM_DPP_ADD(0x4E)   // quad_perm [2, 3, 0, 1]
  PRISM_DPP_ADD(0x141)  // row_half_mirror
  PRISM_DPP_ADD(0x140)  // row_mirror
#undef PRISM_DPP_ADD
  return x;
}

template <int R>
__device__ __forceinline__ void sum_row_group(float (&x)[R]) {
#pragma unroll
  for (int a = 0; a < R; ++a) x[a] = row16_sum(x[a]);
}

// A thread's RW x R block of a state, stored at RW * R consecutive floats of its own.
template <int RW, int R>
__device__ __forceinline__ void store_block(float* dst, const float (&M)[RW][R]) {
  const int tid = threadIdx.x;
  if constexpr ((RW * R) % 4 == 0) {
#pragma unroll
    for (int e = 0; e < RW * R; e += 4) {
      const float4 x = make_float4(M[e / R][e % R], M[(e + 1) / R][(e + 1) % R], M[(e + 2) / R][(e + 2) % R],
                                   M[(e + 3) / R][(e + 3) % R]);
      *reinterpret_cast<float4*>(dst + (size_t)tid * RW * R + e) = x;
    }
  } else {
#pragma unroll
    for (int e = 0; e < RW * R; ++e) dst[(size_t)tid * RW * R + e] = M[e / R][e % R];
  }
}

template <int RW, int R>
__device__ __forceinline__ void load_block(float (&M)[RW][R], const float* src) {
  const int tid = threadIdx.x;
  if constexpr ((RW * R) % 4 == 0) {
#pragma unroll
    for (int e = 0; e < RW * R; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(src + (size_t)tid * RW * R + e);
      M[e / R][e % R] = x.x;
      M[(e + 1) / R][(e + 1) % R] = x.y;
      M[(e + 2) / R][(e + 2) % R] = x.z;
      M[(e + 3) / R][(e + 3) % R] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < RW * R; ++e) M[e / R][e % R] = src[(size_t)tid * RW * R + e];
  }
}

// A thread's entries (rows row0 .., columns c0 ..) of a row-major D x D matrix.
template <int D, int RW, int R>
__device__ __forceinline__ void store_entries(float* dst, int row0, int c0, const float (&M)[RW][R]) {
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    float* p = dst + (size_t)(row0 + r) * D + c0;
    if constexpr (R % 4 == 0) {
#pragma unroll
      for (int c = 0; c < R; c += 4) *reinterpret_cast<float4*>(p + c) = make_float4(M[r][c], M[r][c + 1], M[r][c + 2], M[r][c + 3]);
    } else {
#pragma unroll
      for (int c = 0; c < R; ++c) p[c] = M[r][c];
    }
  }
}

template <int D, int RW, int R>
__device__ __forceinline__ void load_entries(float (&M)[RW][R], const float* src, int row0, int c0) {
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const float* p = src + (size_t)(row0 + r) * D + c0;
    if constexpr (R % 4 == 0) {
#pragma unroll
      for (int c = 0; c < R; c += 4) {
        const float4 x = *reinterpret_cast<const float4*>(p + c);
        M[r][c] = x.x;
        M[r][c + 1] = x.y;
        M[r][c + 2] = x.z;
        M[r][c + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < R; ++c) M[r][c] = p[c];
    }
  }
}

// Sizes shared by the backward kernels: NR rank slots compiled in, NV column vectors
// (dq, dk, du_l) and NS scalars (dg, dbeta, dalpha_l) per token; a state's rows are split
// over NSP workgroups of 16 RW rows each.
template <int D, int NRK, int RW = 1>
struct BwdShape {
  static constexpr int NR = NRK > 0 ? NRK : 1;
  static constexpr int NV = 2 + NR, NS = 3 + NR;
  static constexpr int RED = NV * D + NS;
  static constexpr int NSP = D / (16 * RW);
  static_assert(NSP >= 1 && NSP * 16 * RW == D, "rows per thread must divide the state");
};

// Writes one of a token's summed column entries / scalars (idx < RED) to its gradient.
template <int D, int NRK>
__device__ __forceinline__ void bwd_write_out(const BwdArgs& a, size_t tr, int idx, float s) {
  using Sh = BwdShape<D, NRK>;
  const int L = a.L, Lm1 = L - 1;
  if (idx < D) {
    a.dq[tr * D + idx] = s;
  } else if (idx < 2 * D) {
    a.dk[tr * D + idx - D] = s;
  } else if (idx < Sh::NV * D) {
    const int l = idx / D - 2, j = idx % D;
    if (l < Lm1) a.du[(tr * Lm1 + l) * D + j] = s;
  } else {
    const int sidx = idx - Sh::NV * D;
    if (sidx == 0) a.dg[tr] = s;
    else if (sidx == 1) a.dbeta[tr] = s;
    else if (sidx - 2 < L && L > 1) a.dalpha[tr * L + sidx - 2] = s;
  }
}

// One input's run of a backward stage, in 16-byte units dealt round-robin to the 256
// threads: unit un covers elements un * vec .. of the run, whose rows of row_elems
// elements start at token tok0; rows outside [0, T) are zero and not read.
template <int N, class E>
__device__ __forceinline__ void stage_fetch_seg(uint4 (&dst)[N], const E* base, int nunits, int vec, int row_elems,
                                                int tok0, int T) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int un = threadIdx.x + 256 * i;
    dst[i] = make_uint4(0u, 0u, 0u, 0u);
    if (un < nunits) {
      const int tok = tok0 + un * vec / row_elems;
      if (tok >= 0 && tok < T) dst[i] = *reinterpret_cast<const uint4*>(base + (size_t)un * vec);
    }
  }
}

template <int N, class E>
__device__ __forceinline__ void stage_commit_seg(E* lds, const uint4 (&src)[N], int nunits, int vec) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int un = threadIdx.x + 256 * i;
    if (un < nunits) *reinterpret_cast<uint4*>(lds + (size_t)un * vec) = src[i];
  }
}

// LDS of the backward: the reduction table holds KR tokens' column sums and scalars per
// row block (reduced once per group of KR tokens), beside two stages of NB tokens' inputs.
template <int D, int NR>
constexpr int bwd_red_slot_bytes() { return 16 * ((2 + NR) * D + 3 + NR) * 4; }
template <class E, int D, int NR>
constexpr int bwd_stage_bytes(int nb) { return (4 * nb + 3 + 2 * nb * NR) * D * (int)sizeof(E) + nb * (3 + NR) * 4; }

// Tokens per reduction group: 4 if that table fits beside two 8-token stages, else 2.
template <class E, int D, int NR>
constexpr int bwd_red_group() {
  return 4 * bwd_red_slot_bytes<D, NR>() + 2 * bwd_stage_bytes<E, D, NR>(8) <= 156 * 1024 ? 4 : 2;
}

// Tokens per LDS stage of the backward's inputs: the largest of 16, 8, 4, 2 whose two
// stage buffers fit beside the reduction table (0: inputs read straight from memory).
template <class E, int D, int NR>
constexpr int bwd_stage_tokens() {
  const int red = bwd_red_group<E, D, NR>() * bwd_red_slot_bytes<D, NR>();
  for (int nb = 16; nb >= 2; nb /= 2)
    if (red + 2 * bwd_stage_bytes<E, D, NR>(nb) <= 156 * 1024) return nb;
  return 0;
}

// The segment-parallel kernels keep their LDS small, so that several workgroups share a
// CU: the reduction table alone, two tokens per group when that stays within 48 KB.
template <int D, int NR>
constexpr int bwd_seg_red_group() { return 2 * bwd_red_slot_bytes<D, NR>() <= 48 * 1024 ? 2 : 1; }

// Rows per thread of the segment-parallel kernels: two from D = 32 up (the per-token
// loads, column-side products and reductions of a thread then serve two rows; measured at
// the 16K workload, d = 64: 7.7 -> 5.5 ms per backward against one row; four rows exceed
// 256 VGPRs), so D / 32 workgroups per state.
template <int D>
constexpr int bwd_seg_rows() { return D >= 32 ? 2 : 1; }

// A thread's view of the backward: its rows and columns, the per-token steps (inputs,
// residual chain, forward step, adjoint step) and the adjoint-side registers they carry.
// NRK: rank slots compiled in (0 for L = 1, 3 for L <= 4, 7 for L <= 8); LX: L - 1 when
// it is known at compile time (it equals NRK), else -1 (the rank loops then test L at run
// time, which splits them into short basic blocks).
template <class E, int D, int NRK, int RW, int KR, int LX = -1>
struct BwdCore {
  using Sh = BwdShape<D, NRK, RW>;
  static constexpr int R = D / 16, NR = Sh::NR, NV = Sh::NV, NS = Sh::NS, RED = Sh::RED, NSP = Sh::NSP;
  static constexpr int SD = D * D / NSP;  // floats of a workgroup's slice of a state
  using Tok = BwdTok<R, NR, RW>;
  using AdjTok = BwdAdjTok<R, RW>;

  const BwdArgs& a;
  float (*red)[16][RED];  // the LDS reduction table, [KR][row block][column sums, scalars]
  int tid, rb, cb, pr, sp, hd, row0, T, L, Lm1;
  const E *Q, *K, *V, *U, *GM, *DO;
  float tw[4][RW];               // conv taps of this thread's rows
  float dS[RW][R], St[RW][R];    // dL/dS_t (carried backwards), S_t
  float pend[3][RW], dw[4][RW];  // anchor terms owed to tokens t-1, t-2, t-3; dconv_w share
  int ng, gfirst;  // tokens written into the reduction table, the group's first (last in time)

  __device__ __forceinline__ BwdCore(const BwdArgs& args, float (*table)[16][RED], int pair, int slice)
      : a(args), red(table) {
    tid = threadIdx.x;
    rb = tid >> 4;
    cb = tid & 15;
    pr = pair;
    sp = slice;
    hd = pair % args.H;
    row0 = RW * (16 * slice + rb);
    T = args.T;
    L = LX >= 0 ? LX + 1 : args.L;
    Lm1 = LX >= 0 ? LX : L - 1;
    Q = reinterpret_cast<const E*>(args.q);
    K = reinterpret_cast<const E*>(args.k);
    V = reinterpret_cast<const E*>(args.v);
    U = reinterpret_cast<const E*>(args.u);
    GM = reinterpret_cast<const E*>(args.gamma);
    DO = reinterpret_cast<const E*>(args.d_o);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        tw[j][r] = L > 1 ? args.conv_w[((size_t)hd * 4 + j) * D + row0 + r] : 0.f;
        dw[j][r] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 3; ++j) pend[j][r] = 0.f;
#pragma unroll
      for (int c = 0; c < R; ++c) {
        dS[r][c] = 0.f;
        St[r][c] = 0.f;
      }
    }
    ng = 0;
    gfirst = 0;
  }

  __device__ __forceinline__ void load_tok(int t, Tok& x) const {
    const size_t tr = (size_t)pr * T + t;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      x.k[c] = (float)K[tr * D + cb * R + c];
      x.q[c] = (float)Q[tr * D + cb * R + c];
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      x.v[r] = (float)V[tr * D + row0 + r];
      x.dO[r] = (float)DO[tr * D + row0 + r];
#pragma unroll
      for (int j = 0; j < 3; ++j) x.vh[j][r] = t - 3 + j >= 0 ? (float)V[(tr - 3 + j) * D + row0 + r] : 0.f;
    }
    x.g = a.g[tr];
    x.beta = a.beta[tr];
#pragma unroll
    for (int l = 0; l < NR; ++l) {
      if (l < Lm1) {
#pragma unroll
        for (int c = 0; c < R; ++c) x.u[l][c] = (float)U[(tr * Lm1 + l) * D + cb * R + c];
#pragma unroll
        for (int r = 0; r < RW; ++r) x.gm[l][r] = (float)GM[(tr * Lm1 + l) * D + row0 + r];
      }
    }
#pragma unroll
    for (int l = 0; l <= NR; ++l) x.al[l] = (L > 1 && l < L) ? a.alpha[tr * L + l] : 0.f;
  }

  __device__ __forceinline__ void load_adj(int t, AdjTok& x) const {
    const size_t tr = (size_t)pr * T + t;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      x.k[c] = (float)K[tr * D + cb * R + c];
      x.q[c] = (float)Q[tr * D + cb * R + c];
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) x.dO[r] = (float)DO[tr * D + row0 + r];
    x.g = a.g[tr];
    x.beta = a.beta[tr];
  }

  // residuals r_{t,0..L-1} and written values W_{t,1..L-1} of this thread's rows
  __device__ __forceinline__ void chain(const Tok& x, float (&rr)[NR + 1][RW], float (&W)[NR][RW]) const {
#pragma unroll
    for (int r = 0; r < RW; ++r)
      rr[0][r] = x.v[r] - (tw[0][r] * x.vh[0][r] + tw[1][r] * x.vh[1][r] + tw[2][r] * x.vh[2][r] + tw[3][r] * x.v[r]);
#pragma unroll
    for (int l = 1; l <= NR; ++l) {
      if (l <= Lm1) {
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          rr[l][r] = rr[l - 1][r] - x.al[l - 1] * x.gm[l - 1][r] * rr[l - 1][r];
          W[l - 1][r] = x.al[l] * rr[l][r];
        }
      }
    }
  }

  // S_t from S_{t-1} (in place)
  __device__ __forceinline__ void fwd_step(float (&M)[RW][R], const Tok& x) const {
    float rr[NR + 1][RW], W[NR][RW];
    chain(x, rr, W);
    float p[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      p[r] = 0.f;
#pragma unroll
      for (int c = 0; c < R; ++c) p[r] += M[r][c] * x.k[c];
    }
    sum_row_group(p);
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < R; ++c) {
        float s = x.g * (M[r][c] - x.beta * p[r] * x.k[c]) + x.beta * x.v[r] * x.k[c];
#pragma unroll
        for (int l = 0; l < NR; ++l)
          if (l < Lm1) s += W[l][r] * x.u[l][c];
        M[r][c] = s;
      }
  }

  // X <- X A_t = g (X - beta (X k) k^T): the step of a carried matrix with no write (the
  // segment operator forwards, the adjoint backwards)
  template <class X>
  __device__ __forceinline__ void transition(float (&M)[RW][R], const X& x) const {
    float p[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      p[r] = 0.f;
#pragma unroll
      for (int c = 0; c < R; ++c) p[r] += M[r][c] * x.k[c];
    }
    sum_row_group(p);
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < R; ++c) M[r][c] = x.g * (M[r][c] - x.beta * p[r] * x.k[c]);
  }

  // the group's column sums and scalars, summed over the row blocks (tokens gfirst,
  // gfirst - 1, ..), to the gradients or, with several workgroups per state, to the partials
  __device__ __forceinline__ void flush() {
    __syncthreads();
    for (int idx = tid; idx < ng * RED; idx += 256) {
      const int gi = idx / RED, e = idx - gi * RED, t = gfirst - gi;
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) s += red[gi][j][e];
      if constexpr (NSP == 1) bwd_write_out<D, NRK>(a, (size_t)pr * T + t, e, s);
      else a.part[(((size_t)pr * NSP + sp) * T + t) * RED + e] = s;
    }
    __syncthreads();
    ng = 0;
  }

  // one adjoint step at token t from its inputs x and the state before it, Mp = S_{t-1};
  // on entry dS holds the adjoint of S_t from the tokens after t and St holds S_t
  __device__ __forceinline__ void rev_step(int t, const Tok& x, const float (&Mp)[RW][R]) {
    const size_t tr = (size_t)pr * T + t;
    float rr[NR + 1][RW], W[NR][RW];
    chain(x, rr, W);
    // dS_t gains the readout's term
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < R; ++c) dS[r][c] += x.dO[r] * x.q[c];
    // row sums: p = S_{t-1} k, e = dS k, dW_l = dS u_l
    float p[RW], e[RW], dW[NR][RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      p[r] = 0.f;
      e[r] = 0.f;
#pragma unroll
      for (int c = 0; c < R; ++c) {
        p[r] += Mp[r][c] * x.k[c];
        e[r] += dS[r][c] * x.k[c];
      }
#pragma unroll
      for (int l = 0; l < NR; ++l) {
        dW[l][r] = 0.f;
        if (l < Lm1) {
#pragma unroll
          for (int c = 0; c < R; ++c) dW[l][r] += dS[r][c] * x.u[l][c];
        }
      }
    }
    sum_row_group(p);
    sum_row_group(e);
#pragma unroll
    for (int l = 0; l < NR; ++l)
      if (l < Lm1) sum_row_group(dW[l]);
    // this thread's share of the column sums and of the scalars
    float y[NV][R], sc[NS];
    const float gb = x.g * x.beta;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      float yq = 0.f, yk = 0.f;
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        yq += St[r][c] * x.dO[r];
        yk += dS[r][c] * (x.beta * x.v[r] - gb * p[r]) - gb * Mp[r][c] * e[r];
      }
      y[0][c] = yq;
      y[1][c] = yk;
#pragma unroll
      for (int l = 0; l < NR; ++l) {
        float yu = 0.f;
        if (l < Lm1) {
#pragma unroll
          for (int r = 0; r < RW; ++r) yu += dS[r][c] * W[l][r];
        }
        y[2 + l][c] = yu;
      }
    }
    float sdg = 0.f;
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < R; ++c) sdg += dS[r][c] * Mp[r][c];
#pragma unroll
    for (int s = 1; s < NS; ++s) sc[s] = 0.f;
    if (cb == 0) {  // per-row terms, counted once per row
      float dr[RW];
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        sdg -= x.beta * e[r] * p[r];
        sc[1] += e[r] * (x.v[r] - x.g * p[r]);
        dr[r] = 0.f;
      }
      // back through W_l = alpha_l r_l and r_l = r_{l-1} (1 - alpha_{l-1} gamma_{l-1})
#pragma unroll
      for (int l = NR; l >= 1; --l) {
        if (l <= Lm1) {
#pragma unroll
          for (int r = 0; r < RW; ++r) {
            dr[r] += x.al[l] * dW[l - 1][r];
            sc[2 + l] += dW[l - 1][r] * rr[l][r];
            a.dgamma[(tr * Lm1 + (l - 1)) * D + row0 + r] = -x.al[l - 1] * rr[l - 1][r] * dr[r];
            sc[2 + l - 1] -= dr[r] * x.gm[l - 1][r] * rr[l - 1][r];
            dr[r] *= 1.f - x.al[l - 1] * x.gm[l - 1][r];
          }
        }
      }
      // dr is now the gradient of r_0 = v_t - anchor_t
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        a.dv[tr * D + row0 + r] = x.beta * e[r] + (1.f - tw[3][r]) * dr[r] + pend[0][r];
        pend[0][r] = pend[1][r] - tw[2][r] * dr[r];
        pend[1][r] = pend[2][r] - tw[1][r] * dr[r];
        pend[2][r] = -tw[0][r] * dr[r];
#pragma unroll
        for (int j = 0; j < 3; ++j) dw[j][r] -= dr[r] * x.vh[j][r];
        dw[3][r] -= dr[r] * x.v[r];
      }
    }
    sc[0] = sdg;
    // column sums and scalars: each row block's share into the group's LDS slot, summed
    // over the 16 row blocks when the group is flushed (the scalars first summed over the
    // row's 16 lanes)
    if (ng == 0) gfirst = t;
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int c = 0; c < R; ++c) red[ng][rb][n * D + cb * R + c] = y[n][c];
    // sc[0] has a share in every lane of the row; the others are per-row terms that only
    // lane cb = 0 formed
    sc[0] = row16_sum(sc[0]);
    if (cb == 0) {
#pragma unroll
      for (int s = 0; s < NS; ++s) red[ng][rb][NV * D + s] = sc[s];
    }
    // dS_{t-1}; S_{t-1} becomes the next step's S_t
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < R; ++c) {
        dS[r][c] = x.g * (dS[r][c] - x.beta * e[r] * x.k[c]);
        St[r][c] = Mp[r][c];
      }
    if (++ng == KR) flush();
  }

  // The adjoint steps of tokens b1 - 1 down to b0, the states S_b0 .. S_{b1-2} read back
  // from scr (S_t at scr + (t - b0) SD) and S_{b0-1} from cp; each thread reads back only
  // what it wrote itself.  St must hold S_{b1-1}.  PIPE: software-pipelined (the next
  // token's inputs and previous state are loaded while the current token is processed,
  // into the other of two register buffers); otherwise one buffer, for kernels that rely
  // on other resident waves to cover the loads.
  template <bool PIPE>
  __device__ __forceinline__ void rev_block(int b0, int b1, const float* scr, const float* cp) {
    auto prev_state = [&](int t) __attribute__((always_inline)) { return t > b0 ? scr + (size_t)(t - 1 - b0) * SD : cp; };
    if constexpr (PIPE) {
      float Ma[RW][R], Mb[RW][R];
      Tok xa, xb;
      load_tok(b1 - 1, xa);
      load_block(Ma, prev_state(b1 - 1));
      for (int t = b1 - 1; t >= b0; t -= 2) {  // tokens t (buffers a) and t - 1 (buffers b)
        if (t - 1 >= b0) {
          load_tok(t - 1, xb);
          load_block(Mb, prev_state(t - 1));
        }
        rev_step(t, xa, Ma);
        if (t - 1 >= b0) {
          if (t - 2 >= b0) {
            load_tok(t - 2, xa);
            load_block(Ma, prev_state(t - 2));
          }
          rev_step(t - 1, xb, Mb);
        }
      }
    } else {
      for (int t = b1 - 1; t >= b0; --t) {
        float Mp[RW][R];
        Tok x;
        load_tok(t, x);
        load_block(Mp, prev_state(t));
        rev_step(t, x, Mp);
      }
    }
    if (ng > 0) flush();
  }

  // The forward over tokens b0 .. b1 - 1 from M, each S_t stored at scr + (t - b0) SD
  // (scr == nullptr: not stored); on return M = S_{b1-1}.  PIPE as for rev_block.
  template <bool PIPE>
  __device__ __forceinline__ void fwd_block(float (&M)[RW][R], int b0, int b1, float* scr) const {
    if constexpr (PIPE) {
      Tok xa, xb;
      load_tok(b0, xa);
      for (int t = b0; t < b1; t += 2) {  // tokens t (buffer a) and t + 1 (buffer b)
        if (t + 1 < b1) load_tok(t + 1, xb);
        fwd_step(M, xa);
        if (scr) store_block(scr + (size_t)(t - b0) * SD, M);
        if (t + 1 < b1) {
          if (t + 2 < b1) load_tok(t + 2, xa);
          fwd_step(M, xb);
          if (scr) store_block(scr + (size_t)(t + 1 - b0) * SD, M);
        }
      }
    } else {
      for (int t = b0; t < b1; ++t) {
        Tok x;
        load_tok(t, x);
        fwd_step(M, x);
        if (scr) store_block(scr + (size_t)(t - b0) * SD, M);
      }
    }
  }
};

// ======================= sequential form (one state per pair) ===========================
// D / 16 workgroups per pair.  Every loop over the token sequence is software-pipelined.
template <class E, int D, int NRK>
__global__ __launch_bounds__(256) void bwd_pair_kernel(BwdArgs a) {
  constexpr int NR = BwdShape<D, NRK>::NR;
  constexpr int KR = bwd_red_group<E, D, NR>();
  using Core = BwdCore<E, D, NRK, 1, KR>;
  using Tok = typename Core::Tok;
  constexpr int R = Core::R, RW = 1, CK = kBwdBlock, RED = Core::RED, NSP = Core::NSP, SD = Core::SD;
  __shared__ float red[KR][16][RED];  // [token of the group][row block][column sums, scalars]
  const int pr = blockIdx.x / NSP, sp = blockIdx.x % NSP;
  Core c(a, red, pr, sp);
  const int tid = c.tid, T = c.T, L = c.L, Lm1 = c.Lm1, row0 = c.row0, cb = c.cb;
  float* ckpt = a.ckpt + ((size_t)pr * NSP + sp) * a.nblk * SD;
  float* scr = a.scratch + ((size_t)pr * NSP + sp) * CK * SD;

  float M[RW][R];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int cc = 0; cc < R; ++cc) {
      M[r][cc] = 0.f;
      c.dS[r][cc] = a.dS_final != nullptr ? a.dS_final[(size_t)pr * D * D + (size_t)(cb * R + cc) * D + row0 + r] : 0.f;
    }
  constexpr int NB = bwd_stage_tokens<E, D, NR>();
  if constexpr (NB > 0) {
    // ---- inputs staged through LDS, NB tokens at a time ---------------------------------
    // A stage holds, for tokens s0 .. s0 + NB - 1, the rows of q, k, d_o, the value rows
    // s0 - 3 .. s0 + NB - 1 (the anchor's window), the rank rows of u and gamma (the
    // layouts of the inputs, so each is one contiguous run), and g, beta, alpha.  Both
    // passes visit the stages in a fixed order; the next stage's loads are issued before
    // the current stage is processed and land in the other buffer after it.
    constexpr int VEC = 16 / (int)sizeof(E);
    constexpr int SE = (4 * NB + 3 + 2 * NB * NR) * D;
    constexpr int SS = NB * (3 + NR);
    __shared__ __align__(16) E stv[2][SE];
    __shared__ float sts[2][SS];
    const int nq = NB * D / VEC, nv = (NB + 3) * D / VEC, nu = NB * Lm1 * D / VEC;
    constexpr int UQ = (NB * D / VEC + 255) / 256, UV = ((NB + 3) * D / VEC + 255) / 256;
    constexpr int UU = (NB * NR * D / VEC + 255) / 256;
    uint4 pq[UQ], pk[UQ], po[UQ], pv[UV], pu[UU], pg[UU];  // the next stage, in flight
    float pres = 0.f;
    // one array per loop (no pointer is chosen at run time)
    auto fetch = [&](int s0) __attribute__((always_inline)) {
      const size_t rw0 = (size_t)pr * T + s0;
      stage_fetch_seg(pq, c.Q + rw0 * D, nq, VEC, D, s0, T);
      stage_fetch_seg(pk, c.K + rw0 * D, nq, VEC, D, s0, T);
      stage_fetch_seg(po, c.DO + rw0 * D, nq, VEC, D, s0, T);
      stage_fetch_seg(pv, c.V + rw0 * D - 3 * D, nv, VEC, D, s0 - 3, T);
      if (Lm1 > 0) {
        stage_fetch_seg(pu, c.U + rw0 * Lm1 * D, nu, VEC, Lm1 * D, s0, T);
        stage_fetch_seg(pg, c.GM + rw0 * Lm1 * D, nu, VEC, Lm1 * D, s0, T);
      }
      // scalars: g, beta (NB each), then alpha (NB x L)
      pres = 0.f;
      if (tid < NB * (2 + (L > 1 ? L : 0))) {
        const int tl = tid < 2 * NB ? tid % NB : (tid - 2 * NB) / L;
        const size_t tr = rw0 + tl;
        if (s0 + tl < T) {
          if (tid < NB) pres = a.g[tr];
          else if (tid < 2 * NB) pres = a.beta[tr];
          else pres = a.alpha[tr * L + (tid - 2 * NB) % L];
        }
      }
    };
    auto commit = [&](int bs) __attribute__((always_inline)) {
      E* b = stv[bs];
      stage_commit_seg(b, pq, nq, VEC);
      stage_commit_seg(b + NB * D, pk, nq, VEC);
      stage_commit_seg(b + 2 * NB * D, po, nq, VEC);
      stage_commit_seg(b + 3 * NB * D, pv, nv, VEC);
      if (Lm1 > 0) {
        stage_commit_seg(b + (4 * NB + 3) * D, pu, nu, VEC);
        stage_commit_seg(b + (4 * NB + 3) * D + NB * Lm1 * D, pg, nu, VEC);
      }
      if (tid < SS) sts[bs][tid] = pres;
    };
    const int oU = (4 * NB + 3) * D, oG = oU + NB * Lm1 * D;
    auto load_tok_s = [&](int bs, int tl, Tok& x) __attribute__((always_inline)) {
      const E* b = stv[bs];
#pragma unroll
      for (int cc = 0; cc < R; ++cc) {
        x.q[cc] = (float)b[tl * D + cb * R + cc];
        x.k[cc] = (float)b[(NB + tl) * D + cb * R + cc];
      }
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        x.dO[r] = (float)b[(2 * NB + tl) * D + row0 + r];
        x.v[r] = (float)b[(3 * NB + tl + 3) * D + row0 + r];
#pragma unroll
        for (int j = 0; j < 3; ++j) x.vh[j][r] = (float)b[(3 * NB + tl + j) * D + row0 + r];
      }
#pragma unroll
      for (int l = 0; l < NR; ++l) {
        if (l < Lm1) {
#pragma unroll
          for (int cc = 0; cc < R; ++cc) x.u[l][cc] = (float)b[oU + (tl * Lm1 + l) * D + cb * R + cc];
#pragma unroll
          for (int r = 0; r < RW; ++r) x.gm[l][r] = (float)b[oG + (tl * Lm1 + l) * D + row0 + r];
        }
      }
      x.g = sts[bs][tl];
      x.beta = sts[bs][NB + tl];
#pragma unroll
      for (int l = 0; l <= NR; ++l) x.al[l] = (L > 1 && l < L) ? sts[bs][2 * NB + tl * L + l] : 0.f;
    };

    // ---- pass 1: the forward, keeping the state entering every block -------------------
    const int nst = (T + NB - 1) / NB;
    int cur = 0;
    fetch(0);
    commit(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      const int s0 = st * NB;
      if (st + 1 < nst) fetch(s0 + NB);
      for (int t = s0; t < min(T, s0 + NB); ++t) {
        if (t % CK == 0) store_block(ckpt + (size_t)(t / CK) * SD, M);
        Tok x;
        load_tok_s(cur, t - s0, x);
        c.fwd_step(M, x);
      }
      if (st + 1 < nst) commit(cur ^ 1);
      __syncthreads();
      cur ^= 1;
    }

    // ---- pass 2: per block (last first) its stages ascending (the block's forward again,
    // keeping every S_t), then descending (the adjoint steps, last token first) -------------
    int blk = a.nblk - 1, j = 0;
    bool rev = false;
    auto nstb = [&](int b) __attribute__((always_inline)) { return (min(T, b * CK + CK) - b * CK + NB - 1) / NB; };
    fetch(blk * CK);
    commit(cur);
    __syncthreads();
    float Ma[RW][R], Mb[RW][R];
    while (blk >= 0) {
      const int t0 = blk * CK, t1 = min(T, t0 + CK), s0 = t0 + j * NB, s1 = min(t1, s0 + NB);
      // the visit after this one
      int nb_ = blk, nj = j;
      bool nrev = rev;
      if (!rev) {
        if (j + 1 < nstb(blk)) nj = j + 1;
        else nrev = true;
      } else {
        if (j > 0) nj = j - 1;
        else { nb_ = blk - 1; nj = 0; nrev = false; }
      }
      const bool more = nb_ >= 0;
      if (more) fetch(nb_ * CK + nj * NB);
      if (!rev) {
        if (j == 0) load_block(M, ckpt + (size_t)blk * SD);
        for (int t = s0; t < s1; ++t) {
          Tok x;
          load_tok_s(cur, t - s0, x);
          c.fwd_step(M, x);
          store_block(scr + (size_t)(t - t0) * SD, M);
        }
        if (s1 == t1) {
#pragma unroll
          for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int cc = 0; cc < R; ++cc) c.St[r][cc] = M[r][cc];
        }
      } else {
        const float* cp = ckpt + (size_t)blk * SD;
        auto prev_state = [&](int t) __attribute__((always_inline)) { return t > t0 ? scr + (size_t)(t - 1 - t0) * SD : cp; };
        load_block(Ma, prev_state(s1 - 1));
        for (int t = s1 - 1; t >= s0; t -= 2) {  // tokens t (Ma) and t - 1 (Mb)
          if (t - 1 >= s0) load_block(Mb, prev_state(t - 1));
          Tok x;
          load_tok_s(cur, t - s0, x);
          c.rev_step(t, x, Ma);
          if (t - 1 >= s0) {
            if (t - 2 >= s0) load_block(Ma, prev_state(t - 2));
            Tok y;
            load_tok_s(cur, t - 1 - s0, y);
            c.rev_step(t - 1, y, Mb);
          }
        }
        if (c.ng > 0) c.flush();
      }
      if (more) commit(cur ^ 1);
      __syncthreads();
      cur ^= 1;
      blk = nb_;
      j = nj;
      rev = nrev;
    }
  } else {
    // ---- inputs read straight from memory (shapes whose stages do not fit in LDS) ------
    // ---- pass 1: the forward, keeping the state entering every block -------------------
    for (int blk = 0; blk < a.nblk; ++blk) {
      store_block(ckpt + (size_t)blk * SD, M);
      if (blk + 1 < a.nblk) c.template fwd_block<true>(M, blk * CK, blk * CK + CK, nullptr);
    }
    // ---- pass 2: blocks in reverse: the block's forward again, keeping every S_t, then
    // the adjoint steps, last token first ---------------------------------------------------
    for (int blk = a.nblk - 1; blk >= 0; --blk) {
      const int t0 = blk * CK, t1 = min(T, t0 + CK);
      const float* cp = ckpt + (size_t)blk * SD;
      load_block(M, cp);
      c.template fwd_block<true>(M, t0, t1, scr);
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int cc = 0; cc < R; ++cc) c.St[r][cc] = M[r][cc];
      c.template rev_block<true>(t0, t1, scr, cp);
    }
  }
  if (cb == 0 && L > 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < RW; ++r) a.dconv_part[((size_t)pr * 4 + j) * D + row0 + r] = c.dw[j][r];
  }
}

// ======================= segment-parallel form ==========================================
// Workgroup wg of a segment launch: slice wg % NSP of segment (wg / NSP) % nseg of pair
// wg / (NSP nseg).

// Pass 1: per segment, from a zero state, the state at its end (B_s), the segment operator
// Phi_s = A_{t0} .. A_{t1-1} (its rows evolve like the state's, with no write), and,
// walking the segment backwards with a zero adjoint at its end, the adjoint ell_s at its
// start (dS += d_o q^T, then dS <- dS A_t).  Only row sums are needed: no LDS.
template <class E, int D, int NRK, int RW, int LX>
__global__ __launch_bounds__(256) void bwd_seg_local_kernel(BwdArgs a) {
  using Core = BwdCore<E, D, NRK, RW, 1, LX>;
  using Tok = typename Core::Tok;
  using AdjTok = typename Core::AdjTok;
  constexpr int R = Core::R, NSP = Core::NSP;
  const int wg = blockIdx.x, sp = wg % NSP, seg = (wg / NSP) % a.nseg, pr = wg / (NSP * a.nseg);
  Core c(a, nullptr, pr, sp);
  const int t0 = seg * a.seg_len, t1 = min(c.T, t0 + a.seg_len), c0 = c.cb * R;
  const size_t so = ((size_t)pr * a.nseg + seg) * D * D;
  float M[RW][R], F[RW][R];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int cc = 0; cc < R; ++cc) {
      M[r][cc] = 0.f;
      F[r][cc] = c.row0 + r == c0 + cc ? 1.f : 0.f;
    }
  {
    Tok xa, xb;
    c.load_tok(t0, xa);
    for (int t = t0; t < t1; t += 2) {  // tokens t (buffer a) and t + 1 (buffer b)
      if (t + 1 < t1) c.load_tok(t + 1, xb);
      c.transition(F, xa);
      c.fwd_step(M, xa);
      if (t + 1 < t1) {
        if (t + 2 < t1) c.load_tok(t + 2, xa);
        c.transition(F, xb);
        c.fwd_step(M, xb);
      }
    }
  }
  store_entries<D>(a.seg_B + so, c.row0, c0, M);
  store_entries<D>(a.seg_Phi + so, c.row0, c0, F);
  // the local adjoint (M reused as dS)
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int cc = 0; cc < R; ++cc) M[r][cc] = 0.f;
  AdjTok ya, yb;
  auto adj = [&](const AdjTok& y) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int cc = 0; cc < R; ++cc) M[r][cc] += y.dO[r] * y.q[cc];
    c.transition(M, y);
  };
  c.load_adj(t1 - 1, ya);
  for (int t = t1 - 1; t >= t0; t -= 2) {  // tokens t (buffer a) and t - 1 (buffer b)
    if (t - 1 >= t0) c.load_adj(t - 1, yb);
    adj(ya);
    if (t - 1 >= t0) {
      if (t - 2 >= t0) c.load_adj(t - 2, ya);
      adj(yb);
    }
  }
  store_entries<D>(a.seg_ell + so, c.row0, c0, M);
}

// Pass 2: the two scans over a pair's segments, on rows r0 .. r0 + 3 of the carried matrix
// (blockIdx.y), forwards (blockIdx.z = 0):
//     S_in(0) = 0,  S_in(s + 1) = S_in(s) Phi_s + B_s
// and backwards (blockIdx.z = 1):
//     Lambda_{nseg-1} = dS_final (in S layout; zero if absent),  Lambda_{s-1} = Lambda_s Phi_s^T + ell_s.
// Thread (j, ks) forms the partial products of output column j over the contraction slice
// ks KD .. with its slice of Phi_s in registers; the KS partials meet in LDS.  The operator
// slice and the added term of the next step are loaded while the current step runs, so a
// step waits on no memory.  Two barriers per step.
template <int D>
__global__ __launch_bounds__(256) void bwd_seg_scan_kernel(BwdArgs a) {
  constexpr int NROW = 4, KS = 256 / D, KD = D / KS, NE = (NROW * D + 255) / 256;
  __shared__ float sx[NROW][D];
  __shared__ float spart[KS][NROW][D];
  const int tid = threadIdx.x, j = tid % D, ks = tid / D;
  const int pr = blockIdx.x, r0 = NROW * blockIdx.y;
  const bool rev = blockIdx.z == 1;
  const int nseg = a.nseg;
  const size_t DD = (size_t)D * D, base = (size_t)pr * nseg * DD;
  float* out = rev ? a.seg_Lam : a.seg_Sin;
  const float* add = rev ? a.seg_ell : a.seg_B;
  for (int e = tid; e < NROW * D; e += 256) {
    const int r = e / D, jj = e % D;
    sx[r][jj] = rev && a.dS_final != nullptr ? a.dS_final[(size_t)pr * DD + (size_t)jj * D + r0 + r] : 0.f;
  }
  float ph[2][KD], ad[2][NE];
  // step i's operator slice and added entries (element e = tid + 256 n of the 4 x D rows)
  auto fetch = [&](int i, float (&dst)[KD], float (&da)[NE]) __attribute__((always_inline)) {
    const int s = rev ? nseg - 1 - i : i;
    const float* P = a.seg_Phi + base + (size_t)s * DD;
#pragma unroll
    for (int m = 0; m < KD; ++m) {
      const int k = ks * KD + m;
      dst[m] = rev ? P[(size_t)j * D + k] : P[(size_t)k * D + j];
    }
#pragma unroll
    for (int n = 0; n < NE; ++n) {
      const int e = tid + 256 * n;
      da[n] = e < NROW * D ? add[base + (size_t)s * DD + (size_t)(r0 + e / D) * D + e % D] : 0.f;
    }
  };
  // the carried rows of step i, stored where the step's segment reads them
  auto put = [&](int i) __attribute__((always_inline)) {
    const int s = rev ? nseg - 1 - i : i;
#pragma unroll
    for (int n = 0; n < NE; ++n) {
      const int e = tid + 256 * n;
      if (e < NROW * D) out[base + (size_t)s * DD + (size_t)(r0 + e / D) * D + e % D] = sx[e / D][e % D];
    }
  };
  // step i: x <- x Phi' + added term; then the new rows are stored for step i + 1
  auto step = [&](int i, const float (&phi)[KD], const float (&da)[NE]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < NROW; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < KD; ++m) acc += sx[r][ks * KD + m] * phi[m];
      spart[ks][r][j] = acc;
    }
    __syncthreads();
    const int sn = rev ? nseg - 2 - i : i + 1;  // the segment the new rows enter
#pragma unroll
    for (int n = 0; n < NE; ++n) {
      const int e = tid + 256 * n;
      if (e < NROW * D) {
        const int r = e / D, jj = e % D;
        float v = da[n];
#pragma unroll
        for (int q = 0; q < KS; ++q) v += spart[q][r][jj];
        sx[r][jj] = v;
        if (i + 1 < nseg) out[base + (size_t)sn * DD + (size_t)(r0 + r) * D + jj] = v;
      }
    }
    __syncthreads();
  };
  __syncthreads();
  if (nseg > 0) {
    put(0);
    // operands loaded a step ahead, unconditionally (the index clamps at the last
    // segment), so the loop body is straight-line code and no step waits on a load issued
    // after its own operands
    fetch(0, ph[0], ad[0]);
    int i = 0;
    for (; i + 2 <= nseg; i += 2) {
      fetch(min(i + 1, nseg - 1), ph[1], ad[1]);
      step(i, ph[0], ad[0]);
      fetch(min(i + 2, nseg - 1), ph[0], ad[0]);
      step(i + 1, ph[1], ad[1]);
    }
    if (i < nseg) step(i, ph[0], ad[0]);
  }
}

// Pass 3: the token steps of every segment, from its entering state S_in and the adjoint
// Lambda of its last state: a forward over the segment keeping the state every kBwdSegSub
// tokens, then per sub-block (last first) the sub-block's forward again into a per-workgroup
// scratch and its adjoint steps.  The anchor terms the segment owes the three tokens before
// it, and its dconv_w share, go to the workspace.
template <class E, int D, int NRK, int RW, int LX>
__global__ __launch_bounds__(256) void bwd_seg_kernel(BwdArgs a) {
  constexpr int NR = BwdShape<D, NRK, RW>::NR;
  constexpr int KR = bwd_seg_red_group<D, NR>();
  using Core = BwdCore<E, D, NRK, RW, KR, LX>;
  constexpr int R = Core::R, NSP = Core::NSP, SD = Core::SD, RED = Core::RED, CK = kBwdSegSub;
  __shared__ float red[KR][16][RED];
  const int wg = blockIdx.x, sp = wg % NSP, seg = (wg / NSP) % a.nseg, pr = wg / (NSP * a.nseg);
  Core c(a, red, pr, sp);
  const int t0 = seg * a.seg_len, t1 = min(c.T, t0 + a.seg_len), c0 = c.cb * R;
  const int nsub = (t1 - t0 + CK - 1) / CK;
  float* ckpt = a.ckpt + (size_t)wg * (a.seg_len / CK) * SD;
  float* scr = a.scratch + (size_t)wg * CK * SD;
  const size_t so = ((size_t)pr * a.nseg + seg) * D * D;
  float M[RW][R];
  load_entries<D>(M, a.seg_Sin + so, c.row0, c0);
  load_entries<D>(c.dS, a.seg_Lam + so, c.row0, c0);
  // the states entering sub-blocks 0 .. nsub - 1
  for (int b = 0; b < nsub; ++b) {
    store_block(ckpt + (size_t)b * SD, M);
    if (b + 1 < nsub) c.template fwd_block<false>(M, t0 + b * CK, t0 + b * CK + CK, nullptr);
  }
  for (int b = nsub - 1; b >= 0; --b) {
    const int b0 = t0 + b * CK, b1 = min(t1, b0 + CK);
    const float* cp = ckpt + (size_t)b * SD;
    load_block(M, cp);
    c.template fwd_block<false>(M, b0, b1, scr);
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int cc = 0; cc < R; ++cc) c.St[r][cc] = M[r][cc];
    c.template rev_block<false>(b0, b1, scr, cp);
  }
  if (c.cb == 0 && c.L > 1) {
    const size_t ps = (size_t)pr * a.nseg + seg;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
#pragma unroll
      for (int j = 0; j < 3; ++j) a.carry[(ps * 3 + j) * D + c.row0 + r] = c.pend[j][r];
#pragma unroll
      for (int j = 0; j < 4; ++j) a.dconv_part[(ps * 4 + j) * D + c.row0 + r] = c.dw[j][r];
    }
  }
}

// Pass 4: the anchor terms that cross a segment start: segment s (s >= 1) owes tokens
// t0 - 1, t0 - 2, t0 - 3 (all in earlier segments, which are at least 16 tokens long).
__global__ __launch_bounds__(256) void bwd_seg_carry_kernel(BwdArgs a, int D) {
  const int pr = blockIdx.x / a.nseg, seg = blockIdx.x % a.nseg;
  if (seg == 0) return;
  const int t0 = seg * a.seg_len;
  const size_t ps = (size_t)pr * a.nseg + seg;
  for (int e = threadIdx.x; e < 3 * D; e += 256) {
    const int j = e / D, i = e % D, t = t0 - 1 - j;
    a.dv[((size_t)pr * a.T + t) * D + i] += a.carry[(ps * 3 + j) * D + i];
  }
}

// Column sums and scalars of a state whose rows were split over NSP workgroups: the
// partials added in a fixed order (deterministic); 8 tokens per workgroup.
template <int D, int NRK, int RW>
__global__ __launch_bounds__(256) void bwd_part_reduce_kernel(BwdArgs a) {
  using Sh = BwdShape<D, NRK, RW>;
  const int T = a.T, nt8 = (T + 7) / 8;
  const int pr = blockIdx.x / nt8, t8 = blockIdx.x % nt8;
  for (int tl = 0; tl < 8; ++tl) {
    const int t = t8 * 8 + tl;
    if (t >= T) break;
    for (int idx = threadIdx.x; idx < Sh::RED; idx += 256) {
      float s = 0.f;
      for (int sp = 0; sp < Sh::NSP; ++sp) s += a.part[(((size_t)pr * Sh::NSP + sp) * T + t) * Sh::RED + idx];
      bwd_write_out<D, NRK>(a, (size_t)pr * T + t, idx, s);
    }
  }
}

// dconv_w[h] = sum over the batch and the nseg shares of each pair, shares laid out
// [B][H][nseg][4][D]: workgroup (h, block of 64 entries); thread (entry, quarter) sums every
// fourth share in order, then the four quarter sums are added in order (deterministic).
__global__ __launch_bounds__(256) void bwd_conv_reduce_kernel(const float* part, float* dconv_w, int B, int H, int D,
                                                              int nseg) {
  __shared__ float q4[4][64];
  const int h = blockIdx.x, i = 64 * blockIdx.y + (threadIdx.x & 63), qt = threadIdx.x >> 6;
  const int n = B * nseg;
  float s = 0.f;
  if (i < 4 * D) {
    for (int x = qt; x < n; x += 4) {
      const int b = x / nseg, sg = x % nseg;
      s += part[(((size_t)b * H + h) * nseg + sg) * 4 * D + i];
    }
  }
  q4[qt][threadIdx.x & 63] = s;
  __syncthreads();
  if (qt == 0 && i < 4 * D)
    dconv_w[(size_t)h * 4 * D + i] = (q4[0][threadIdx.x] + q4[1][threadIdx.x]) + (q4[2][threadIdx.x] + q4[3][threadIdx.x]);
}

}  // namespace prism
