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
//   dS_{t-1} = g (dS_t - beta e k_t^T)
//
// The rows of S and dS evolve independently (the recurrence acts on the right), so a
// pair's D rows are split over D / 16 workgroups of 256 threads; thread (rb, cb) =
// (tid / 16, tid % 16) of workgroup sp owns row 16 sp + rb and columns cb R .. (R = D / 16).
// Sums over a row run through the 16 lanes of the thread's row group (DPP butterfly); sums
// over a column through an LDS table with one slot per token of a group of KR tokens,
// indexed by row block and reduced once per group (two barriers per group), then over the
// workgroups of the pair in bwd_part_reduce_kernel.  Pass 1 runs the forward and keeps the state
// entering every block of kBwdBlock tokens; pass 2 walks the blocks backwards, re-runs
// each block's forward into a per-pair scratch (every thread reads back only what it
// wrote itself) and then the adjoint steps of the block in reverse order.
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

// Sizes shared by the backward kernels: NR rank slots compiled in, NV column vectors
// (dq, dk, du_l) and NS scalars (dg, dbeta, dalpha_l) per token; a pair's state rows are
// split over NSP workgroups of 16 rows each.
template <int D, int NRK>
struct BwdShape {
  static constexpr int NR = NRK > 0 ? NRK : 1;
  static constexpr int NV = 2 + NR, NS = 3 + NR;
  static constexpr int RED = NV * D + NS;
  static constexpr int NSP = D / 16;
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

// NRK: rank slots compiled in (0 for L = 1, 3 for L <= 4, 7 for L <= 8).  Every loop
// over the token sequence is software-pipelined: the next token's inputs (and, in the
// adjoint, its previous state) are loaded while the current token is processed, into
// the other of two register buffers.
template <class E, int D, int NRK>
__global__ __launch_bounds__(256) void bwd_pair_kernel(BwdArgs a) {
  using Sh = BwdShape<D, NRK>;
  constexpr int R = D / 16, RW = 1, CK = kBwdBlock, NR = Sh::NR, NV = Sh::NV, NS = Sh::NS, RED = Sh::RED;
  constexpr int NSP = Sh::NSP, SD = D * D / NSP;  // workgroups per pair, floats of a state slice
  using Tok = BwdTok<R, NR, RW>;
  constexpr int KR = bwd_red_group<E, D, NR>();
  __shared__ float red[KR][16][RED];  // [token of the group][row block][column sums, scalars]
  const int tid = threadIdx.x;
  const int rb = tid >> 4, cb = tid & 15;
  const int pr = blockIdx.x / NSP, sp = blockIdx.x % NSP, hd = pr % a.H;
  const int row0 = 16 * sp + rb;  // this thread's state row
  const int T = a.T, L = a.L, Lm1 = L - 1;
  const E* Q = reinterpret_cast<const E*>(a.q);
  const E* K = reinterpret_cast<const E*>(a.k);
  const E* V = reinterpret_cast<const E*>(a.v);
  const E* U = reinterpret_cast<const E*>(a.u);
  const E* GM = reinterpret_cast<const E*>(a.gamma);
  const E* DO = reinterpret_cast<const E*>(a.d_o);
  const float *Gg = a.g, *Gb = a.beta, *Ga = a.alpha;
  float* ckpt = a.ckpt + ((size_t)pr * NSP + sp) * (a.all_states ? T : a.nblk) * SD;
  float* scr = a.scratch + ((size_t)pr * NSP + sp) * CK * SD;

  float tw[4][RW];  // conv taps of this thread's rows
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < RW; ++r) tw[j][r] = L > 1 ? a.conv_w[((size_t)hd * 4 + j) * D + row0 + r] : 0.f;

  auto load_tok = [&](int t, Tok& x) __attribute__((always_inline)) {
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
  };
  // residuals r_{t,0..L-1} and written values W_{t,1..L-1} of this thread's rows
  auto chain = [&](const Tok& x, float (&rr)[NR + 1][RW], float (&W)[NR][RW]) __attribute__((always_inline)) {
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
  };
  // S_t from S_{t-1} (in place)
  auto fwd_step = [&](float (&M)[RW][R], const Tok& x) __attribute__((always_inline)) {
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
  };

  float dS[RW][R], St[RW][R];                   // dL/dS_t (carried backwards), S_t
  float pend[3][RW], dw[4][RW];                 // anchor terms owed to tokens t, t-1, t-2; dconv_w share
  int ng = 0, gfirst = 0;  // tokens written into the reduction table, the group's first (last in time)
  // one adjoint step at token t from its inputs x and the state before it, Mp = S_{t-1}
  // the group's column sums and scalars, summed over the row blocks (tokens gfirst,
  // gfirst - 1, ..), to the gradients or, with several workgroups per pair, to the partials
  auto flush = [&]() __attribute__((always_inline)) {
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
  };
  auto rev_step = [&](int t, const Tok& x, const float (&Mp)[RW][R]) __attribute__((always_inline)) {
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
#pragma unroll
    for (int s = 0; s < NS; ++s) sc[s] = row16_sum(sc[s]);
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
  };

  float Ma[RW][R], Mb[RW][R];
  float M[RW][R];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
#pragma unroll
    for (int c = 0; c < R; ++c) {
      M[r][c] = 0.f;
      dS[r][c] = a.dS_final != nullptr ? a.dS_final[(size_t)pr * D * D + (size_t)(cb * R + c) * D + row0 + r] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) pend[j][r] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) dw[j][r] = 0.f;
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
      const size_t row0 = (size_t)pr * T + s0;
      stage_fetch_seg(pq, Q + row0 * D, nq, VEC, D, s0, T);
      stage_fetch_seg(pk, K + row0 * D, nq, VEC, D, s0, T);
      stage_fetch_seg(po, DO + row0 * D, nq, VEC, D, s0, T);
      stage_fetch_seg(pv, V + row0 * D - 3 * D, nv, VEC, D, s0 - 3, T);
      if (Lm1 > 0) {
        stage_fetch_seg(pu, U + row0 * Lm1 * D, nu, VEC, Lm1 * D, s0, T);
        stage_fetch_seg(pg, GM + row0 * Lm1 * D, nu, VEC, Lm1 * D, s0, T);
      }
      // scalars: g, beta (NB each), then alpha (NB x L)
      pres = 0.f;
      if (tid < NB * (2 + (L > 1 ? L : 0))) {
        const int tl = tid < 2 * NB ? tid % NB : (tid - 2 * NB) / L;
        const size_t tr = row0 + tl;
        if (s0 + tl < T) {
          if (tid < NB) pres = Gg[tr];
          else if (tid < 2 * NB) pres = Gb[tr];
          else pres = Ga[tr * L + (tid - 2 * NB) % L];
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
      for (int c = 0; c < R; ++c) {
        x.q[c] = (float)b[tl * D + cb * R + c];
        x.k[c] = (float)b[(NB + tl) * D + cb * R + c];
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
          for (int c = 0; c < R; ++c) x.u[l][c] = (float)b[oU + (tl * Lm1 + l) * D + cb * R + c];
#pragma unroll
          for (int r = 0; r < RW; ++r) x.gm[l][r] = (float)b[oG + (tl * Lm1 + l) * D + row0 + r];
        }
      }
      x.g = sts[bs][tl];
      x.beta = sts[bs][NB + tl];
#pragma unroll
      for (int l = 0; l <= NR; ++l) x.al[l] = (L > 1 && l < L) ? sts[bs][2 * NB + tl * L + l] : 0.f;
    };

    // ---- pass 1: the forward, keeping the state entering every block (or, with
    // all_states, the state after every token) ----------------------------------------------
    const int nst = (T + NB - 1) / NB;
    const bool all = a.all_states != 0;
    int cur = 0;
    fetch(0);
    commit(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      const int s0 = st * NB;
      if (st + 1 < nst) fetch(s0 + NB);
      for (int t = s0; t < min(T, s0 + NB); ++t) {
        if (!all && t % CK == 0) store_block(ckpt + (size_t)(t / CK) * SD, M);
        Tok x;
        load_tok_s(cur, t - s0, x);
        fwd_step(M, x);
        if (all) store_block(ckpt + (size_t)t * SD, M);
      }
      if (st + 1 < nst) commit(cur ^ 1);
      __syncthreads();
      cur ^= 1;
    }
    if (all) {
      // ---- pass 2 with every S_t kept: the adjoint steps over the stages, last first -----
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int c = 0; c < R; ++c) St[r][c] = M[r][c];
      // S_{t-1}: the kept state, zero before the first token
      auto prev_state = [&](float (&Mx)[RW][R], int t) __attribute__((always_inline)) {
        if (t > 0) {
          load_block(Mx, ckpt + (size_t)(t - 1) * SD);
        } else {
#pragma unroll
          for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int c = 0; c < R; ++c) Mx[r][c] = 0.f;
        }
      };
      fetch((nst - 1) * NB);
      commit(cur);
      __syncthreads();
      for (int st = nst - 1; st >= 0; --st) {
        const int s0 = st * NB, s1 = min(T, s0 + NB);
        if (st > 0) fetch(s0 - NB);
        prev_state(Ma, s1 - 1);
        for (int t = s1 - 1; t >= s0; t -= 2) {  // tokens t (Ma) and t - 1 (Mb)
          if (t - 1 >= s0) prev_state(Mb, t - 1);
          Tok x;
          load_tok_s(cur, t - s0, x);
          rev_step(t, x, Ma);
          if (t - 1 >= s0) {
            if (t - 2 >= s0) prev_state(Ma, t - 2);
            Tok y;
            load_tok_s(cur, t - 1 - s0, y);
            rev_step(t - 1, y, Mb);
          }
        }
        if (ng > 0) flush();
        if (st > 0) commit(cur ^ 1);
        __syncthreads();
        cur ^= 1;
      }
    } else {

    // ---- pass 2: per block (last first) its stages ascending (the block's forward again,
    // keeping every S_t), then descending (the adjoint steps, last token first) -------------
    int blk = a.nblk - 1, j = 0;
    bool rev = false;
    auto nstb = [&](int b) __attribute__((always_inline)) { return (min(T, b * CK + CK) - b * CK + NB - 1) / NB; };
    fetch(blk * CK);
    commit(cur);
    __syncthreads();
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
          fwd_step(M, x);
          store_block(scr + (size_t)(t - t0) * SD, M);
        }
        if (s1 == t1) {
#pragma unroll
          for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int c = 0; c < R; ++c) St[r][c] = M[r][c];
        }
      } else {
        const float* cp = ckpt + (size_t)blk * SD;
        auto prev_state = [&](int t) __attribute__((always_inline)) { return t > t0 ? scr + (size_t)(t - 1 - t0) * SD : cp; };
        load_block(Ma, prev_state(s1 - 1));
        for (int t = s1 - 1; t >= s0; t -= 2) {  // tokens t (Ma) and t - 1 (Mb)
          if (t - 1 >= s0) load_block(Mb, prev_state(t - 1));
          Tok x;
          load_tok_s(cur, t - s0, x);
          rev_step(t, x, Ma);
          if (t - 1 >= s0) {
            if (t - 2 >= s0) load_block(Ma, prev_state(t - 2));
            Tok y;
            load_tok_s(cur, t - 1 - s0, y);
            rev_step(t - 1, y, Mb);
          }
        }
        if (ng > 0) flush();
      }
      if (more) commit(cur ^ 1);
      __syncthreads();
      cur ^= 1;
      blk = nb_;
      j = nj;
      rev = nrev;
    }
    }
  } else {
    // ---- inputs read straight from memory (shapes whose stages do not fit in LDS) ------
    // ---- pass 1: the forward, keeping the state entering every block -------------------
    Tok xa, xb;
    load_tok(0, xa);
    for (int t = 0; t < T; t += 2) {  // tokens t (buffer a) and t + 1 (buffer b)
      if (t % CK == 0) store_block(ckpt + (size_t)(t / CK) * SD, M);
      if (t + 1 < T) load_tok(t + 1, xb);
      fwd_step(M, xa);
      if (t + 1 < T) {
        if ((t + 1) % CK == 0) store_block(ckpt + (size_t)((t + 1) / CK) * SD, M);
        if (t + 2 < T) load_tok(t + 2, xa);
        fwd_step(M, xb);
      }
    }

    // ---- pass 2: blocks in reverse -------------------------------------------------------
    for (int blk = a.nblk - 1; blk >= 0; --blk) {
      const int t0 = blk * CK, t1 = min(T, t0 + CK);
      const float* cp = ckpt + (size_t)blk * SD;
      // the block's forward again, keeping every S_t
      load_block(M, cp);
      load_tok(t0, xa);
      for (int t = t0; t < t1; t += 2) {
        if (t + 1 < t1) load_tok(t + 1, xb);
        fwd_step(M, xa);
        store_block(scr + (size_t)(t - t0) * SD, M);
        if (t + 1 < t1) {
          if (t + 2 < t1) load_tok(t + 2, xa);
          fwd_step(M, xb);
          store_block(scr + (size_t)(t + 1 - t0) * SD, M);
        }
      }
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int c = 0; c < R; ++c) St[r][c] = M[r][c];
      // the adjoint steps, last token first (S_{t-1} is the block state t - 1 - t0, or the
      // checkpoint for the first token)
      auto prev_state = [&](int t) __attribute__((always_inline)) { return t > t0 ? scr + (size_t)(t - 1 - t0) * SD : cp; };
      load_tok(t1 - 1, xa);
      load_block(Ma, prev_state(t1 - 1));
      for (int t = t1 - 1; t >= t0; t -= 2) {  // tokens t (buffers a) and t - 1 (buffers b)
        if (t - 1 >= t0) {
          load_tok(t - 1, xb);
          load_block(Mb, prev_state(t - 1));
        }
        rev_step(t, xa, Ma);
        if (t - 1 >= t0) {
          if (t - 2 >= t0) {
            load_tok(t - 2, xa);
            load_block(Ma, prev_state(t - 2));
          }
          rev_step(t - 1, xb, Mb);
        }
      }
      if (ng > 0) flush();
    }
  }
  if (cb == 0 && L > 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < RW; ++r) a.dconv_part[((size_t)pr * 4 + j) * D + row0 + r] = dw[j][r];
  }
}

// Column sums and scalars of a pair whose rows were split over NSP workgroups: the
// partials added in a fixed order (deterministic); 8 tokens per workgroup.
template <int D, int NRK>
__global__ __launch_bounds__(256) void bwd_part_reduce_kernel(BwdArgs a) {
  using Sh = BwdShape<D, NRK>;
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

// dconv_w[h] = sum over the batch of the pairs' shares (fixed order: deterministic).
__global__ __launch_bounds__(256) void bwd_conv_reduce_kernel(const float* part, float* dconv_w, int B, int H, int D) {
  const int h = blockIdx.x;
  for (int i = threadIdx.x; i < 4 * D; i += 256) {
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += part[((size_t)b * H + h) * 4 * D + i];
    dconv_w[(size_t)h * 4 * D + i] = s;
  }
}

}  // namespace prism
