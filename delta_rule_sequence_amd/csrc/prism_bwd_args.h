// prism_bwd_args.h - the argument block of the backward kernels (prism_bwd.h), on its own
// so the host code can fill it without compiling the kernels.
#pragma once

namespace prism {

constexpr int kBwdBlock = 64;  // tokens between state checkpoints

struct BwdArgs {
  const void *q, *k, *v, *u, *gamma, *d_o;
  const float *g, *beta, *alpha, *conv_w, *dS_final;
  float *dq, *dk, *dv, *dg, *dbeta, *du, *dalpha, *dgamma;
  float* dconv_part;  // [P][4][D] this pair's share of dconv_w
  float* ckpt;        // [P][nblk][D * D] state entering each block (thread-block order), or
                      // with all_states: [P][T][D * D] the state after every token
  float* scratch;     // [P][kBwdBlock][D * D] states S_t of the block being reversed
  float* part;        // [P][NSP][T][RED] per-workgroup column sums and scalars (NSP > 1)
  int H, T, L, nblk;
  int all_states;  // 1: keep every S_t (one forward sweep fewer); only with LDS staging
};

}  // namespace prism
