// prism_bwd_args.h - the argument block of the backward kernels (prism_bwd.h), on its own
// so the host code can fill it without compiling the kernels.
#pragma once

namespace prism {

constexpr int kBwdBlock = 64;   // tokens between state checkpoints of the sequential backward
constexpr int kBwdSegSub = 8;   // tokens between state checkpoints inside a segment
constexpr int kBwdGroup = 4;    // chunks per group of the chunked form's two-level scan

struct BwdArgs {
  const void *q, *k, *v, *u, *gamma, *d_o;
  const float *g, *beta, *alpha, *conv_w, *dS_final;
  float *dq, *dk, *dv, *dg, *dbeta, *du, *dalpha, *dgamma;
  float* dconv_part;  // [P][nseg][4][D] dconv_w shares (nseg = 1 for the sequential kernel)
  float* ckpt;        // sequential: [P][NSP][nblk][D * D / NSP] state entering each block;
                      // segments: [P][nseg][NSP][seg_len / kBwdSegSub][..] per sub-block
  float* scratch;     // [..][block tokens][D * D / NSP] states S_t of the block being reversed
  float* part;        // [P][NSP][T][RED] per-workgroup column sums and scalars (NSP > 1)
  // segment-parallel and chunked forms only, float32 [P][nseg][D][D] in S layout (row =
  // value index; the chunked form keeps seg_B and seg_ell in H layout, H = S^T):
  float* seg_B;    // state at the segment end from a zero start
  float* seg_Phi;  // segment operator A_{t0} .. A_{t1-1}
  float* seg_ell;  // adjoint at the segment start from the segment's own outputs
  float* seg_Sin;  // state entering the segment
  float* seg_Lam;  // adjoint of the segment's last state from the tokens after it
  float* carry;    // [P][nseg][3][D] anchor terms a segment owes the three tokens before it
  // chunked form only, bf16 [P][nseg][64][64]: the chunk operator in H layout (H = S^T),
  // the chunk's entering state and the adjoint arriving at its end (S layout)
  void *c_Acc, *c_Sin, *c_Lam;
  void* chunk_mats;  // chunked form only: bf16 [P][nseg][3 + L][64][64] T, Uc, Wc, V' and the
                     // residuals r_0 .. r_{L-2} of each chunk
  // chunked form only, float32 [P][ngrp][64][64], groups of kBwdGroup chunks: the group
  // operator (H layout) and its transpose, its end state from zero and local adjoint (H
  // layout), its entering state and arriving adjoint (S layout)
  float *grp_Acc, *grp_Phi, *grp_B, *grp_ell, *grp_Sin, *grp_Lam;
  int ngrp;
  int H, T, L, nblk;
  int nseg, seg_len;
};

}  // namespace prism
