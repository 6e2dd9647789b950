// prism_host.h - host-side pieces shared by the translation units of libprism.
//
// The kernels are compiled in several translation units so that the library builds in
// parallel: the generic forward per (I/O type, key width), the bfloat16 d = 64 fast path,
// and the backward.  prism_api.hip validates arguments, plans the workspace and calls the
// launch functions declared here; each launch function enqueues its kernels on the
// stream and reports launch failures.
#pragma once
#include <hip/hip_runtime.h>

#include "prism.h"
#include "prism_kernels.h"

namespace prism {

struct BwdArgs;
struct NlArgs;
struct NlPredArgs;

namespace host {

// Kernel launches of one forward: the segment sweep, the inter-segment scan and the
// output correction over P pairs, nch chunks and nseg segments per sequence.  `ev`
// (nullable) receives events before the sweep and after each of the three kernels.
struct LaunchShape {
  int P, nch, nseg;
};

inline bool record(hipEvent_t* ev, int i, hipStream_t stream) {
  return ev == nullptr || hipEventRecord(ev[i], stream) == hipSuccess;
}

// Generic sweep (any supported dk, dv, chunk): one function per I/O type and key width.
#define PRISM_DECL_GENERIC(NAME) \
  prism_status NAME(int dv, int chunk, const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream);
PRISM_DECL_GENERIC(launch_generic_bf16_dk16)
PRISM_DECL_GENERIC(launch_generic_bf16_dk32)
PRISM_DECL_GENERIC(launch_generic_bf16_dk64)
PRISM_DECL_GENERIC(launch_generic_bf16_dk128)
PRISM_DECL_GENERIC(launch_generic_f32_dk16)
PRISM_DECL_GENERIC(launch_generic_f32_dk32)
PRISM_DECL_GENERIC(launch_generic_f32_dk64)
PRISM_DECL_GENERIC(launch_generic_f32_dk128)
#undef PRISM_DECL_GENERIC

// The residual chain a forward runs.  kLinear: factors gamma, r <- r (1 - alpha gamma),
// written alpha r.  kGelu: gains in gamma's place, each factor p Phi(p r) formed on the way
// (d = 64 sweep only).  kDelta: factors of the written corrections, d = gamma r,
// r <- r - d, written alpha d (FwdArgs::chain_delta = 1).
enum class ChainForm { kLinear, kGelu, kDelta };

// The bfloat16, dk = dv = 64, chunk 64 path (prism_sweep8.h, prism_fast.h): the segment
// sweep of the chain form (fwd_fast_*.hip), the scan and the output correction.
prism_status launch_fast(const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream,
                         ChainForm form);
void launch_sweep8_linear(const FwdArgs& a, dim3 grid, hipStream_t stream);
void launch_sweep8_nl(const FwdArgs& a, dim3 grid, hipStream_t stream);
void launch_sweep8_delta(const FwdArgs& a, dim3 grid, hipStream_t stream);

// The bfloat16, dk = dv = 128, chunk 64 path: the half-split segment sweep
// (prism_sweep128.h, grid (nseg, P, 2)) of the chain form, then the d = 128 scan and
// MFMA output correction of the generic path (launch_tail_bf16_d128).
prism_status launch_fast128(const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream,
                            ChainForm form);
// (false: no instantiation for a.L)
bool launch_sweep128_linear(const FwdArgs& a, dim3 grid, hipStream_t stream);
bool launch_sweep128_delta(const FwdArgs& a, dim3 grid, hipStream_t stream);
bool launch_sweep128_nl(const FwdArgs& a, dim3 grid, hipStream_t stream);
prism_status launch_tail_bf16_d128(const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream);

// The backward (prism_bwd.h).  launch_bwd: with segments the segment-parallel passes
// (a.nseg segments of a.seg_len tokens), otherwise the sequential per-pair sweep; then the
// partial sums and, for L > 1, the batch sum of the conv-weight gradient into dconv_w.
// bwd_seg_slices: workgroups per state of the segment-parallel passes at head dim d.
int bwd_seg_slices(int d);
prism_status launch_bwd(prism_dtype dt, int d, const BwdArgs& a, int B, int P, float* dconv_w, bool segments,
                        hipStream_t stream);
// The chunked backward (prism_bwd_chunk.h): bfloat16, dk = dv = 64, one segment per 64-token
// chunk (a.nseg chunks per pair): chunk operators, the chunk scans, chunk gradients, the
// anchor carry and the batch sum of dconv_w.
prism_status launch_bwd_chunked(const BwdArgs& a, int B, int P, float* dconv_w, hipStream_t stream);

// Nonlinear refinement (prism_nl.h, nl.hip).  launch_gain: the chain factors from given
// gains, for the linear chain or (delta) the written corrections.  launch_pred: the factors
// from gains predicted on the anchor (linear chain), or with front the written-correction
// front end (factors, unit keys and gates).
prism_status launch_gain(const NlArgs& a, prism_dtype dt, dim3 grid, bool delta, hipStream_t stream);
prism_status launch_pred(const NlPredArgs& a, int dv, dim3 grid, bool front, hipStream_t stream);

}  // namespace host
}  // namespace prism
