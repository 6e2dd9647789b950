// bwd.hip - launches of the backward (prism_bwd.h): the sequential per-pair adjoint sweep
// and the segment-parallel passes, the fixed-order sum of per-workgroup partials and the
// batch sum of dconv_w; and the chunked MFMA form (prism_bwd_chunk.h), which shares the
// anchor carry and the dconv_w sum with the segment-parallel form.
#include "prism_bwd.h"
#include "prism_bwd_chunk.h"
#include "prism_host.h"

namespace prism {
namespace host {

namespace {

// Sequential: D / 16 workgroups per pair (16 state rows each); then, when that is more than
// one, the fixed-order sum of their per-token partials (8 tokens per workgroup, 1-D grid).
template <class E, int D, int NRK>
void bwd_launch_d(const BwdArgs& a, int P, hipStream_t stream) {
  constexpr int NSP = BwdShape<D, NRK>::NSP;
  hipLaunchKernelGGL((bwd_pair_kernel<E, D, NRK>), dim3((unsigned)P * NSP), dim3(256), 0, stream, a);
  if constexpr (NSP > 1) {
    const unsigned nt8 = (unsigned)((a.T + 7) / 8);
    hipLaunchKernelGGL((bwd_part_reduce_kernel<D, NRK, 1>), dim3((unsigned)P * nt8), dim3(256), 0, stream, a);
  }
}

// Segment-parallel: segment states, operators and local adjoints; the two scans; the
// token steps of every segment; partial sums (NSP > 1); the anchor terms across segment
// starts.
// (the token-step kernels are compiled with L fixed when L - 1 fills the rank slots: L = 1,
// 4 and 8, so that their rank loops carry no run-time test)
template <class E, int D, int NRK>
void bwd_seg_launch_d(const BwdArgs& a, int P, hipStream_t stream) {
  constexpr int RW = bwd_seg_rows<D>(), NSP = BwdShape<D, NRK, RW>::NSP;
  const unsigned nwg = (unsigned)P * (unsigned)a.nseg * NSP;
  const bool exact = a.L - 1 == NRK;
  if (exact) hipLaunchKernelGGL((bwd_seg_local_kernel<E, D, NRK, RW, NRK>), dim3(nwg), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((bwd_seg_local_kernel<E, D, NRK, RW, -1>), dim3(nwg), dim3(256), 0, stream, a);
  hipLaunchKernelGGL((bwd_seg_scan_kernel<D>), dim3((unsigned)P, D / 4, 2), dim3(256), 0, stream, a);
  if (exact) hipLaunchKernelGGL((bwd_seg_kernel<E, D, NRK, RW, NRK>), dim3(nwg), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((bwd_seg_kernel<E, D, NRK, RW, -1>), dim3(nwg), dim3(256), 0, stream, a);
  if constexpr (NSP > 1) {
    const unsigned nt8 = (unsigned)((a.T + 7) / 8);
    hipLaunchKernelGGL((bwd_part_reduce_kernel<D, NRK, RW>), dim3((unsigned)P * nt8), dim3(256), 0, stream, a);
  }
  if (a.L > 1 && a.nseg > 1)
    hipLaunchKernelGGL(bwd_seg_carry_kernel, dim3((unsigned)P * (unsigned)a.nseg), dim3(256), 0, stream, a, D);
}

template <class E, int NRK, bool SEG>
void bwd_launch(int d, const BwdArgs& a, int P, hipStream_t stream) {
#define PRISM_BWD_D(D) (SEG ? bwd_seg_launch_d<E, D, NRK>(a, P, stream) : bwd_launch_d<E, D, NRK>(a, P, stream))
  switch (d) {
    case 16: PRISM_BWD_D(16); break;
    case 32: PRISM_BWD_D(32); break;
    case 64: PRISM_BWD_D(64); break;
    default: PRISM_BWD_D(128); break;
  }
#undef PRISM_BWD_D
}

// rank slots compiled in: 0 for L = 1, 3 for L <= 4, 7 for L <= 8
template <class E, bool SEG>
void bwd_dispatch(int d, const BwdArgs& a, int P, hipStream_t stream) {
  if (a.L == 1) bwd_launch<E, 0, SEG>(d, a, P, stream);
  else if (a.L <= 4) bwd_launch<E, 3, SEG>(d, a, P, stream);
  else bwd_launch<E, 7, SEG>(d, a, P, stream);
}

}  // namespace

int bwd_seg_slices(int d) {
  switch (d) {
    case 16: return 16 / (16 * bwd_seg_rows<16>());
    case 32: return 32 / (16 * bwd_seg_rows<32>());
    case 64: return 64 / (16 * bwd_seg_rows<64>());
    default: return 128 / (16 * bwd_seg_rows<128>());
  }
}

prism_status launch_bwd(prism_dtype dt, int d, const BwdArgs& a, int B, int P, float* dconv_w, bool segments,
                        hipStream_t stream) {
  if (segments) {
    if (dt == PRISM_BF16) bwd_dispatch<bf16_t, true>(d, a, P, stream);
    else bwd_dispatch<float, true>(d, a, P, stream);
  } else {
    if (dt == PRISM_BF16) bwd_dispatch<bf16_t, false>(d, a, P, stream);
    else bwd_dispatch<float, false>(d, a, P, stream);
  }
  if (hipGetLastError() != hipSuccess) return PRISM_ERR_HIP;
  if (a.L == 1) return PRISM_OK;
  hipLaunchKernelGGL(bwd_conv_reduce_kernel, dim3(a.H, (4 * d + 63) / 64), dim3(256), 0, stream,
                     static_cast<const float*>(a.dconv_part), dconv_w, B, a.H, d, segments ? a.nseg : 1);
  return hipGetLastError() == hipSuccess ? PRISM_OK : PRISM_ERR_HIP;
}

// Chunked form: segments of one chunk (a.nseg chunks per pair, a.seg_len = 64).
namespace {
template <int NL>
void bwdc_launch(const BwdArgs& a, int P, hipStream_t stream) {
  const dim3 grid((unsigned)a.nseg, (unsigned)P);
  const dim3 ggrid((unsigned)a.ngrp, (unsigned)P);
  hipLaunchKernelGGL((bwdc::bwdc_local_kernel<NL>), grid, dim3(bwdc::NT), 0, stream, a);
  hipLaunchKernelGGL(bwdc::bwdc_compose_kernel, ggrid, dim3(bwdc::NT), 0, stream, a);
  hipLaunchKernelGGL(bwdc::bwdc_scan_kernel, dim3((unsigned)P, 64 / bwdc::kScanCols, 2), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(bwdc::bwdc_expand_kernel, dim3((unsigned)a.ngrp, (unsigned)P, 2), dim3(bwdc::NT), 0, stream, a);
  hipLaunchKernelGGL((bwdc::bwdc_grad_kernel<NL>), grid, dim3(bwdc::NT), 0, stream, a);
}
}  // namespace

prism_status launch_bwd_chunked(const BwdArgs& a, int B, int P, float* dconv_w, hipStream_t stream) {
  switch (a.L) {
    case 1: bwdc_launch<0>(a, P, stream); break;
    case 2: bwdc_launch<1>(a, P, stream); break;
    case 3: bwdc_launch<2>(a, P, stream); break;
    case 4: bwdc_launch<3>(a, P, stream); break;
    case 5: bwdc_launch<4>(a, P, stream); break;
    case 6: bwdc_launch<5>(a, P, stream); break;
    case 7: bwdc_launch<6>(a, P, stream); break;
    case 8: bwdc_launch<7>(a, P, stream); break;
    default: return PRISM_ERR_UNSUPPORTED;
  }
  if (hipGetLastError() != hipSuccess) return PRISM_ERR_HIP;
  if (a.L == 1) return PRISM_OK;
  if (a.nseg > 1)
    hipLaunchKernelGGL(bwd_seg_carry_kernel, dim3((unsigned)P * (unsigned)a.nseg), dim3(256), 0, stream, a, 64);
  hipLaunchKernelGGL(bwdc::bwdc_conv_reduce_kernel, dim3(a.H, 4), dim3(1024), 0, stream,
                     static_cast<const float*>(a.dconv_part), dconv_w, B, a.H, a.nseg);
  return hipGetLastError() == hipSuccess ? PRISM_OK : PRISM_ERR_HIP;
}

}  // namespace host
}  // namespace prism
