// fwd_generic_bf16_dk128.hip - the generic forward for bf16 I/O and key width 128: every
// value width (16, 32, 64, 128) and chunk size (16, 32, 64) whose tiles fit a CU's LDS;
// also the scan and output correction that follow the d = 128 half-split sweep.
#include "prism_generic_launch.h"
#include "prism_scan128.h"

PRISM_DEFINE_GENERIC(launch_generic_bf16_dk128, prism::bf16_t, 128)

namespace prism {
namespace host {

// the scan (float32 MFMA) and the output correction of the d = 128 half-split sweep
// (fwd_fast128_*.hip); H_in passes between them in bfloat16.  The scan runs one workgroup
// per CU: 16 state columns per workgroup while that keeps every workgroup of the grid
// resident at once, else 32 (half the workgroups, twice the products per step).
prism_status launch_tail_bf16_d128(const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream) {
  if ((size_t)s.P * (128 / 16) <= 256)  // MI355X: 256 CUs
    hipLaunchKernelGGL((seg_scan128_mfma_kernel<16>), dim3(s.P, 128 / 16), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((seg_scan128_mfma_kernel<32>), dim3(s.P, 128 / 32), dim3(512), 0, stream, a);
  if (hipGetLastError() != hipSuccess || !record(ev, 2, stream)) return PRISM_ERR_HIP;
  hipLaunchKernelGGL((seg_fixup_mfma_kernel<128, 64, true>), dim3((s.nch + kFixupChunks - 1) / kFixupChunks, s.P),
                     dim3(256), 0, stream, a);
  if (hipGetLastError() != hipSuccess || !record(ev, 3, stream)) return PRISM_ERR_HIP;
  return PRISM_OK;
}

}  // namespace host
}  // namespace prism
