// fwd_fast.hip - launches of the bfloat16, dk = dv = 64, chunk 64 forward: the two-role
// segment sweep (prism_sweep8.h), the inter-segment scan and the MFMA output correction
// (prism_fast.h).
#include "prism_host.h"
#include "prism_sweep8.h"

namespace prism {
namespace host {

prism_status launch_fast(const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream,
                         bool nl_gains) {
  if (!record(ev, 0, stream)) return PRISM_ERR_HIP;
  // L = 1, 2, 4, 8 with the rank-L steps unrolled; other L through the runtime step loop
  const dim3 grid(s.nseg, s.P), block(512);
  if (nl_gains) {  // a.gamma holds the gains of the nonlinear refinement
    switch (a.L) {
      case 2: hipLaunchKernelGGL((seg_sweep8_nl_kernel<64, 64, 1>), grid, block, 0, stream, a); break;
      case 4: hipLaunchKernelGGL((seg_sweep8_nl_kernel<64, 64, 3>), grid, block, 0, stream, a); break;
      case 8: hipLaunchKernelGGL((seg_sweep8_nl_kernel<64, 64, 7>), grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL((seg_sweep8_nl_kernel<64, 64, -1>), grid, block, 0, stream, a); break;
    }
  } else {
    switch (a.L) {
      case 1: hipLaunchKernelGGL((seg_sweep8_kernel<64, 64, 0>), grid, block, 0, stream, a); break;
      case 2: hipLaunchKernelGGL((seg_sweep8_kernel<64, 64, 1>), grid, block, 0, stream, a); break;
      case 4: hipLaunchKernelGGL((seg_sweep8_kernel<64, 64, 3>), grid, block, 0, stream, a); break;
      case 8: hipLaunchKernelGGL((seg_sweep8_kernel<64, 64, 7>), grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL((seg_sweep8_kernel<64, 64, -1>), grid, block, 0, stream, a); break;
    }
  }
  if (hipGetLastError() != hipSuccess || !record(ev, 1, stream)) return PRISM_ERR_HIP;
  hipLaunchKernelGGL((seg_scan_fast_kernel<64, 64>), dim3(s.P, 64 / 2), dim3(256), 0, stream, a);
  if (hipGetLastError() != hipSuccess || !record(ev, 2, stream)) return PRISM_ERR_HIP;
  hipLaunchKernelGGL((seg_fixup_fast_kernel<64, 64>), dim3(s.nseg, s.P), dim3(256), 0, stream, a);
  if (hipGetLastError() != hipSuccess || !record(ev, 3, stream)) return PRISM_ERR_HIP;
  return PRISM_OK;
}

}  // namespace host
}  // namespace prism
