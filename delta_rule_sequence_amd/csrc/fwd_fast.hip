// fwd_fast.hip - the bfloat16, dk = dv = 64, chunk 64 forward: the segment sweep (one of
// the chain forms, each instantiated in its own translation unit), then the inter-segment
// scan and the MFMA output correction (prism_fast.h).
#include "prism_fast.h"
#include "prism_host.h"

namespace prism {
namespace host {

prism_status launch_fast(const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream,
                         ChainForm form) {
  if (!record(ev, 0, stream)) return PRISM_ERR_HIP;
  const dim3 grid(s.nseg, s.P);
  switch (form) {
    case ChainForm::kGelu: launch_sweep8_nl(a, grid, stream); break;
    case ChainForm::kDelta: launch_sweep8_delta(a, grid, stream); break;
    default: launch_sweep8_linear(a, grid, stream); break;
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
