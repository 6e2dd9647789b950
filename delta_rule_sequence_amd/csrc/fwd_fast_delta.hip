// fwd_fast_delta.hip - the d = 64 segment sweep with the written-correction chain (a.gamma
// holds the corrections' per-channel factors).  L >= 2.
#include "prism_host.h"
#include "prism_sweep8.h"

namespace prism {
namespace host {

void launch_sweep8_delta(const FwdArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(512);
  switch (a.L) {
    case 2: hipLaunchKernelGGL((seg_sweep8_delta_kernel<64, 64, 1>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((seg_sweep8_delta_kernel<64, 64, 3>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((seg_sweep8_delta_kernel<64, 64, 7>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((seg_sweep8_delta_kernel<64, 64, -1>), grid, block, 0, stream, a); break;
  }
}

}  // namespace host
}  // namespace prism
