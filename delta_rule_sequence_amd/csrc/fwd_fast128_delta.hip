// fwd_fast128_delta.hip - the d = 128 half-split segment sweep with the written-correction
// chain (a.gamma holds the corrections' per-channel factors).  L >= 2.
#include "prism_host.h"
#include "prism_sweep128.h"

namespace prism {
namespace host {

void launch_sweep128_delta(const FwdArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(512);
  switch (a.L) {
    case 2: hipLaunchKernelGGL((seg_sweep128_delta_kernel<1>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((seg_sweep128_delta_kernel<3>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((seg_sweep128_delta_kernel<7>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((seg_sweep128_delta_kernel<-1>), grid, block, 0, stream, a); break;
  }
}

}  // namespace host
}  // namespace prism
