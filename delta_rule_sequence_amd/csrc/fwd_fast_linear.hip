// fwd_fast_linear.hip - the d = 64 segment sweep with the linear residual chain; L = 1, 2,
// 4, 8 with the rank-L steps unrolled, other L through the run-time step loop.
#include "prism_host.h"
#include "prism_sweep8.h"

namespace prism {
namespace host {

void launch_sweep8_linear(const FwdArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(512);
  switch (a.L) {
    case 1: hipLaunchKernelGGL((seg_sweep8_kernel<64, 64, 0>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((seg_sweep8_kernel<64, 64, 1>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((seg_sweep8_kernel<64, 64, 3>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((seg_sweep8_kernel<64, 64, 7>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((seg_sweep8_kernel<64, 64, -1>), grid, block, 0, stream, a); break;
  }
}

}  // namespace host
}  // namespace prism
