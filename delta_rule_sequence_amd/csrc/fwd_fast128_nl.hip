// fwd_fast128_nl.hip - the d = 128 half-split segment sweep with the GELU residual chain
// (a.gamma holds the gains; each factor p Phi(p r) is formed in the sweep's own chain), one
// instantiation per L = 2 .. 8.
#include "prism_host.h"
#include "prism_sweep128.h"

namespace prism {
namespace host {

bool launch_sweep128_nl(const FwdArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(512);
  switch (a.L) {
    case 2: hipLaunchKernelGGL((seg_sweep128_nl_kernel<1>), grid, block, 0, stream, a); return true;
    case 3: hipLaunchKernelGGL((seg_sweep128_nl_kernel<2>), grid, block, 0, stream, a); return true;
    case 4: hipLaunchKernelGGL((seg_sweep128_nl_kernel<3>), grid, block, 0, stream, a); return true;
    case 5: hipLaunchKernelGGL((seg_sweep128_nl_kernel<4>), grid, block, 0, stream, a); return true;
    case 6: hipLaunchKernelGGL((seg_sweep128_nl_kernel<5>), grid, block, 0, stream, a); return true;
    case 7: hipLaunchKernelGGL((seg_sweep128_nl_kernel<6>), grid, block, 0, stream, a); return true;
    case 8: hipLaunchKernelGGL((seg_sweep128_nl_kernel<7>), grid, block, 0, stream, a); return true;
    default: return false;
  }
}

}  // namespace host
}  // namespace prism
