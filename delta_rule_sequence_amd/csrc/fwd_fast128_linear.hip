// fwd_fast128_linear.hip - the d = 128 half-split segment sweep with the linear residual
// chain (one instantiation per L = 1 .. 8, the rank-L steps unrolled), and the launch
// sequence of the d = 128 bfloat16 path.
#include "prism_host.h"
#include "prism_sweep128.h"

namespace prism {
namespace host {

bool launch_sweep128_linear(const FwdArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(512);
  switch (a.L) {
    case 1: hipLaunchKernelGGL((seg_sweep128_kernel<0>), grid, block, 0, stream, a); return true;
    case 2: hipLaunchKernelGGL((seg_sweep128_kernel<1>), grid, block, 0, stream, a); return true;
    case 3: hipLaunchKernelGGL((seg_sweep128_kernel<2>), grid, block, 0, stream, a); return true;
    case 4: hipLaunchKernelGGL((seg_sweep128_kernel<3>), grid, block, 0, stream, a); return true;
    case 5: hipLaunchKernelGGL((seg_sweep128_kernel<4>), grid, block, 0, stream, a); return true;
    case 6: hipLaunchKernelGGL((seg_sweep128_kernel<5>), grid, block, 0, stream, a); return true;
    case 7: hipLaunchKernelGGL((seg_sweep128_kernel<6>), grid, block, 0, stream, a); return true;
    case 8: hipLaunchKernelGGL((seg_sweep128_kernel<7>), grid, block, 0, stream, a); return true;
    default: return false;
  }
}

prism_status launch_fast128(const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream,
                            ChainForm form) {
  if (!record(ev, 0, stream)) return PRISM_ERR_HIP;
  const dim3 grid(s.nseg, s.P, 2);
  const bool ok = form == ChainForm::kDelta  ? launch_sweep128_delta(a, grid, stream)
                  : form == ChainForm::kGelu ? launch_sweep128_nl(a, grid, stream)
                                             : launch_sweep128_linear(a, grid, stream);
  if (!ok) return PRISM_ERR_UNSUPPORTED;
  if (hipGetLastError() != hipSuccess || !record(ev, 1, stream)) return PRISM_ERR_HIP;
  return launch_tail_bf16_d128(a, s, ev, stream);
}

}  // namespace host
}  // namespace prism
