// nl.hip - launches of the nonlinear-refinement kernels (prism_nl.h): the chain-factor
// passes (linear chain or written corrections) and the predictor passes on the anchor
// (gains only, or the whole front end: gains, keys and gates).
#include "prism_host.h"
#include "prism_nl.h"

namespace prism {
namespace host {

prism_status launch_gain(const NlArgs& a, prism_dtype dt, dim3 grid, bool delta, hipStream_t stream) {
  if (dt == PRISM_BF16) {
    if (delta) hipLaunchKernelGGL((nl_gain_kernel<bf16_t, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((nl_gain_kernel<bf16_t, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (delta) hipLaunchKernelGGL((nl_gain_kernel<float, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((nl_gain_kernel<float, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? PRISM_OK : PRISM_ERR_HIP;
}

template <int D>
void launch_pred_d(const NlPredArgs& a, dim3 grid, bool front, hipStream_t stream) {
  if (front) hipLaunchKernelGGL((nl_pred_gain_kernel<D, true, true>), grid, dim3(256), 0, stream, a);
  else if constexpr (D == 128) hipLaunchKernelGGL((nl_pred_gain_lds_kernel<D>), grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((nl_pred_gain_kernel<D, false, false>), grid, dim3(256), 0, stream, a);
}

prism_status launch_pred(const NlPredArgs& a, int dv, dim3 grid, bool front, hipStream_t stream) {
  switch (dv) {
    case 32: launch_pred_d<32>(a, grid, front, stream); break;
    case 64: launch_pred_d<64>(a, grid, front, stream); break;
    default: launch_pred_d<128>(a, grid, front, stream); break;
  }
  return hipGetLastError() == hipSuccess ? PRISM_OK : PRISM_ERR_HIP;
}

}  // namespace host
}  // namespace prism
