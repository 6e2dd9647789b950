// bwd.hip - launches of the backward (prism_bwd.h): the per-pair adjoint sweep, the
// fixed-order sum of its per-workgroup partials and the batch sum of dconv_w.
#include "prism_bwd.h"
#include "prism_host.h"

namespace prism {
namespace host {

namespace {

template <class E>
bool bwd_staged_e(int d, int L) {
  const int nr = L == 1 ? 1 : L <= 4 ? 3 : 7;
#define PRISM_NB(D) (nr == 1 ? bwd_stage_tokens<E, D, 1>() : nr == 3 ? bwd_stage_tokens<E, D, 3>() \
                                                                      : bwd_stage_tokens<E, D, 7>())
  const int nb = d == 16 ? PRISM_NB(16) : d == 32 ? PRISM_NB(32) : d == 64 ? PRISM_NB(64) : PRISM_NB(128);
#undef PRISM_NB
  return nb > 0;
}

// D / 16 workgroups per pair (16 state rows each); then, when that is more than one, the
// fixed-order sum of their per-token partials (8 tokens per workgroup, 1-D grid).
template <class E, int D, int NRK>
void bwd_launch_d(const BwdArgs& a, int P, hipStream_t stream) {
  constexpr int NSP = D / 16;
  hipLaunchKernelGGL((bwd_pair_kernel<E, D, NRK>), dim3((unsigned)P * NSP), dim3(256), 0, stream, a);
  if constexpr (NSP > 1) {
    const unsigned nt8 = (unsigned)((a.T + 7) / 8);
    hipLaunchKernelGGL((bwd_part_reduce_kernel<D, NRK>), dim3((unsigned)P * nt8), dim3(256), 0, stream, a);
  }
}

template <class E, int NRK>
void bwd_launch(int d, const BwdArgs& a, int P, hipStream_t stream) {
  switch (d) {
    case 16: bwd_launch_d<E, 16, NRK>(a, P, stream); break;
    case 32: bwd_launch_d<E, 32, NRK>(a, P, stream); break;
    case 64: bwd_launch_d<E, 64, NRK>(a, P, stream); break;
    default: bwd_launch_d<E, 128, NRK>(a, P, stream); break;
  }
}

// rank slots compiled in: 0 for L = 1, 3 for L <= 4, 7 for L <= 8
template <class E>
void bwd_dispatch(int d, const BwdArgs& a, int P, hipStream_t stream) {
  if (a.L == 1) bwd_launch<E, 0>(d, a, P, stream);
  else if (a.L <= 4) bwd_launch<E, 3>(d, a, P, stream);
  else bwd_launch<E, 7>(d, a, P, stream);
}

}  // namespace

bool bwd_staged(prism_dtype dt, int d, int L) {
  return dt == PRISM_BF16 ? bwd_staged_e<bf16_t>(d, L) : bwd_staged_e<float>(d, L);
}

prism_status launch_bwd(prism_dtype dt, int d, const BwdArgs& a, int B, int P, float* dconv_w,
                        hipStream_t stream) {
  if (dt == PRISM_BF16) bwd_dispatch<bf16_t>(d, a, P, stream);
  else bwd_dispatch<float>(d, a, P, stream);
  if (hipGetLastError() != hipSuccess) return PRISM_ERR_HIP;
  if (a.L == 1) return PRISM_OK;
  hipLaunchKernelGGL(bwd_conv_reduce_kernel, dim3(a.H), dim3(256), 0, stream,
                     static_cast<const float*>(a.dconv_part), dconv_w, B, a.H, d);
  return hipGetLastError() == hipSuccess ? PRISM_OK : PRISM_ERR_HIP;
}

}  // namespace host
}  // namespace prism
