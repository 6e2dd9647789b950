// fwd_generic_bf16_dk128.hip - the generic forward for bf16 I/O and key width 128: every
// value width (16, 32, 64, 128) and chunk size (16, 32, 64) whose tiles fit a CU's LDS;
// also the scan and output correction that follow the d = 128 half-split sweep.
#include "prism_generic_launch.h"

PRISM_DEFINE_GENERIC(launch_generic_bf16_dk128, prism::bf16_t, 128)

namespace prism {
namespace host {

// the scan and the output correction of the d = 128 half-split sweep (fwd_fast128_*.hip)
prism_status launch_tail_bf16_d128(const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream) {
  return launch_generic_tail<bf16_t, 128, 128, 64, true>(a, s, ev, stream);
}

}  // namespace host
}  // namespace prism
