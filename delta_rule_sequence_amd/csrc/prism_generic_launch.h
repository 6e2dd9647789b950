// prism_generic_launch.h - launches of the generic forward (prism_kernels.h) for one I/O
// type and key width; included by the fwd_generic_*.hip translation units, each of which
// instantiates the value widths and chunk sizes of one (type, dk).
#pragma once
#include <type_traits>

#include "prism_host.h"

namespace prism {
namespace host {

// The scan and the output correction after a generic sweep (events 2 and 3).
template <class E, int DK, int DV, int C>
prism_status launch_generic_tail(const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream) {
  constexpr int NQ = DK >= 128 ? 8 : 4;      // state columns per scan workgroup
  constexpr int DEPTH = NQ == 8 ? 4 : 8;     // the scan's steps loaded ahead
  const dim3 sgrid(s.P, DV / NQ), sblock(NQ * DK);
  if (s.nseg <= DEPTH)
    hipLaunchKernelGGL((seg_scan_kernel<DK, DV, true>), sgrid, sblock, 0, stream, a);
  else
    hipLaunchKernelGGL((seg_scan_kernel<DK, DV, false>), sgrid, sblock, 0, stream, a);
  if (hipGetLastError() != hipSuccess || !record(ev, 2, stream)) return PRISM_ERR_HIP;
  if constexpr (std::is_same<E, bf16_t>::value && DK == 128 && DV == 128 && C == 64)
    hipLaunchKernelGGL((seg_fixup_mfma_kernel<DK, C, false>), dim3((s.nch + kFixupChunks - 1) / kFixupChunks, s.P),
                       dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((seg_fixup_kernel<E, DK, DV, C>), dim3(s.nch, s.P), dim3(256), 0, stream, a);
  if (hipGetLastError() != hipSuccess || !record(ev, 3, stream)) return PRISM_ERR_HIP;
  return PRISM_OK;
}

template <class E, int DK, int DV, int C>
prism_status launch_generic(const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t stream) {
  if constexpr (!SegLds<E, DK, DV, C>::fits) {
    return PRISM_ERR_UNSUPPORTED;
  } else {
    // eight waves when a tile side is 128 wide (one value and one key column block per
    // wave, two waves per SIMD), four otherwise
    constexpr int NW = (DK >= 128 || DV >= 128) ? 8 : 4;
    if (!record(ev, 0, stream)) return PRISM_ERR_HIP;
    hipLaunchKernelGGL((seg_local_kernel<E, DK, DV, C, NW>), dim3(s.nseg, s.P), dim3(64 * NW), 0, stream, a);
    if (hipGetLastError() != hipSuccess || !record(ev, 1, stream)) return PRISM_ERR_HIP;
    return launch_generic_tail<E, DK, DV, C>(a, s, ev, stream);
  }
}

template <class E, int DK, int DV>
prism_status launch_generic_c(int chunk, const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev, hipStream_t st) {
  switch (chunk) {
    case 16: return launch_generic<E, DK, DV, 16>(a, s, ev, st);
    case 32: return launch_generic<E, DK, DV, 32>(a, s, ev, st);
    case 64: return launch_generic<E, DK, DV, 64>(a, s, ev, st);
    default: return PRISM_ERR_UNSUPPORTED;
  }
}

template <class E, int DK>
prism_status launch_generic_dk(int dv, int chunk, const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev,
                               hipStream_t st) {
  switch (dv) {
    case 16: return launch_generic_c<E, DK, 16>(chunk, a, s, ev, st);
    case 32: return launch_generic_c<E, DK, 32>(chunk, a, s, ev, st);
    case 64: return launch_generic_c<E, DK, 64>(chunk, a, s, ev, st);
    case 128: return launch_generic_c<E, DK, 128>(chunk, a, s, ev, st);
    default: return PRISM_ERR_UNSUPPORTED;
  }
}

}  // namespace host
}  // namespace prism

#define PRISM_DEFINE_GENERIC(NAME, E, DK)                                                               \
  namespace prism {                                                                                     \
  namespace host {                                                                                      \
  prism_status NAME(int dv, int chunk, const FwdArgs& a, const LaunchShape& s, hipEvent_t* ev,           \
                    hipStream_t stream) {                                                               \
    return launch_generic_dk<E, DK>(dv, chunk, a, s, ev, stream);                                       \
  }                                                                                                     \
  }                                                                                                     \
  }
