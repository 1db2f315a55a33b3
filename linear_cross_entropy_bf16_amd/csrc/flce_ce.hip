// Launchers of the cross-entropy kernels on given logits for one element type
// (FLCE_T), built once per type.
#include "flce_launch.hpp"

#ifndef FLCE_T
#error "FLCE_T (uint16_t or float) must be defined"
#endif

namespace flce {

namespace {
template <typename T, bool kSoftcap, bool kSumZ>
void launch_ce_key(const CeArgs<T>& a, int mode, bool argmax, hipStream_t s) {
  const dim3 rows(static_cast<unsigned>(a.n));
  if (mode == 1) {
    hipLaunchKernelGGL((k_ce_bwd<T, kSoftcap>), rows, dim3(256), 0, s, a);
  } else if (mode == 2) {
    hipLaunchKernelGGL((k_ce_fused<T, kSoftcap, kSumZ>), rows, dim3(kCeThreads), 0, s, a);
  } else if (argmax) {
    hipLaunchKernelGGL((k_ce_fwd<T, kSoftcap, kSumZ, true>), rows, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_ce_fwd<T, kSoftcap, kSumZ, false>), rows, dim3(256), 0, s, a);
  }
}
}  // namespace

template <typename T>
void launch_ce(const CeArgs<T>& a, int mode, int key, bool argmax, hipStream_t s) {
  switch (mode == 1 ? (key & 1) : key) {   // the backward needs no sum of z
    case 0: launch_ce_key<T, false, false>(a, mode, argmax, s); break;
    case 1: launch_ce_key<T, true, false>(a, mode, argmax, s); break;
    case 2: launch_ce_key<T, false, true>(a, mode, argmax, s); break;
    default: launch_ce_key<T, true, true>(a, mode, argmax, s); break;
  }
}

template void launch_ce<FLCE_T>(const CeArgs<FLCE_T>&, int, int, bool, hipStream_t);

}  // namespace flce
