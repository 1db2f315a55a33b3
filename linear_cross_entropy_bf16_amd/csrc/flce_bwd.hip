// Launchers of the backward contractions for one element type: the G kernel
// (k_bwd_g) for one option key when FLCE_KEY is defined, else the dW and dX
// contractions (k_dw, k_dx).  Built once per (FLCE_T, FLCE_KEY) pair and once
// per FLCE_T without a key, so the instantiations compile in parallel.
#include "flce_launch.hpp"

#ifndef FLCE_T
#error "FLCE_T (uint16_t or float) must be defined"
#endif

namespace flce {

#ifdef FLCE_KEY
template <typename T, int kKey>
void launch_g(const GArgs<T>& a, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((k_bwd_g<T, (kKey & 1) != 0, (kKey & 2) != 0, (kKey & 4) != 0>),
                     dim3(static_cast<unsigned>(grid)), dim3(tile::kThreads), 0, s, a);
}
template void launch_g<FLCE_T, FLCE_KEY>(const GArgs<FLCE_T>&, int64_t, hipStream_t);
#else
template <typename T, typename DW>
void launch_dw(const DwArgs<T, DW>& a, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((k_dw<T, DW>), dim3(static_cast<unsigned>(grid)), dim3(tile::kThreads), 0, s, a);
}
template <typename T>
void launch_dx(const DxArgs<T>& a, int64_t grid, bool last, hipStream_t s) {
  if (last)
    hipLaunchKernelGGL((k_dx<T, true>), dim3(static_cast<unsigned>(grid)), dim3(tile::kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_dx<T, false>), dim3(static_cast<unsigned>(grid)), dim3(tile::kThreads), 0, s, a);
}
template void launch_dw<FLCE_T, float>(const DwArgs<FLCE_T, float>&, int64_t, hipStream_t);
template void launch_dw<FLCE_T, uint16_t>(const DwArgs<FLCE_T, uint16_t>&, int64_t, hipStream_t);
template void launch_dx<FLCE_T>(const DxArgs<FLCE_T>&, int64_t, bool, hipStream_t);
#endif

}  // namespace flce
