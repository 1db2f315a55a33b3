// Launcher of the forward GEMM with its online-softmax epilogue (k_fwd) for
// one element type and one option key.  Built once per (FLCE_T, FLCE_KEY) pair
// by the build script, so the instantiations compile in parallel.
#include "flce_launch.hpp"

#ifndef FLCE_T
#error "FLCE_T (uint16_t or float) must be defined"
#endif
#ifndef FLCE_KEY
#error "FLCE_KEY (0..7) must be defined"
#endif

namespace flce {

namespace {
// Work-queue counters of both launches below (8 each) back to zero.
__global__ void k_zero_queue(int32_t* q) { q[threadIdx.x] = 0; }

template <typename T, bool kBias, bool kSoftcap, bool kSumZ, bool kArgmax, bool kStore>
void launch_fwd_mode(const FwdArgs<T>& a, const FwdGrid& g, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_queue, dim3(1), dim3(16), 0, s, a.queue);
  if (g.main_chunks > 0) {
    FwdArgs<T> m = a;
    m.vt_base = 0;
    m.vt_end = g.v_full;
    m.chunk_base = 0;
    m.n_chunks = g.main_chunks;
    m.tiles_per_chunk = g.tiles_per_chunk;
    const int64_t items = g.n_tiles * m.n_chunks;
    const int64_t grid = queue_grid(items);
    hipLaunchKernelGGL((k_fwd<T, kBias, kSoftcap, kSumZ, false, kArgmax, kStore>),
                       dim3(static_cast<unsigned>(grid)), dim3(tile::kThreads), 0, s, m);
  }
  if (g.v_full < g.v_tiles) {
    FwdArgs<T> t = a;
    t.vt_base = g.v_full;
    t.vt_end = g.v_tiles;
    t.chunk_base = g.main_chunks;
    t.n_chunks = 1;
    t.tiles_per_chunk = 1;
    t.queue += 8;
    const int64_t grid = queue_grid(g.n_tiles);
    hipLaunchKernelGGL((k_fwd<T, kBias, kSoftcap, kSumZ, true, kArgmax, kStore>),
                       dim3(static_cast<unsigned>(grid)), dim3(tile::kThreads), 0, s, t);
  }
}
}  // namespace

template <typename T, int kKey>
void launch_fwd(const FwdArgs<T>& a, const FwdGrid& g, FwdMode mode, hipStream_t s) {
  constexpr bool kBias = (kKey & 1) != 0, kSoftcap = (kKey & 2) != 0, kSumZ = (kKey & 4) != 0;
  switch (mode) {
    case FwdMode::kArgmax: launch_fwd_mode<T, kBias, kSoftcap, kSumZ, true, false>(a, g, s); break;
    case FwdMode::kStore: launch_fwd_mode<T, kBias, kSoftcap, kSumZ, false, true>(a, g, s); break;
    default: launch_fwd_mode<T, kBias, kSoftcap, kSumZ, false, false>(a, g, s); break;
  }
}

template void launch_fwd<FLCE_T, FLCE_KEY>(const FwdArgs<FLCE_T>&, const FwdGrid&, FwdMode, hipStream_t);

}  // namespace flce
