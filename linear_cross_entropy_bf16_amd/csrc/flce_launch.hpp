// Host-side launchers of the MFMA kernels.  Each launcher family is defined in
// its own source file and instantiated there for one element type and one
// option key per object file (flce_fwd.hip, flce_bwd.hip, flce_ce.hip), so the
// heavy kernel instantiations compile in parallel; flce.hip (the C ABI) only
// calls these declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce_kernels.hpp"
#include "flce_ce.hpp"

namespace flce {

// Grid of the forward GEMM: whole vocabulary tiles go to one launch over
// n_tiles x main_chunks work items (tiles_per_chunk tiles each, handed out by
// take_item); a partial last vocabulary tile (V mod 256 rows) gets a launch of
// its own.
struct FwdGrid {
  int64_t n_tiles;          // token tiles (upper bound: all rows valid)
  int64_t v_full, v_tiles;  // whole vocabulary tiles; all vocabulary tiles
  int64_t main_chunks, tiles_per_chunk;
};

// Forward mode: plain, with the argmax (predicted tokens), or keeping the raw
// logit tiles (stored-logits schedule).
enum class FwdMode { kPlain = 0, kArgmax = 1, kStore = 2 };

// Option keys: forward  bit 0 bias, bit 1 softcap, bit 2 sum of z (smoothing);
//              G kernel bit 0 bias, bit 1 softcap, bit 2 class weights.
// a.queue: 16 ints of device memory, the work-queue counters of the two
// launches (zeroed here first).
template <typename T, int kKey>
void launch_fwd(const FwdArgs<T>& a, const FwdGrid& g, FwdMode mode, hipStream_t s);

template <typename T, int kKey>
void launch_g(const GArgs<T>& a, int64_t grid, hipStream_t s);

template <typename T, typename DW>
void launch_dw(const DwArgs<T, DW>& a, int64_t grid, hipStream_t s);

template <typename T>
void launch_dx(const DxArgs<T>& a, int64_t grid, bool last, hipStream_t s);

// Cross-entropy on logits: mode 0 forward, 1 backward, 2 fused; key bit 0
// softcap, bit 1 sum of z; argmax only with the forward.
template <typename T>
void launch_ce(const CeArgs<T>& a, int mode, int key, bool argmax, hipStream_t s);

}  // namespace flce
