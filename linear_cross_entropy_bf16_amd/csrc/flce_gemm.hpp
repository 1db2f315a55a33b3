// MFMA tile engine shared by the four contractions of the fused linear
// cross-entropy (forward logits, recomputed logits, dW and dX).
//
// C[m, n] = sum_k A[m, k] * B[n, k] over one 256 x 256 output tile, fp32
// accumulation, both operands stored K-major (element (r, k) at
// base[r * ld + k]); the backward materialises the transposed operands it
// needs (X^T once, W^T per vocabulary slice, G in both orientations) because
// K-major tiles are what this engine streams fastest.
//
// Work split: 256 threads = 4 wave64s in a 2 x 2 grid, each wave owning a
// 128 x 128 quarter as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (bf16) or
// v_mfma_f32_32x32x2_f32 (fp32).  K advances in slabs of 128 bytes per row
// (64 bf16 / 32 fp32) staged in LDS while later slabs' global loads are in
// flight: bf16 through a ring of five 32 KiB operand slots (all 160 KiB of a
// gfx950 CU), fp32 through a 2 x 64 KiB double buffer.
//
// Accumulator layout (per lane l, block (mb, nb), register r in 0..15):
//   row m = wm*128 + mb*32 + 8*(r/4) + 4*(l/32) + (r%4)
//   col n = wn*128 + nb*32 + (l%32)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace tile {
constexpr int kThreads = 256;
constexpr int kM = 256;                     // output tile rows
constexpr int kN = 256;                     // output tile columns
constexpr int kRowBytes = 128;              // one operand row of one K-slab
constexpr int kOpBytes = kM * kRowBytes;    // one operand, one slab: 32 KiB
constexpr int kStageBytes = 2 * kOpBytes;   // A + B
constexpr int kLdsBytes = 5 * kOpBytes;     // bf16 ring (fp32 uses 2 stages of it): 160 KiB
}  // namespace tile

// Elements per 16-byte chunk.  bf16 is carried as raw uint16_t bits.
template <typename T> struct Vec;
template <> struct Vec<uint16_t> { static constexpr int n = 8; };
template <> struct Vec<float> { static constexpr int n = 4; };

template <typename T>
constexpr int slab_k() { return tile::kRowBytes / (int)sizeof(T); }

// LDS address of 16-byte chunk `chunk` (0..7) of tile row `row` (0..255).
// The XOR swizzle spreads both the 8 rows read by consecutive lanes and the
// 8 rows written by one transposing thread over all 8 chunk positions, so
// 16-byte LDS reads and writes are free of bank conflicts.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * tile::kRowBytes + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// K-major operand view: element (r, k) at base[r * ld + k].
template <typename T>
struct Operand {
  const T* base;
  int64_t ld;   // elements between consecutive rows
  int64_t mn;   // valid rows (M or N extent); rows at or beyond it read as 0
  int64_t k;    // valid extent along K (multiple of 8); columns beyond read as 0
};

// ---------------------------------------------------------------- loaders
// Thread t loads chunk (t % 8) of rows t/8 + 32 i, i = 0..7.
template <typename T>
__device__ __forceinline__ void load_slab(u32x4 (&r)[8], const Operand<T>& op,
                                          int64_t mn0, int64_t k0, int tid) {
  const int64_t k = k0 + (int64_t)(tid & 7) * Vec<T>::n;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = mn0 + (tid >> 3) + 32 * i;
    if (row < op.mn && k < op.k)
      r[i] = *reinterpret_cast<const u32x4*>(op.base + row * op.ld + k);
    else
      r[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_slab(char* s, const u32x4 (&r)[8], int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4*>(s + lds_off((tid >> 3) + 32 * i, tid & 7)) = r[i];
}

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ void mma(f32x16& acc, const u32x4& a, const u32x4& b, uint16_t) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// fp32: the four floats of a chunk are four K steps of 32x32x2; A and B use
// the same (chunk, element) -> k assignment, so the sum is the same.  (Each
// element is copied to a scalar before the bit cast: a bit cast applied to a
// vector-element expression directly reads element 0.)
__device__ __forceinline__ void mma(f32x16& acc, const u32x4& a, const u32x4& b, float) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t ae = a[e], be = b[e];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(ae), __uint_as_float(be), acc, 0, 0, 0);
  }
}

template <typename T>
__device__ __forceinline__ void compute_slab(const char* sA, const char* sB, f32x16 (&acc)[4][4],
                                             int wm, int wn, int lane) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int chunk = 2 * ks + (lane >> 5);
    u32x4 fa[4], fb[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      fa[mb] = *reinterpret_cast<const u32x4*>(sA + lds_off(wm * 128 + mb * 32 + (lane & 31), chunk));
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      fb[nb] = *reinterpret_cast<const u32x4*>(sB + lds_off(wn * 128 + nb * 32 + (lane & 31), chunk));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) mma(acc[mb][nb], fa[mb], fb[nb], T{});
  }
}

// Register-staged path (used for fp32): the next slab's global loads land in
// VGPRs while the current slab is multiplied, then go to the other LDS buffer.
template <typename T>
__device__ __forceinline__ void gemm_tile_regs(const Operand<T>& A, const Operand<T>& B,
                                          int64_t m0, int64_t n0, int64_t K, char* lds,
                                          f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;

  constexpr int SK = slab_k<T>();
  const int64_t nslab = (K + SK - 1) / SK;
  u32x4 ra[8], rb[8];
  load_slab(ra, A, m0, 0, tid);
  load_slab(rb, B, n0, 0, tid);
  store_slab(lds, ra, tid);
  store_slab(lds + tile::kOpBytes, rb, tid);
  __syncthreads();
  for (int64_t s = 0; s < nslab; ++s) {
    const bool more = s + 1 < nslab;
    if (more) {
      load_slab(ra, A, m0, (s + 1) * SK, tid);
      load_slab(rb, B, n0, (s + 1) * SK, tid);
    }
    const char* cur = lds + (s & 1) * tile::kStageBytes;
    compute_slab<T>(cur, cur + tile::kOpBytes, acc, wm, wn, lane);
    if (more) {
      char* nxt = lds + ((s + 1) & 1) * tile::kStageBytes;
      store_slab(nxt, ra, tid);
      store_slab(nxt + tile::kOpBytes, rb, tid);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- bf16 DMA path
// bf16 tiles travel global -> LDS with buffer_load ... lds (no staging
// registers, no LDS store instructions), double-buffered in 64-wide K slabs
// so every row segment is a whole 128-byte line.  Out-of-range rows and
// columns are loads with an out-of-range buffer offset, which the hardware
// turns into zeros, so the loop has no branches.
//
// Operand slabs stream through a ring of five LDS slots in the order A0 B0
// A1 B1 A2 ...; slab j of that stream sits in slot j mod 5.  Per slab:
// fragments of the next 16-wide K step are read while the MFMAs of the current
// one run; after the third step the waves meet at one barrier (slab s+1 has
// landed, slab s is no longer read).  B(s+2) then goes out into A(s)'s slot
// with the fourth step, and A(s+3) into B(s)'s slot with the first step of
// slab s+1: B lands a slab ahead of its use, A two slabs ahead.
//
// Measured on a 8192 x 8192 x 4096 product (one CU per tile, Gaussian data):
// with a double buffer all 16 loads of a wave went out in one 512-cycle step
// while the address unit needs ~1450 cycles for a slab's 64 KiB, the waves
// stalled on load issue and the matrix cores were busy 67% of the cycles; the
// ring spreads the loads over two steps and leaves slack for the A half, 79%.
namespace dma {
constexpr int kBK = 64;                    // bf16 elements of K per slab
constexpr int kOpBytes = 32768;            // one operand, one slab
constexpr int kSlots = 5;
constexpr int kLdsBytes = kSlots * kOpBytes; // 160 KiB
static_assert(kLdsBytes == tile::kLdsBytes, "LDS sizes disagree");
constexpr uint32_t kOob = 0x80000000u;     // buffer offset beyond num_records: reads 0

// s_waitcnt immediate (gfx9 layout): vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; lgkm = 15 leaves LDS/scalar loads unchecked.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// K-major slab: 256 rows x 128 bytes.  The 16-byte chunk is swizzled by
// (row / 2) mod 8: any 16 consecutive rows read at one logical chunk then
// cover all 16 chunk positions of a 256-byte bank line (two rows per line).
__device__ __forceinline__ int kmaj_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int kmaj_off(int row, int chunk) {
  return row * 128 + ((chunk ^ kmaj_swz(row)) << 4);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)kOob, 0x00020000);
}

// One operand's slab = 32 wave-wide 1 KiB blocks, 8 per wave.  The byte
// offsets of a wave's 8 blocks, with rows past the operand already replaced
// by the out-of-range marker, are fixed for the whole tile; per slab only the
// K tail is checked.  A row's byte offset stays below 2^31 (row < 256,
// ld * 2 < 2^23 for every operand the library builds or accepts), so
// in-range lanes never reach the marker.
struct SlabStream {
  const uint16_t* base;   // operand row mn0, column 0
  int64_t kdim;
  uint32_t off[8];
  int c8[2];              // K offset (elements) of this lane's chunk, blocks of even / odd index
};

__device__ __forceinline__ SlabStream slab_stream(const Operand<uint16_t>& op, int64_t mn0,
                                                  int wave, int lane) {
  SlabStream st;
  st.base = op.base + mn0 * op.ld;
  st.kdim = op.k;
  const int64_t rows = op.mn - mn0;
  const int rows_left = rows < 256 ? static_cast<int>(rows) : 256;
  const uint32_t ld2 = static_cast<uint32_t>(op.ld) * 2u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (wave * 8 + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ kmaj_swz(row);            // logical chunk of this lane's slot
    st.off[i] = row < rows_left ? static_cast<uint32_t>(row) * ld2 + static_cast<uint32_t>(c * 16)
                                : kOob;
    if (i < 2) st.c8[i] = c * 8;                         // the swizzle depends on i only via i & 1
  }
  return st;
}

__device__ __forceinline__ void issue_slab(const SlabStream& st, int64_t k0, char* dst, int wave) {
  const __amdgpu_buffer_rsrc_t r = rsrc(st.base + k0);
  const int64_t cols = st.kdim - k0;
  const int cols_left = cols < kBK ? static_cast<int>(cols) : kBK;   // may be <= 0
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool ok = cols_left == kBK || st.c8[i & 1] < cols_left;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + (wave * 8 + i) * 1024), 16,
                                             ok ? st.off[i] : kOob, 0, 0, 0);
  }
}

// A slab known to lie wholly inside K: no per-chunk mask (rows past the
// operand are already out of range in st.off).  Keeping the K-tail test out of
// the main loop removed 16 selects and 22 scalar instructions per slab and
// 2.9% of the cycles of an 8192 x 8192 x 4096 product (160.6 k -> 156.0 k per
// tile).
__device__ __forceinline__ void issue_full_slab(const SlabStream& st, int64_t k0, char* dst, int wave) {
  const __amdgpu_buffer_rsrc_t r = rsrc(st.base + k0);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + (wave * 8 + i) * 1024), 16,
                                             st.off[i], 0, 0, 0);
}

// Fragments of 4 MFMA blocks (32 rows each, starting at tile row `base`) for
// K step `ks` (16 wide) of the slab at `src`.
__device__ __forceinline__ void frags(u32x4 (&f)[4], const char* src, int base, int ks, int lane) {
  const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
  for (int b = 0; b < 4; ++b)
    f[b] = *reinterpret_cast<const u32x4*>(src + kmaj_off(base + b * 32 + (lane & 31), chunk));
}

// Scheduling groups (masks: 0x008 MFMA, 0x100 DS read, 0x020 VMEM read): the
// next step's 8 fragment reads after the step's first 8 MFMAs, one each, and,
// in the steps that carry them, the 8 slab loads after its last 8 MFMAs.
// The fragment reads must come before the slab loads in program order: a
// buffer_load ... lds writes LDS, and the compiler cannot tell that it writes
// a slot no read of this step touches, so reads placed after the loads were
// held behind all of them (into the step's last MFMAs, where the next step
// then waited for them).
template <bool kLoads, int I = 0>
__device__ __forceinline__ void interleave() {
  if constexpr (I < 16) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if constexpr (kLoads && I >= 8) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    interleave<kLoads, I + 1>();
  }
}

}  // namespace dma

// First four slabs of a tile's stream (A0 B0 A1 B1 into slots 0..3).  Issued
// by gemm_tile_dma itself, or ahead of it (kPrefetched) while the previous
// tile's epilogue runs; either way the ring must be idle (no loads in flight,
// no reads pending), which the end of gemm_tile_dma guarantees.
__device__ __forceinline__ void gemm_prologue_dma(const Operand<uint16_t>& A,
                                                  const Operand<uint16_t>& B, int64_t m0,
                                                  int64_t n0, char* lds) {
  using namespace dma;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SlabStream sa = slab_stream(A, m0, wave, lane), sb = slab_stream(B, n0, wave, lane);
  issue_slab(sa, 0, lds, wave);
  issue_slab(sb, 0, lds + kOpBytes, wave);
  issue_slab(sa, kBK, lds + 2 * kOpBytes, wave);
  issue_slab(sb, kBK, lds + 3 * kOpBytes, wave);
}

// kSplit: a main loop over slabs wholly inside K without the K-tail mask,
// then the masked loop for the rest; otherwise one masked loop.  The split is
// faster where the epilogue is light (G 1.8%, dW and dX 0.5%); in the
// forward, whose epilogue keeps more state across tiles, the second copy of
// the loop raised its spills from 30 to 56 registers and made it 2.2% slower.
template <bool kPrefetched = false, bool kSplit = true>
__device__ __forceinline__ void gemm_tile_dma(const Operand<uint16_t>& A,
                                              const Operand<uint16_t>& B, int64_t m0,
                                              int64_t n0, int64_t K, char* lds,
                                              f32x16 (&acc)[4][4]) {
  using namespace dma;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS addresses in SGPRs
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;

  const int64_t nslab = (K + kBK - 1) / kBK;
  // p = slot of A(s); the stream positions after it follow as p + 1, p + 2, ...
  int p = 0;
  auto slot = [&](int c) -> char* {
    int q = p + c;
    q = q >= kSlots ? q - kSlots : q;
    return lds + q * kOpBytes;
  };
  // c = 0: fragments of slab s, c = 2: of slab s+1
  auto load_frags = [&](u32x4 (&fa)[4], u32x4 (&fb)[4], int c, int ks) {
    frags(fa, slot(c), wm * 128, ks, lane);
    frags(fb, slot(c + 1), wn * 128, ks, lane);
  };
  auto mfmas = [&](const u32x4 (&fa)[4], const u32x4 (&fb)[4]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) mma(acc[mb][nb], fa[mb], fb[nb], uint16_t{});
  };

  // Slabs past the end of K are all out of range and land as zeros.
  const SlabStream sa = slab_stream(A, m0, wave, lane), sb = slab_stream(B, n0, wave, lane);
  if constexpr (!kPrefetched) gemm_prologue_dma(A, B, m0, n0, lds);
  // A0, B0 landed: the first 16 of this wave's loads since the ring went idle
  // (loads complete in issue order; any stores issued in between only make the
  // count stricter)
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(16, 15));
  __builtin_amdgcn_s_barrier();
  u32x4 a0[4], b0[4], a1[4], b1[4];
  load_frags(a0, b0, 0, 0);
  // One slab of the loop; `issue` sends out the slabs two ahead.
  auto slab = [&](int64_t s, auto issue) {
    load_frags(a1, b1, 0, 1);                       // reads first (see interleave)
    issue(sa, (s + 2) * kBK, slot(4));              // B(s-1)'s slot
    mfmas(a0, b0);
    interleave<true>();
    load_frags(a0, b0, 0, 2);
    mfmas(a1, b1);
    interleave<false>();
    load_frags(a1, b1, 0, 3);
    mfmas(a0, b0);
    interleave<false>();
    // Keep this step's MFMAs above the wait: they cover the latency of the
    // fragment reads issued with their first half (the scheduler otherwise
    // sinks most of them below the barrier and the wait stalls on reads it
    // has just issued).
    __builtin_amdgcn_sched_barrier(0);
    // every load but A(s+2) done, so A(s+1) and B(s+1) landed (own loads);
    // own reads of slab s done; after the barrier both hold for every wave
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(8, 0));
    __builtin_amdgcn_s_barrier();
    load_frags(a0, b0, 2, 0);
    issue(sb, (s + 2) * kBK, slot(5));              // A(s)'s slot
    mfmas(a1, b1);
    interleave<true>();
    p = p >= 3 ? p - 3 : p + 2;
  };
  // Main loop while the slabs two ahead lie wholly inside K, then the last
  // ones (a partial slab, or slabs past K that land as zeros) with the mask.
  int64_t k_in = K < sa.kdim ? K : sa.kdim;          // the operands' valid K (callers pass K = both)
  k_in = k_in < sb.kdim ? k_in : sb.kdim;
  const int64_t full_slabs = k_in / kBK;
  const int64_t main_end = full_slabs > 2 ? full_slabs - 2 : 0;
  int64_t s = 0;
  if constexpr (kSplit)
    for (; s < main_end; ++s)
      slab(s, [&](const SlabStream& st, int64_t k0, char* dst) { issue_full_slab(st, k0, dst, wave); });
  for (; s < nslab; ++s)
    slab(s, [&](const SlabStream& st, int64_t k0, char* dst) { issue_slab(st, k0, dst, wave); });
  __builtin_amdgcn_s_waitcnt(0);            // drain the loads still in flight
  __builtin_amdgcn_s_barrier();
}

// One 256 x 256 output tile at (m0, n0), K = [0, K).  All 256 threads must
// call it; it ends with a barrier, so `lds` is free again on return.
// kPrefetched (bf16 only): gemm_prefetch has already issued this tile's first
// slabs.
template <typename T, bool kPrefetched = false, bool kSplit = true>
__device__ __forceinline__ void gemm_tile(const Operand<T>& A, const Operand<T>& B, int64_t m0,
                                          int64_t n0, int64_t K, char* lds, f32x16 (&acc)[4][4]) {
  if constexpr (sizeof(T) == 2)
    gemm_tile_dma<kPrefetched, kSplit>(A, B, m0, n0, K, lds, acc);
  else
    gemm_tile_regs<T>(A, B, m0, n0, K, lds, acc);
}

// Start the slab stream of the next tile while the caller still works on the
// previous one in registers (bf16; a no-op for fp32, whose mainloop starts its
// own stream).  Only after gemm_tile has returned, and the caller must not
// touch `lds` until the matching gemm_tile<T, true> call.
template <typename T>
__device__ __forceinline__ void gemm_prefetch(const Operand<T>& A, const Operand<T>& B, int64_t m0,
                                              int64_t n0, char* lds) {
  if constexpr (sizeof(T) == 2) gemm_prologue_dma(A, B, m0, n0, lds);
}

// ---------------------------------------------------------------- tile order
// Workgroups are handed to the 8 XCDs round-robin by id.  Remap the id so each
// XCD walks a contiguous range of logical tiles: the grid (a multiple of 8) is
// sized for an upper bound of the tiles (the valid rows are known only on the
// device), each XCD takes an equal share of the `total` tiles and its surplus
// workgroups return false.
__device__ __forceinline__ bool xcd_logical_n(int64_t wg, int64_t total, int64_t& L) {
  const int64_t per = (total + 7) >> 3;
  const int64_t i = wg >> 3;
  L = (wg & 7) * per + i;
  return i < per && L < total;
}

// Work queue over the XCDs: items [0, total) are cut into 8 contiguous ranges
// of ceil(total / 8), range y meant for XCD y, and q[y] counts the items
// handed out from range y.  A workgroup on XCD x takes the next item of its
// own range and, once that is used up, of the others in turn, so an XCD that
// runs faster also finishes a slower one's last items; -1 when all are taken.
// One atomic per probe, nothing waits on another workgroup; which workgroup
// computes an item does not change its result.
__device__ __forceinline__ int64_t take_item(int32_t* q, int x, int64_t total) {
  const int64_t per = (total + 7) >> 3;
  for (int k = 0; k < 8; ++k) {
    const int y = (x + k) & 7;
    const int64_t lo = y * per;
    const int64_t n = total - lo < per ? total - lo : per;
    if (n <= 0) continue;
    const int64_t t = atomicAdd(reinterpret_cast<int*>(q + y), 1);
    if (t < n) return lo + t;
  }
  return -1;
}

// Grid for take_item: 1/16 more workgroups per XCD than its range holds, to
// take over items of slower XCDs (the rest find every range used up and leave).
__host__ __device__ constexpr int64_t queue_grid(int64_t items) {
  const int64_t per = (items + 7) / 8;
  return 8 * (per + (per + 15) / 16);
}

// Tile of a workgroup in a launch of one tile per workgroup.  Without a queue:
// xcd_logical_n.  With one: the tiles are cut into the 8 ranges of take_item;
// the first 7/8 of each range go to workgroups by id exactly as in
// xcd_logical_n (no atomic), the last 1/8 (its tail) through the queue, q[y]
// counting the tail tiles of range y handed out.  A workgroup past its XCD's
// head takes the next tail tile of the XCD it runs on (hardware XCC_ID), then
// of the others, so a faster XCD finishes a slower one's last tiles (the grid,
// queue_grid, has 1/16 more workgroups per XCD for that).  The tile reaches
// the other threads through `lds` (free: called before any slab is loaded)
// and is made wave-uniform, so addresses derived from it stay scalar.  Returns
// false when the workgroup has no tile.
__device__ __forceinline__ bool claim_tile(int64_t wg, int64_t total, int32_t* q, char* lds,
                                           int64_t& L) {
  if (!q) return xcd_logical_n(wg, total, L);
  const int64_t per = (total + 7) >> 3;
  const int64_t tail = (per + 7) >> 3;
  auto head_of = [&](int64_t y, int64_t& n) {   // tiles of range y, and its head
    const int64_t left = total - y * per;
    n = left < 0 ? 0 : (left < per ? left : per);
    return n > tail ? n - tail : 0;
  };
  const int64_t x = wg & 7, i = wg >> 3;
  int64_t n_x;
  const int64_t head_x = head_of(x, n_x);
  if (i < head_x) {
    L = x * per + i;
    return true;
  }
  if (threadIdx.x == 0) {
    const int hw = static_cast<int>(__builtin_amdgcn_s_getreg((15 << 11) | 20)) & 7;
    int32_t item = -1;
    for (int k = 0; k < 8 && item < 0; ++k) {
      const int y = (hw + k) & 7;
      int64_t n_y;
      const int64_t h = head_of(y, n_y);
      if (n_y - h <= 0) continue;
      const int64_t t = atomicAdd(reinterpret_cast<int*>(q + y), 1);
      if (t < n_y - h) item = static_cast<int32_t>(y * per + h + t);
    }
    *reinterpret_cast<int32_t*>(lds) = item;
  }
  __syncthreads();
  L = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int32_t*>(lds));
  __syncthreads();
  return L >= 0;
}

// Grouped raster: logical tile -> (a, b) with `group` consecutive a-tiles
// sharing each b, so tiles in flight on one XCD reuse each other's panels.
__device__ __forceinline__ void grouped(int64_t L, int64_t ta, int64_t tb, int64_t group,
                                        int64_t& a, int64_t& b) {
  const int64_t per_group = group * tb;
  const int64_t g = L / per_group;
  const int64_t in = L - g * per_group;
  const int64_t a0 = g * group;
  const int64_t gs = (ta - a0) < group ? (ta - a0) : group;
  a = a0 + in % gs;
  b = in / gs;
}

}  // namespace flce
