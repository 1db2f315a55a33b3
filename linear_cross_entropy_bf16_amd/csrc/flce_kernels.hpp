// HIP kernels of the fused linear cross-entropy hot path (gfx950).
//
//   k_prep_count, k_prep_scatter  target range check, ordered map of the valid
//                 rows, n_valid, gradient scale (two passes over row blocks)
//   k_fwd         logits tile by tile (MFMA) with an online-softmax epilogue:
//                 per (row, vocabulary chunk) partial max / sum-exp / sum-z,
//                 target logit captured by the one tile that holds it
//   k_merge       partials -> lse, per-row loss, per-block loss sums
//   k_loss_final  fixed-order sum of the block sums -> scalar loss
//   k_block_sums, k_accuracy_final  the same for per-row hits -> token accuracy
//   k_transpose   X^T once per backward, W^T once per vocabulary slice
//   k_pack_lse    lse of the valid rows, in packed-row order
//   k_bwd_g       recomputed logits of one vocabulary slice -> G slice, in
//                 both orientations
//   k_dw          dW[slice] = scale G_slice^T X   (K = N, written once)
//   k_dx          dX (+)= G_slice W_slice, scaled at the last slice (K = slice width)
//   k_db          db[slice] = scale sum_n G_slice
//
// Every reduction has a fixed order and nothing is accumulated with atomics,
// so results are bitwise reproducible run to run.  The only atomics are the
// work counters of take_item / claim_tile, which decide which workgroup
// computes which tile, not what it computes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce_gemm.hpp"

namespace flce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int64_t kGroup = 8;   // grouped-raster width (tiles sharing a panel)

struct Ctl {           // first bytes of the workspace
  int32_t n_valid;
  int32_t status;      // 0 = targets fine, 1 = some target out of range
  float scale;         // d loss / d (row loss): g / wsum (mean) or g (sum)
  float wall;          // sum of the class weights over the vocabulary (V without weights)
  float wsum;          // what 'mean' divides by: n_valid, or the valid rows' target weights
};

// Valid packed rows of a backward token chunk: the chunk starts at packed row
// row0 and holds at most cap rows (the whole batch is one chunk by default).
__device__ __forceinline__ int64_t chunk_valid(const Ctl* ctl, int64_t row0, int64_t cap) {
  const int64_t left = static_cast<int64_t>(ctl->n_valid) - row0;
  return left < 0 ? 0 : (left < cap ? left : cap);
}

__device__ __forceinline__ float ld_elem(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float ld_elem(const float* p, int64_t i) { return p[i]; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (round to nearest even) in one dword, a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ void store4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = float4{a, b, c, d};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh(x) and its derivative 1 - tanh(x)^2 from q = 2 / (e^(2|x|) + 1), which
// lies in (0, 1]: tanh = sign(x) (1 - q) and 1 - tanh^2 = q (2 - q).  Both keep
// their relative accuracy where tanh saturates (1 - tanh^2 formed from tanh
// would cancel to 0 there); exp2 -> inf gives q = 0, tanh = +-1, derivative 0.
__device__ __forceinline__ float tanh_q(float x) {
  const float e = fast_exp2(__builtin_fabsf(x) * (2.0f * kLog2e));
  return __builtin_amdgcn_rcpf(__builtin_fmaf(e, 0.5f, 0.5f));
}
__device__ __forceinline__ float tanh_from_q(float x, float q) { return __builtin_copysignf(1.0f - q, x); }
__device__ __forceinline__ float fast_tanh(float x) { return tanh_from_q(x, tanh_q(x)); }

// Online softmax state of a set of logits (page "Cutting LLM Memory by 84%",
// "Definition and Forward Pass": a running maximum and a running sum of
// exponentials rescaled whenever the maximum grows): m = max z and
// d = sum of e^(z - m), each term evaluated as 2^((z - m) log2e).  z - m is
// exact near the maximum, so the maximum's own term is exactly 1 and d holds
// ln sum_v e^(z_v - m) to a few ulp of 1 whatever the size of |z|.
// (m, d) <- merged with (m2, d2).  Contraction into fmas is off so that every
// kernel (and every instantiation of one) rounds the merge identically.
__device__ __forceinline__ void lse_merge(float& m, float& d, float m2, float d2) {
#pragma clang fp contract(off)
  const float mx = fmaxf(m, m2);
  if (mx == -INFINITY) return;
  d = d * fast_exp2((m - mx) * kLog2e) + d2 * fast_exp2((m2 - mx) * kLog2e);
  m = mx;
}

// d 2^x + sum, rounded the same way wherever the online update runs
__device__ __forceinline__ float rescale_add(float d, float x, float sum) {
#pragma clang fp contract(off)
  return d * fast_exp2(x) + sum;
}

// lse and the row loss of a valid row from its merged state (m, d), target
// logit z_t and sum of logits sz (page "Cutting LLM Memory by 84%",
// "Definition and Forward Pass": lse - z_t; smoothing and z-loss terms of
// the option set):
//   lse  = m + lam,  lam = ln d = ln sum_v e^(z_v - m)
//   loss = lse - (1-eps) z_t - (eps/V) sz + s lse^2
//        = (1-eps)(m - z_t) + lam + (eps m - (eps/V) sz) + s lse^2
// formed from m - z_t rather than lse - z_t: where the target holds the row's
// maximum m - z_t is exactly 0 and the loss keeps the accuracy of lam, not the
// ulp of lse.  Contraction off: identical rounding in every kernel.
struct RowResult {
  float lse, loss, gap;    // gap = lse - z_t, formed as (m - z_t) + lam
};
__device__ __forceinline__ RowResult finish_row(float m, float d, float zt, float sz, float keep,
                                                float eps, float eps_over_v, float zloss) {
#pragma clang fp contract(off)
  const float lam = log2f(d) * kLn2;
  const float lse = m + lam;
  const float loss = keep * (m - zt) + lam + (eps * m - eps_over_v * sz) + zloss * lse * lse;
  return RowResult{lse, loss, (m - zt) + lam};
}

// ------------------------------------------------------------------- prep
// Target scan in two passes over blocks of kPrepRows rows (one thread per
// row), so it spreads over the GPU at any N: k_prep_count reduces each block
// to its valid-row count, range flag and weight sums (a PrepPart); then
// k_prep_scatter gives each valid row its place in the ordered row map from
// the counts of the blocks before it and a ballot within the block, and
// block 0 sums the partials in block order into the control block.  Every
// sum has a fixed order.
constexpr int kPrepRows = 1024;

struct PrepPart {
  int32_t count;   // valid rows of the block
  int32_t bad;     // 1 if a target of the block is out of range
  double wt;       // sum of the class weights of the block's valid targets
  double wa;       // sum of the class weights over the block's share of the vocabulary
};

#ifdef FLCE_HOST_KERNELS
// fixed-order sum over the 1024 threads of a block (wave trees, then the 16
// wave results in order); every thread gets the result
__device__ __forceinline__ double block_sum_1024(double x, double* sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if (lane == 0) sm[wave] = x;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < 16; ++w) t += sm[w];
  return t;
}

static __global__ __launch_bounds__(kPrepRows) void k_prep_count(const int32_t* __restrict__ targets,
                                                                 int64_t n, int64_t v, int32_t ignore_index,
                                                                 const float* __restrict__ weight,
                                                                 PrepPart* __restrict__ part) {
  __shared__ double sm[16];
  __shared__ int32_t s_cnt[16], s_bad[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kPrepRows + threadIdx.x;
  const int32_t t = i < n ? targets[i] : ignore_index;
  const bool ok = t != ignore_index;
  const bool in = ok && t >= 0 && static_cast<int64_t>(t) < v;
  const int32_t cnt = __popcll(__ballot(ok));
  const int32_t bad = __ballot(ok && !in) != 0 ? 1 : 0;
  if (lane == 0) {
    s_cnt[wave] = cnt;
    s_bad[wave] = bad;
  }
  double wt = 0.0, wa = 0.0;
  if (weight) {
    wt = in ? static_cast<double>(weight[t]) : 0.0;
    // this block's share of the vocabulary for the sum of all class weights
    const int64_t per = (v + gridDim.x - 1) / gridDim.x;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t c1 = c0 + per < v ? c0 + per : v;
    for (int64_t c = c0 + threadIdx.x; c < c1; c += kPrepRows) wa += weight[c];
    wt = block_sum_1024(wt, sm);
    wa = block_sum_1024(wa, sm);
  } else {
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int32_t c = 0, b = 0;
    for (int w = 0; w < 16; ++w) {
      c += s_cnt[w];
      b |= s_bad[w];
    }
    part[blockIdx.x] = PrepPart{c, b, wt, wa};
  }
}

static __global__ __launch_bounds__(kPrepRows) void k_prep_scatter(
    const int32_t* __restrict__ targets, int64_t n, int64_t v, int32_t ignore_index,
    const float* __restrict__ grad_output, int32_t reduction_mean, const float* __restrict__ weight,
    const PrepPart* __restrict__ part, Ctl* __restrict__ ctl, int32_t* __restrict__ rows) {
  __shared__ double sm[16];
  __shared__ int32_t s_cnt[16];
  __shared__ int64_t s_base;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = gridDim.x;
  // valid rows of the blocks before this one
  int64_t before = 0;
  for (int j = threadIdx.x; j < static_cast<int>(blockIdx.x); j += kPrepRows) before += part[j].count;
  const double base = block_sum_1024(static_cast<double>(before), sm);   // exact: an integer < 2^23
  if (threadIdx.x == 0) s_base = static_cast<int64_t>(base);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kPrepRows + threadIdx.x;
  const bool ok = i < n && targets[i] != ignore_index;
  const uint64_t m = __ballot(ok);
  if (lane == 0) s_cnt[wave] = __popcll(m);
  __syncthreads();
  int64_t k = s_base;
  for (int w = 0; w < wave; ++w) k += s_cnt[w];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes under this one
  if (ok) rows[k + __popcll(m & below)] = static_cast<int32_t>(i);
  if (blockIdx.x != 0) return;
  // block 0: totals over all blocks, each thread a contiguous range in order
  const int per = (nb + kPrepRows - 1) / kPrepRows;
  const int j0 = threadIdx.x * per, j1 = j0 + per < nb ? j0 + per : nb;
  int64_t nv = 0;
  int32_t any_bad = 0;
  double wts = 0.0, was = 0.0;
  for (int j = j0; j < j1; ++j) {
    nv += part[j].count;
    any_bad |= part[j].bad;
    wts += part[j].wt;
    was += part[j].wa;
  }
  nv = static_cast<int64_t>(block_sum_1024(static_cast<double>(nv), sm));
  any_bad = block_sum_1024(static_cast<double>(any_bad), sm) > 0.0 ? 1 : 0;
  wts = block_sum_1024(wts, sm);
  was = block_sum_1024(was, sm);
  if (threadIdx.x == 0) {
    const float g = grad_output ? grad_output[0] : 1.0f;
    const float den = weight ? static_cast<float>(wts) : static_cast<float>(nv);
    ctl->n_valid = static_cast<int32_t>(nv);
    ctl->status = any_bad;
    ctl->wsum = den;
    ctl->wall = weight ? static_cast<float>(was) : static_cast<float>(v);
    ctl->scale = reduction_mean ? (den > 0.f ? g / den : 0.0f) : g;
  }
}
#endif  // FLCE_HOST_KERNELS

// Valid rows of X (and their targets) packed to the front, in row order: every
// GEMM below runs on n_valid rows only (ignored rows have zero loss and zero
// gradient, page "Cutting LLM Memory by 84%", "Kernel Implementation").
template <typename T>
__global__ __launch_bounds__(256) void k_gather_rows(const T* __restrict__ x, int64_t d,
                                                     const int32_t* __restrict__ targets,
                                                     const int32_t* __restrict__ rows,
                                                     const Ctl* __restrict__ ctl,
                                                     T* __restrict__ xc, int32_t* __restrict__ tc) {
  const int64_t j = blockIdx.x;
  if (j >= ctl->n_valid) return;
  const int64_t r = rows[j];
  const uint4* src = reinterpret_cast<const uint4*>(x + r * d);   // d * sizeof(T) is a multiple of 16
  uint4* dst = reinterpret_cast<uint4*>(xc + j * d);
  const int64_t vecs = d * static_cast<int64_t>(sizeof(T)) / 16;
  for (int64_t i = threadIdx.x; i < vecs; i += 256) dst[i] = src[i];
  if (threadIdx.x == 0) tc[j] = targets[r];
}

#ifdef FLCE_HOST_KERNELS
// lse of each valid row in packed-row order, so the backward's per-token loads
// are independent of the row map.
static __global__ __launch_bounds__(256) void k_pack_lse(const float* __restrict__ lse,
                                                  const int32_t* __restrict__ rows,
                                                  const Ctl* __restrict__ ctl,
                                                  float* __restrict__ lsep) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j < ctl->n_valid) lsep[j] = lse[rows[j]];
}
#endif  // FLCE_HOST_KERNELS

// Rows of dX whose target is ignore_index are zero.
template <typename T>
__global__ __launch_bounds__(256) void k_zero_ignored_rows(T* __restrict__ dx, int64_t d,
                                                           const int32_t* __restrict__ targets,
                                                           int32_t ignore_index) {
  const int64_t r = blockIdx.x;
  if (targets[r] != ignore_index) return;
  uint4* dst = reinterpret_cast<uint4*>(dx + r * d);
  const int64_t vecs = d * static_cast<int64_t>(sizeof(T)) / 16;
  for (int64_t i = threadIdx.x; i < vecs; i += 256) dst[i] = uint4{0u, 0u, 0u, 0u};
}

// ------------------------------------------------------------------- forward
template <typename T>
struct FwdArgs {
  const T* x;             // [n, d] valid rows packed to the front (n_valid of them)
  const T* w;             // [v, d]
  const T* bias;          // [v] or null
  const int32_t* targets;  // packed like x
  int64_t n, d, v;
  float softcap, inv_softcap;
  int64_t n_chunks, tiles_per_chunk, group;   // chunks of this launch; tiles per chunk
  int64_t vt_base, vt_end;   // vocabulary tiles [vt_base, vt_end) of this launch
  int64_t chunk_base;        // partials row of this launch's first chunk
  float* part_m;          // [n_chunks, n] running max of z
  float* part_d;          // [n_chunks, n] sum of e^(z - max), see lse_merge
  float* part_s;          // [n_chunks, n] sum of z
  float* part_b;          // [n_chunks, n] largest z (predicted tokens only)
  int32_t* part_i;        // [n_chunks, n] its lowest vocabulary index
  float* zt;              // [n] target logit, by packed row
  const Ctl* ctl;         // n_valid: rows of x (packed) that take part
  int64_t row0, cap;      // token chunk: first packed row (pointers above start there), capacity
  const float* weight;    // [v] class weights or null: part_s then holds sum_v w_v z_v
  int32_t* queue;         // [8] work-queue counters of this launch, zero at its start (take_item)
  float* zs;              // null, or the raw logit tiles of the chunk, stored in register order
  int64_t zs_vt;          // vocabulary tiles per token tile in zs
};

// Raw logits of one 256 x 256 tile stored for a later pass, in the
// accumulators' register order: tile (nt, vt) owns 64 Ki floats at
// (nt * vt_count + vt) * 65536, wave w's register group i = (mb, nb, q) the
// 1 KiB at (w * 64 + i) * 256, lane l's four values at 4 l.  Every store and
// load of it is one contiguous 1 KiB wave access.
__device__ __forceinline__ float4* stored_tile(float* zs, int64_t nt, int64_t vt, int64_t vt_count,
                                               int wave, int lane) {
  return reinterpret_cast<float4*>(zs + (nt * vt_count + vt) * 65536) + wave * 4096 + lane;
}

// max without NaN canonicalisation (logits here are finite or -inf)
__device__ __forceinline__ float fmax_fast(float a, float b) { return a > b ? a : b; }

// (b, i) <- the larger of (b, i) and (b2, i2), the lower index on a tie
__device__ __forceinline__ void argmax_merge(float& b, int32_t& i, float b2, int32_t i2) {
  if (b2 > b || (b2 == b && i2 < i)) {
    b = b2;
    i = i2;
  }
}

template <typename T, bool kBias, bool kSoftcap, bool kSumZ, bool kMasked, bool kArgmax>
__device__ __forceinline__ void fwd_tile_epilogue(const FwdArgs<T>& a, const f32x16 (&acc)[4][4],
                                                  int64_t v0, int vw, int vlim,
                                                  const int32_t (&tgt)[4], int64_t n0, int wn,
                                                  int lane, float (&m_run)[4], float (&d_run)[4],
                                                  float (&s_run)[4], float (&b_run)[4],
                                                  int32_t (&i_run)[4]) {
  // 32-bit throughout: targets and vocabulary offsets are below 2^31
  const int v0i = static_cast<int>(v0);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int rel32 = tgt[nb] - v0i - vw;
    const bool hit_col = rel32 >= 0 && rel32 < 128 && (rel32 & 4) == 0;
    const int rel = hit_col ? rel32 : -1;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      // one 32 x 32 block at a time: keeps the 16 logits of a block, not the
      // whole tile, in VGPRs
      __builtin_amdgcn_sched_barrier(0);
      float z[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int vl = vw + mb * 32 + 8 * (r >> 2) + (r & 3);
        float zz = acc[mb][nb][r];
        if (kBias) zz += (!kMasked || vl < vlim) ? ld_elem(a.bias, v0 + vl) : 0.f;
        if (kSoftcap) zz = a.softcap * fast_tanh(zz * a.inv_softcap);
        // masked rows (beyond V) drop out of the max and the sums
        z[r] = (!kMasked || vl < vlim) ? zz : -INFINITY;
      }
      // Target logit: at most one lane-value per row in the whole vocabulary.
      if ((rel >> 5) == mb) {
        const int idx = ((rel >> 3) & 3) * 4 + (rel & 3);
        float zt = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) zt = r == idx ? z[r] : zt;
        a.zt[n0 + wn * 128 + nb * 32 + (lane & 31)] = zt;
      }
      // block maximum as a tree of v_max_f32 (a compare-select chain here
      // cost three issue slots and a hazard wait per element, in series)
      float m8[8], m4[4];
#pragma unroll
      for (int k = 0; k < 8; ++k) m8[k] = __builtin_fmaxf(z[2 * k], z[2 * k + 1]);
#pragma unroll
      for (int k = 0; k < 4; ++k) m4[k] = __builtin_fmaxf(m8[2 * k], m8[2 * k + 1]);
      const float mt = __builtin_fmaxf(__builtin_fmaxf(m4[0], m4[1]), __builtin_fmaxf(m4[2], m4[3]));
      if (kArgmax) {
        // r ascends with the vocabulary index: the first r holding the block
        // maximum is its lowest index; blocks and tiles arrive in ascending
        // vocabulary order, so a strict comparison keeps the lowest overall
        int first = 15;
#pragma unroll
        for (int r = 15; r >= 0; --r) first = z[r] == mt ? r : first;
        if (mt > b_run[nb]) {
          b_run[nb] = mt;
          i_run[nb] = v0i + vw + mb * 32 + 8 * (first >> 2) + (first & 3);
        }
      }
      if (kSumZ) {
        float sz = 0.f;
        if (a.weight) {   // class weights: sum_v w_v z_v
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int vl = vw + mb * 32 + 8 * (r >> 2) + (r & 3);
            if (!kMasked || vl < vlim) sz += a.weight[v0 + vl] * z[r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) sz += (!kMasked || z[r] != -INFINITY) ? z[r] : 0.f;
        }
        s_run[nb] += sz;
      }
      if (kMasked && mt == -INFINITY) continue;
      // running maximum and sum of e^(z - max) (see lse_merge)
      const float m_new = fmax_fast(m_run[nb], mt);
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += fast_exp2((z[r] - m_new) * kLog2e);
      d_run[nb] = rescale_add(d_run[nb], (m_run[nb] - m_new) * kLog2e, sum);
      m_run[nb] = m_new;
    }
  }
}

// One workgroup: a 256-token tile against `tiles_per_chunk` consecutive
// 256-wide vocabulary tiles; the logits tile is reduced in registers and
// never leaves the chip (page "[CuteDSL] FLCE", Summary: the forward stores
// only the per-row LSE and target logit).
// kSumZ: label smoothing needs sum_v z of every row.
// kMasked: this launch covers the one partial vocabulary tile (V mod 256 rows);
// the main launch covers whole tiles only and carries no masking code.
// kArgmax: also the largest logit of each row and its lowest index (predicted
// tokens, token accuracy).  kStore: also keep the raw logit tiles in a.zs (a
// separate instantiation: the store code costs the plain forward registers).
template <typename T, bool kBias, bool kSoftcap, bool kSumZ, bool kMasked, bool kArgmax,
          bool kStore = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fwd(FwdArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char lds[tile::kLdsBytes];
  // wave-row exchange of the final partials; gemm_tile has released `lds` by then
  float (*xch)[2][4][32] = reinterpret_cast<float (*)[2][4][32]>(lds);
  // token tiles of the valid rows only, spread over the XCDs
  const int64_t nv = chunk_valid(a.ctl, a.row0, a.cap);
  const int64_t n_tiles = (nv + tile::kN - 1) / tile::kN;
  int64_t L;
  {
    // The XCDs do not run equally fast (one 6% behind another in measured
    // launches), so the work items go out through take_item, keyed by the
    // XCD the workgroup runs on (hardware register XCC_ID).  The item reaches
    // the other threads through LDS before the slab stream uses it, and is
    // made wave-uniform again (readfirstlane), so the tile addresses derived
    // from it stay in scalar registers; taken as a per-lane value it made the
    // forward spill 12 more registers and run 28% slower.  Items fit in 32
    // bits (at most 2^14 token tiles times 2^12 chunks).
    if (threadIdx.x == 0) {
      const int xcd = static_cast<int>(__builtin_amdgcn_s_getreg((15 << 11) | 20)) & 7;
      *reinterpret_cast<int32_t*>(lds) = static_cast<int32_t>(take_item(a.queue, xcd, n_tiles * a.n_chunks));
    }
    __syncthreads();
    L = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int32_t*>(lds));
    __syncthreads();
    if (L < 0) return;                                              // whole workgroup leaves
  }
  int64_t nt, ch;
  grouped(L, n_tiles, a.n_chunks, a.group, nt, ch);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n0 = nt * tile::kN;

  int32_t tgt[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t tok = n0 + wn * 128 + nb * 32 + (lane & 31);
    tgt[nb] = tok < nv ? a.targets[tok] : -1;
  }
  float m_run[4], d_run[4], s_run[4], b_run[4];
  int32_t i_run[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    m_run[nb] = -INFINITY; d_run[nb] = 0.f; s_run[nb] = 0.f;
    b_run[nb] = -INFINITY; i_run[nb] = 0x7fffffff;
  }

  const Operand<T> A{a.w, a.d, a.v, a.d};   // rows: vocabulary
  const Operand<T> B{a.x, a.d, nv, a.d};    // rows: valid tokens
  const int64_t vt_first = a.vt_base + ch * a.tiles_per_chunk;
  const int64_t vt_end = vt_first + a.tiles_per_chunk < a.vt_end ? vt_first + a.tiles_per_chunk
                                                                 : a.vt_end;
  // The slab stream of the next vocabulary tile starts before this tile's
  // epilogue, which works in registers only, so its load latency is hidden.
  if (vt_first < vt_end) gemm_prefetch(A, B, vt_first * tile::kM, n0, lds);
  for (int64_t vt = vt_first; vt < vt_end; ++vt) {
    const int64_t v0 = vt * tile::kM;
    f32x16 acc[4][4];
    gemm_tile<T, true, false>(A, B, v0, n0, a.d, lds, acc);   // one masked loop (see gemm_tile_dma)
    if (vt + 1 < vt_end) gemm_prefetch(A, B, v0 + tile::kM, n0, lds);
    // tile-local vocabulary row of (mb, r) = vw + mb*32 + 8(r/4) + r%4
    const int vw = wm * 128 + 4 * (lane >> 5);
    const int vlim = a.v - v0 < tile::kM ? static_cast<int>(a.v - v0) : tile::kM;

    // One token column and one 32-row block at a time: 16 logits of this lane,
    // bias and softcap applied in registers, merged into the running
    // (max, sum-exp) of the column; the accumulators are never written back.
    fwd_tile_epilogue<T, kBias, kSoftcap, kSumZ, kMasked, kArgmax>(a, acc, v0, vw, vlim, tgt, n0, wn,
                                                                   lane, m_run, d_run, s_run, b_run,
                                                                   i_run);
    // after the epilogue: the accumulators are still intact, and the store
    // adds no registers to the epilogue
    if constexpr (kStore) {   // logits kept for the stored-logits backward
      float4* z = stored_tile(a.zs, nt, vt, a.zs_vt, wave, lane);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            z[((mb * 4 + nb) * 4 + q) * 64] = float4{acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1],
                                                     acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]};
    }
  }

  // Combine the two lane halves (same token, disjoint vocabulary rows) ...
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const float m2 = __shfl_xor(m_run[nb], 32);
    const float d2 = __shfl_xor(d_run[nb], 32);
    const float s2 = __shfl_xor(s_run[nb], 32);
    lse_merge(m_run[nb], d_run[nb], m2, d2);
    s_run[nb] += s2;
    if (kArgmax) argmax_merge(b_run[nb], i_run[nb], __shfl_xor(b_run[nb], 32), __shfl_xor(i_run[nb], 32));
  }
  // ... then the two wave rows through LDS, in a fixed order.
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      xch[0][wn][nb][lane] = m_run[nb];
      xch[1][wn][nb][lane] = d_run[nb];
      xch[2][wn][nb][lane] = s_run[nb];
      if (kArgmax) {
        xch[3][wn][nb][lane] = b_run[nb];
        xch[4][wn][nb][lane] = __int_as_float(i_run[nb]);
      }
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      lse_merge(m_run[nb], d_run[nb], xch[0][wn][nb][lane], xch[1][wn][nb][lane]);
      const float s = s_run[nb] + xch[2][wn][nb][lane];
      if (kArgmax)
        argmax_merge(b_run[nb], i_run[nb], xch[3][wn][nb][lane], __float_as_int(xch[4][wn][nb][lane]));
      const int64_t tok = n0 + wn * 128 + nb * 32 + lane;
      if (tok < nv) {
        const int64_t slot = (a.chunk_base + ch) * a.n + tok;
        a.part_m[slot] = m_run[nb];
        a.part_d[slot] = d_run[nb];
        a.part_s[slot] = s;
        if (kArgmax) {
          a.part_b[slot] = b_run[nb];
          a.part_i[slot] = i_run[nb];
        }
      }
    }
  }
}

struct MergeArgs {
  const float* part_m;
  const float* part_d;
  const float* part_s;
  const float* part_b;  // null unless predicted tokens are wanted
  const int32_t* part_i;
  int32_t* pred;        // [n] or null: predicted token, -1 on ignored rows
  float* hits;          // [n] or null: 1 where the prediction is the target
  const float* zt;
  const int32_t* targets;
  int64_t n, v, n_chunks;
  int32_t ignore_index;
  float keep_target;    // 1 - eps
  float eps_over_v;     // eps / V
  float zloss;          // s
  float* lse;           // [n]
  float* row_loss;      // [n] or null
  float* loss_rows;     // [n] or null (reduction none)
  double* block_sums;   // [n / 256]
  const int32_t* rows;  // packed row -> row
  const Ctl* ctl;
  int64_t row0;         // this launch covers rows [row0, row0 + 256 gridDim.x)
  float* lsep;          // null, or [n] lse by packed row
  const float* weight;  // [v] class weights or null
  float eps;            // eps itself (keep_target = 1 - eps)
};

#ifdef FLCE_HOST_KERNELS
// Partials merged in a fixed order -> lse and row loss (finish_row) on valid
// rows, 0 elsewhere.
static __global__ __launch_bounds__(256) void k_merge(MergeArgs a) {
  __shared__ double red[256];
  if (a.row0 + static_cast<int64_t>(blockIdx.x) * 256 >= a.n) return;   // whole block past the batch
  const int64_t j = a.row0 + static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nv = a.ctl->n_valid;
  double row = 0.0;
  if (j < nv) {                      // packed row j: partials, target logit, sum z by packed index
    float m = -INFINITY, d = 0.f, s = 0.f;
    // 8 chunks' partials loaded ahead of their merges (same order: the same
    // result); one load at a time kept ~0.6 TB/s on this latency-bound loop
    int64_t c = 0;
    for (; c + 8 <= a.n_chunks; c += 8) {
      float pm[8], pd[8], ps[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        pm[k] = a.part_m[(c + k) * a.n + j];
        pd[k] = a.part_d[(c + k) * a.n + j];
        ps[k] = a.part_s[(c + k) * a.n + j];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        lse_merge(m, d, pm[k], pd[k]);
        s += ps[k];
      }
    }
    for (; c < a.n_chunks; ++c) {
      lse_merge(m, d, a.part_m[c * a.n + j], a.part_d[c * a.n + j]);
      s += a.part_s[c * a.n + j];
    }
    const RowResult res = finish_row(m, d, a.zt[j], s, a.keep_target, a.eps, a.eps_over_v, a.zloss);
    const float lse = res.lse;
    const int64_t r = a.rows[j];
    float rl = res.loss;
    if (a.weight) {   // (1-eps) w_t (lse - z_t) + (eps/V)(sum_v w_v lse - sum_v w_v z_v) + s w_t lse^2
      const int32_t t = a.targets[r];
      const float wt = (t >= 0 && t < a.v) ? a.weight[t] : 0.f;
      rl = a.keep_target * wt * res.gap + a.eps_over_v * (a.ctl->wall * lse - s) + a.zloss * wt * lse * lse;
    }
    a.lse[r] = lse;
    if (a.lsep) a.lsep[j] = lse;
    if (a.row_loss) a.row_loss[r] = rl;
    if (a.loss_rows) a.loss_rows[r] = rl;
    row = rl;
    if (a.pred) {
      // chunks in ascending vocabulary order: a strict comparison keeps the
      // lowest index among equal maxima
      float b = -INFINITY;
      int32_t idx = -1;
      for (int64_t c = 0; c < a.n_chunks; ++c) {
        const float bc = a.part_b[c * a.n + j];
        if (bc > b) {
          b = bc;
          idx = a.part_i[c * a.n + j];
        }
      }
      a.pred[r] = idx;
      a.hits[r] = idx == a.targets[r] ? 1.f : 0.f;
    }
  }
  if (j < a.n && a.targets[j] == a.ignore_index) {   // row j itself, if ignored
    a.lse[j] = 0.f;
    if (a.row_loss) a.row_loss[j] = 0.f;
    if (a.loss_rows) a.loss_rows[j] = 0.f;
    if (a.pred) {
      a.pred[j] = -1;
      a.hits[j] = 0.f;
    }
  }
  red[threadIdx.x] = row;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.block_sums[a.row0 / 256 + blockIdx.x] = red[0];
}
#endif  // FLCE_HOST_KERNELS

#ifdef FLCE_HOST_KERNELS
// block_sums[b] = sum of vals [256 b, 256 b + 256) in double, fixed order.
static __global__ __launch_bounds__(256) void k_block_sums(const float* __restrict__ vals, int64_t n,
                                                    double* __restrict__ block_sums) {
  __shared__ double red[256];
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  red[threadIdx.x] = i < n ? static_cast<double>(vals[i]) : 0.0;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) block_sums[blockIdx.x] = red[0];
}
#endif  // FLCE_HOST_KERNELS

#ifdef FLCE_HOST_KERNELS
// Token accuracy: the block sums of the per-row hits over n_valid (0 if none).
static __global__ __launch_bounds__(256) void k_accuracy_final(const double* __restrict__ block_sums,
                                                        int64_t nblocks, const Ctl* __restrict__ ctl,
                                                        float* __restrict__ accuracy) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < nblocks; i += 256) s += block_sums[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int32_t nv = ctl->n_valid;
    accuracy[0] = nv > 0 ? static_cast<float>(red[0] / nv) : 0.f;
  }
}
#endif  // FLCE_HOST_KERNELS

#ifdef FLCE_HOST_KERNELS
static __global__ __launch_bounds__(256) void k_loss_final(const double* __restrict__ block_sums,
                                                    int64_t nblocks, const Ctl* __restrict__ ctl,
                                                    int32_t reduction_mean, float* __restrict__ loss) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < nblocks; i += 256) s += block_sums[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double den = ctl->wsum;   // n_valid, or the valid rows' target weights
    loss[0] = static_cast<float>(reduction_mean ? (den > 0.0 ? red[0] / den : 0.0) : red[0]);
  }
}
#endif  // FLCE_HOST_KERNELS

// ------------------------------------------------------------------- backward
// Every backward contraction reads both operands K-major (K contiguous), the
// layout the MFMA engine streams fastest: X^T is materialised once per
// backward, W^T once per vocabulary slice, and the G slice is written in both
// orientations ([tokens][slice] for dX, [slice][tokens] for dW and db).

// out[c][r] = in[r][c] for r < rows, c < cols; 0 for the padding r < ld_out,
// c < out_rows.  64 x 64 tiles through LDS.  Every global access is one
// 16-byte vector (8 bf16 or 4 fp32 of a row): the library's row pitches are
// multiples of 8 elements and its bases 16-byte aligned, so 64 lanes move
// 1 KiB per load or store (one element per lane ran at ~1.75 TB/s).  A
// thread loads vectors of tile rows into LDS, then gathers one vector of an
// output row (a tile column) element by element.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ in, int64_t rows,
                                                   int64_t cols, int64_t ld_in,
                                                   T* __restrict__ out, int64_t out_rows,
                                                   int64_t ld_out, const Ctl* __restrict__ ctl,
                                                   int64_t row0) {
  constexpr int kV = 16 / static_cast<int>(sizeof(T));   // elements per vector
  constexpr int kVpr = 64 / kV;                          // vectors per tile row
  constexpr int kRpp = 256 / kVpr;                       // tile rows per pass of the block
  constexpr int kPitch = 64 + kV;                        // LDS row pitch: 16-byte aligned rows
  __shared__ __attribute__((aligned(16))) T t[64 * kPitch];
  if (ctl) rows = chunk_valid(ctl, row0, rows);   // X: only the chunk's packed valid rows
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t c0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int lv = threadIdx.x % kVpr, lr = threadIdx.x / kVpr;
#pragma unroll
  for (int i = 0; i < 64 / kRpp; ++i) {
    const int rr = lr + kRpp * i;
    const int64_t r = r0 + rr, c = c0 + lv * kV;   // cols is a multiple of kV: a vector is all in or all out
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (r < rows && c < cols) v = *reinterpret_cast<const u32x4*>(in + r * ld_in + c);
    *reinterpret_cast<u32x4*>(t + rr * kPitch + lv * kV) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 64 / kRpp; ++i) {
    const int cc = lr + kRpp * i;                  // tile column = output row
    const int64_t c = c0 + cc, r = r0 + lv * kV;
    if (c < out_rows && r < ld_out) {
      union {
        T e[kV];
        u32x4 v;
      } g;
#pragma unroll
      for (int j = 0; j < kV; ++j) g.e[j] = t[(lv * kV + j) * kPitch + cc];
      *reinterpret_cast<u32x4*>(out + c * ld_out + r) = g.v;
    }
  }
}

template <typename T>
struct GArgs {
  const T* x;
  const T* w;
  const T* bias;
  const int32_t* targets;
  const float* lsep;    // lse by packed row
  int64_t n, d, v;
  int32_t ignore_index;
  float softcap, inv_softcap;
  float keep_target;    // 1 - eps
  float eps_over_v;
  float two_s;          // 2 s (z-loss)
  int64_t v0, slice_len, ldg, ldt;
  T* g;                 // [n, ldg]       G slice, columns >= slice_len written as 0
  T* gt;                // [gcols, ldt]   the same slice transposed, tokens >= n_valid as 0
  int64_t s_tiles, group;   // vocabulary tiles of the slice; raster group
  int64_t row0;         // token chunk: its first packed row (x, targets, lsep start there)
  const Ctl* ctl;
  const float* zs;      // null, or the chunk's raw logit tiles (see stored_tile): read, not recomputed
  int64_t zs_vt;        // vocabulary tiles per token tile in zs (the slice is then all of V)
  const float* weight;  // [v] class weights (with kWeight)
  int32_t* queue;       // [8] tail counters of this launch (claim_tile), zero at its start, or null
  int32_t* queue_next;  // [8] or null: the next launch's counters, zeroed by workgroup 0
};

__device__ __forceinline__ void store1(uint16_t* p, float a) {
  *p = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
}
__device__ __forceinline__ void store1(float* p, float a) { *p = a; }

// bf16 G tile -> G [n, ldg] and G^T [gcols, ldt] through LDS (free again once
// gemm_tile returns): the tile is staged once per orientation, then every row
// leaves as 32 coalesced 16-byte stores.
// G (row = token): rows padded to 528 bytes.
constexpr int kStagePitch = 264;   // bf16 elements per staged token row (256 + 8)
static_assert(256 * kStagePitch * 2 <= tile::kLdsBytes, "staged G tile exceeds LDS");
// G^T (row = vocabulary): rows 576 bytes apart, and in rows with bit 2 set the
// 16-byte chunks are moved by 8.  A wave's 4-byte write below covers tile rows
// r, r+1, r+4, r+5 (r even) at 16 consecutive token pairs each; the pitch puts
// r and r+1 16 banks apart, the chunk move r+4 and r+5 another 32, so the 64
// lanes hit 64 distinct banks.
constexpr int kStagePitchT = 288;
static_assert(256 * kStagePitchT * 2 <= tile::kLdsBytes, "staged G^T tile exceeds LDS");
__device__ __forceinline__ int gt_stage_off(int row, int col) {
  return row * kStagePitchT + ((((col >> 3) ^ (((row >> 2) & 1) << 3)) << 3) | (col & 7));
}

// gp[nb][mb][2q + h] holds tile rows vw + mb*32 + 8q + 2h and the next one,
// for token column nb.
template <typename T>
__device__ __forceinline__ void store_g_staged(const GArgs<T>& a, const uint32_t (&gp)[4][4][8],
                                               char* lds, int64_t n0, int64_t vl0, int vw, int wn,
                                               int lane, int tid, int64_t nv) {
  uint16_t* sm = reinterpret_cast<uint16_t*>(lds);
  const int tcol = wn * 128 + (lane & 31);        // tile-local token of (nb = 0)
  // G^T: neighbouring lanes hold neighbouring tokens, so each pair of lanes
  // swaps its words (DPP, lanes 2k <-> 2k+1) and keeps one half of each: the
  // even lane then holds row vl for its token and the next, the odd lane row
  // vl + 1 for the previous token and its own, and each writes one 4-byte
  // word.  Address: row (vw + odd) + the block's row offset, token
  // (tcol - odd) + 32 nb, with the chunk move of gt_stage_off folded into nb
  // (for lanes 32..63, whose rows have bit 2 set, 8 chunks = token block nb ^ 2).
  const int odd = lane & 1, hi = lane >> 5;
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;   // v_perm bytes: odd {o.hi, w.hi}, even {w.lo, o.lo}
  const int base = (vw + odd) * kStagePitchT + (tcol - odd);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    uint16_t* col = sm + base + 32 * (nb ^ (2 * hi));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w = gp[nb][mb][i];
        const uint32_t o = static_cast<uint32_t>(
            __builtin_amdgcn_mov_dpp(static_cast<int>(w), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
        *reinterpret_cast<uint32_t*>(col + (mb * 32 + 8 * (i >> 1) + 2 * (i & 1)) * kStagePitchT) =
            __builtin_amdgcn_perm(o, w, sel);
      }
  }
  __syncthreads();
  const int chunk = tid & 31, row0 = tid >> 5;
#pragma unroll 4
  for (int i = 0; i < 32; ++i) {
    const int row = row0 + 8 * i;
    const u32x4 v = *reinterpret_cast<const u32x4*>(sm + gt_stage_off(row, chunk * 8));
    *reinterpret_cast<u32x4*>(a.gt + (vl0 + row) * a.ldt + n0 + chunk * 8) = v;
  }
  __syncthreads();
  // G: staged row = token, 256 vocabulary entries per row (4 consecutive per lane)
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint2*>(sm + (tcol + nb * 32) * kStagePitch + vw + mb * 32 + 8 * q) =
            uint2{gp[nb][mb][2 * q], gp[nb][mb][2 * q + 1]};
  __syncthreads();
#pragma unroll 4
  for (int i = 0; i < 32; ++i) {
    const int row = row0 + 8 * i;
    if (n0 + row < nv) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(sm + row * kStagePitch + chunk * 8);
      *reinterpret_cast<u32x4*>(a.g + (n0 + row) * a.ldg + vl0 + chunk * 8) = v;
    }
  }
}

// fp32 G tile (too large to stage): stored from the accumulator layout.
template <typename T>
__device__ __forceinline__ void store_g_direct(const GArgs<T>& a, const f32x16 (&acc)[4][4],
                                               int64_t n0, int64_t vl0, int vw, int wn, int lane,
                                               int64_t nv) {
  const int ldt = static_cast<int>(a.ldt);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t tok = n0 + wn * 128 + nb * 32 + (lane & 31);
    T* row = a.g + tok * a.ldg + vl0;
    T* col = a.gt + (vl0 + vw) * a.ldt + tok;   // element (vw + i, tok) at col[i * ldt]
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int j = 0; j < 4; ++j) store1(col + (mb * 32 + 8 * q + j) * ldt, acc[mb][nb][4 * q + j]);
        if (tok < nv)
          store4(row + vw + mb * 32 + 8 * q, acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1],
                 acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]);
      }
  }
}

// One element of G from its logit before bias and softcap; is_t marks the
// target column.
// keep_t: (1-eps) times the target's weight; epsw: eps/V times this column's
// weight (both without weights: 1-eps and eps/V).
template <bool kBias, bool kSoftcap, typename T>
__device__ __forceinline__ float g_elem(const GArgs<T>& a, float z, float bv, float lse2, float zfac,
                                        bool is_t, float keep_t, float epsw) {
  if (kBias) z += bv;
  float dz = 1.0f;
  if (kSoftcap) {
    const float x = z * a.inv_softcap;
    const float q = tanh_q(x);
    z = a.softcap * tanh_from_q(x, q);
    dz = q * (2.0f - q);          // 1 - tanh^2, accurate where tanh saturates
  }
  const float p = fast_exp2(__builtin_fmaf(z, kLog2e, -lse2));
  const float sub = is_t ? epsw + keep_t : epsw;
  float g = __builtin_fmaf(p, zfac, -sub);
  if (kSoftcap) g *= dz;
  return g;
}

// bf16 G of one tile, straight from the accumulators into bf16 pairs, then
// staged out.  kEdge: the tile reaches past n_valid or past the slice, whose
// entries are 0.
template <typename T, bool kBias, bool kSoftcap, bool kWeight, bool kEdge>
__device__ __forceinline__ void g_tile_bf16(const GArgs<T>& a, const f32x16 (&acc)[4][4], char* lds,
                                            int64_t n0, int64_t vl0, int vw, int wn, int lane, int tid,
                                            int64_t nv, int vlim, const float (&lse2)[4],
                                            const float (&zfac)[4], const int (&hit)[4],
                                            const bool (&valid)[4], const float (&keep_t)[4]) {
  uint32_t gp[4][4][8];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 2 * i;                                   // rows r, r + 1 of the 32 x 32 block
      const int vl = vw + mb * 32 + 8 * (i >> 1) + 2 * (i & 1);
      const bool in0 = !kEdge || vl < vlim, in1 = !kEdge || vl + 1 < vlim;
      float bv0 = 0.f, bv1 = 0.f;
      if (kBias) {
        bv0 = in0 ? ld_elem(a.bias, a.v0 + vl0 + vl) : 0.f;
        bv1 = in1 ? ld_elem(a.bias, a.v0 + vl0 + vl + 1) : 0.f;
      }
      float ew0 = a.eps_over_v, ew1 = a.eps_over_v;
      if (kWeight) {
        ew0 *= in0 ? a.weight[a.v0 + vl0 + vl] : 0.f;
        ew1 *= in1 ? a.weight[a.v0 + vl0 + vl + 1] : 0.f;
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float g0 = g_elem<kBias, kSoftcap>(a, acc[mb][nb][r], bv0, lse2[nb], zfac[nb], mb * 16 + r == hit[nb],
                                           keep_t[nb], ew0);
        float g1 = g_elem<kBias, kSoftcap>(a, acc[mb][nb][r + 1], bv1, lse2[nb], zfac[nb],
                                           mb * 16 + r + 1 == hit[nb], keep_t[nb], ew1);
        if (kEdge) {
          g0 = (valid[nb] && in0) ? g0 : 0.f;
          g1 = (valid[nb] && in1) ? g1 : 0.f;
        }
        gp[nb][mb][i] = pack_bf16x2(g0, g1);
      }
    }
  store_g_staged(a, gp, lds, n0, vl0, vw, wn, lane, tid, nv);
}

// Recompute one 256 x 256 logits tile of the slice and turn it into
// G = [p (1 + 2 s lse) - (1-eps) onehot - eps/V] (1 - (z/c)^2), p = exp(z - lse)
// (page "Cutting LLM Memory by 84%", "Kernel Implementation", backward:
// probabilities recomputed from the stored LSE, ground truth subtracted).
// kWeight: class weights (per-token target weight, per-column smoothing weight).
template <typename T, bool kBias, bool kSoftcap, bool kWeight>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_bwd_g(GArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char lds[tile::kLdsBytes];
  if (a.queue_next && blockIdx.x == 0 && threadIdx.x < 8) a.queue_next[threadIdx.x] = 0;
  const int64_t nv = chunk_valid(a.ctl, a.row0, a.n);
  const int64_t n_tiles = (nv + tile::kN - 1) / tile::kN;   // valid rows only
  int64_t L;
  if (!claim_tile(blockIdx.x, n_tiles * a.s_tiles, a.queue, lds, L)) return;
  int64_t nt, st;
  grouped(L, n_tiles, a.s_tiles, a.group, nt, st);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n0 = nt * tile::kN, vl0 = st * tile::kM;

  // Per-token inputs are requested before the mainloop, which hides their
  // latency; rows past n_valid read row n_valid - 1 and are masked below.
  int32_t tgt[4];
  float lse_t[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t tok = n0 + wn * 128 + nb * 32 + (lane & 31);
    const int64_t j = tok < nv ? tok : nv - 1;
    tgt[nb] = a.targets[j];
    lse_t[nb] = a.lsep[j];
  }

  f32x16 acc[4][4];
  if (a.zs) {
    const float4* z = stored_tile(const_cast<float*>(a.zs), nt, st, a.zs_vt, wave, lane);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = z[((mb * 4 + nb) * 4 + q) * 64];
          acc[mb][nb][4 * q] = v.x;
          acc[mb][nb][4 * q + 1] = v.y;
          acc[mb][nb][4 * q + 2] = v.z;
          acc[mb][nb][4 * q + 3] = v.w;
        }
  } else {
    const Operand<T> A{a.w + a.v0 * a.d, a.d, a.v - a.v0, a.d};
    const Operand<T> B{a.x, a.d, nv, a.d};       // packed valid rows
    gemm_tile(A, B, vl0, n0, a.d, lds, acc);
  }

  const int vw = wm * 128 + 4 * (lane >> 5);              // tile-local v of (mb = 0, r = 0)
  const int vlim = a.slice_len - vl0 < tile::kM ? static_cast<int>(a.slice_len - vl0) : tile::kM;
  // Rows past the slice and missing tokens get 0.  Per-token terms first,
  // then one vocabulary row (and its bias) at a time across the token blocks.
  float lse2[4], zfac[4], keep_t[4];
  int hit[4];
  bool valid[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t tok = n0 + wn * 128 + nb * 32 + (lane & 31);
    const int32_t t = tgt[nb];
    valid[nb] = tok < nv;          // packed rows all have a target
    const float l = valid[nb] ? lse_t[nb] : 0.f;
    lse2[nb] = l * kLog2e;
    if (kWeight) {   // p [(1-eps) w_t + (eps/V) sum w + 2 s w_t lse] - (1-eps) w_t [v = t] - (eps/V) w_v
      const float wt = (valid[nb] && t >= 0 && t < a.v) ? a.weight[t] : 0.f;
      keep_t[nb] = a.keep_target * wt;
      zfac[nb] = keep_t[nb] + a.eps_over_v * a.ctl->wall + a.two_s * wt * l;
    } else {
      keep_t[nb] = a.keep_target;
      zfac[nb] = 1.0f + a.two_s * l;
    }
    const int64_t rel64 = static_cast<int64_t>(t) - a.v0 - vl0 - vw;
    hit[nb] = (valid[nb] && rel64 >= 0 && rel64 < 128 && (rel64 & 4) == 0)
                  ? static_cast<int>((rel64 >> 5) * 16 + ((rel64 >> 3) & 3) * 4 + (rel64 & 3))
                  : -1;
  }
  if constexpr (sizeof(T) == 2) {
    if (n0 + tile::kN <= nv && vlim == tile::kM)
      g_tile_bf16<T, kBias, kSoftcap, kWeight, false>(a, acc, lds, n0, vl0, vw, wn, lane, tid, nv, vlim,
                                                      lse2, zfac, hit, valid, keep_t);
    else
      g_tile_bf16<T, kBias, kSoftcap, kWeight, true>(a, acc, lds, n0, vl0, vw, wn, lane, tid, nv, vlim,
                                                     lse2, zfac, hit, valid, keep_t);
  } else {
    // fp32: G replaces the logits in the accumulators, then leaves directly
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int vl = vw + mb * 32 + 8 * (r >> 2) + (r & 3);
        const bool vin = vl < vlim;
        const float bv = (kBias && vin) ? ld_elem(a.bias, a.v0 + vl0 + vl) : 0.f;
        const float ew = kWeight ? (vin ? a.eps_over_v * a.weight[a.v0 + vl0 + vl] : 0.f) : a.eps_over_v;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const float g = g_elem<kBias, kSoftcap>(a, acc[mb][nb][r], bv, lse2[nb], zfac[nb],
                                                  mb * 16 + r == hit[nb], keep_t[nb], ew);
          acc[mb][nb][r] = (valid[nb] && vin) ? g : 0.f;
        }
      }
    store_g_direct(a, acc, n0, vl0, vw, wn, lane, nv);
  }
}

template <typename T, typename DW>
struct DwArgs {
  const T* xt;          // [d, ldt]      X^T of the chunk's packed rows, tokens past them 0
  const T* gt;          // [gcols, ldt]  G^T slice
  int64_t d, v0, slice_len, ldt, gcols;
  const Ctl* ctl;
  DW* dw;               // [v, d] fp32, or bf16 bits
  int64_t d_tiles, s_tiles;
  int64_t row0, cap;    // token chunk: first packed row, capacity
  int32_t accumulate;   // add to dW (a later token chunk) instead of overwriting it
};

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}

// dW[v0 + v, :] = scale sum_n G[n, v] X[n, :]: one dedicated contraction over
// all tokens, each output tile written exactly once (page "Cutting LLM Memory
// by 84%", "Path to Production": a dW kernel whose programs own a block of W
// and iterate over the batch).  Computed as C[d, v] so each lane stores four
// consecutive d.
template <typename T, typename DW>
__device__ __forceinline__ void dw_tile(const DwArgs<T, DW>& a, int64_t L, char* lds) {
  int64_t dt, st;
  grouped(L, a.d_tiles, a.s_tiles, kGroup, dt, st);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t kdim = (chunk_valid(a.ctl, a.row0, a.cap) + 7) / 8 * 8;   // the chunk's valid rows
  const Operand<T> A{a.xt, a.ldt, a.d, kdim};       // (d, n) at xt[d*ldt + n]
  const Operand<T> B{a.gt, a.ldt, a.gcols, kdim};   // (v, n) at gt[v*ldt + n]
  f32x16 acc[4][4];
  gemm_tile(A, B, dt * tile::kM, st * tile::kN, kdim, lds, acc);

  const float scale = a.ctl->scale;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t vl = st * tile::kN + wn * 128 + nb * 32 + (lane & 31);
    if (vl >= a.slice_len) continue;
    DW* row = a.dw + (a.v0 + vl) * a.d;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t dd = dt * tile::kM + wm * 128 + mb * 32 + 8 * q + 4 * (lane >> 5);
        if (dd < a.d) {
          float4 v{scale * acc[mb][nb][4 * q], scale * acc[mb][nb][4 * q + 1],
                   scale * acc[mb][nb][4 * q + 2], scale * acc[mb][nb][4 * q + 3]};
          if (a.accumulate) {
            const float4 p = load4(row + dd);
            v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
          }
          store4(row + dd, v.x, v.y, v.z, v.w);
        }
      }
  }
}

template <typename T>
struct DxArgs {
  const T* wt;          // [d, ldg]  W^T slice, vocabulary >= slice length is 0
  const T* g;           // [n, ldg]  packed rows
  int64_t n, d, kdim, ldg;
  const Ctl* ctl;
  float* acc_buf;       // running sum over slices, one 256 x 256 block per output tile (see k_dx)
  T* dx;                // [n, d]
  int32_t first;
  int64_t d_tiles;
  const int32_t* rows;  // packed row -> row (from the chunk's first packed row)
  int64_t row0;         // token chunk: first packed row; n is its capacity
  int32_t* queue;       // [8] tail counters of this launch (claim_tile), zero at its start, or null
  int32_t* queue_next;  // [8] or null: the next launch's counters, zeroed by workgroup 0
};

// dX (+)= G_slice W_slice, computed as C[d, n] tile by tile.  The running
// fp32 sum over slices lives in the workspace in the accumulators' own
// layout: output tile (token tile nt, d tile dt) owns 64 Ki floats at
// ((nt * d_tiles + dt) * 4 + wave) * 16384, and register group i = (mb, nb, q)
// of a wave is the 1 KiB at i * 256 floats, lane l's four values at 4 l.  Every
// load and store of the sum is one contiguous 1 KiB wave access and no staging
// is needed; only the last slice applies the gradient scale and writes dX rows.
constexpr int kDxPitch = 260;   // fp32 per staged token row (256 + 4)
static_assert(128 * kDxPitch * 4 <= tile::kLdsBytes, "staged dX half tile exceeds LDS");
// kLast: the last slice, which scatters the finished rows to dX.
template <typename T, bool kLast>
__device__ __forceinline__ void dx_tile(const DxArgs<T>& a, int64_t L, int64_t nv, int64_t n_tiles,
                                        char* lds) {
  int64_t nt, dt;
  grouped(L, n_tiles, a.d_tiles, kGroup, nt, dt);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const Operand<T> A{a.wt, a.ldg, a.d, a.kdim};   // (d, v) at wt[d*ldg + v]
  const Operand<T> B{a.g, a.ldg, nv, a.kdim};     // (packed row, v) at g[n*ldg + v]
  f32x16 acc[4][4];
  gemm_tile(A, B, dt * tile::kM, nt * tile::kN, a.kdim, lds, acc);

  float4* sum = reinterpret_cast<float4*>(a.acc_buf) +
                ((nt * a.d_tiles + dt) * 4 + wave) * 4096 + lane;
  if (!a.first) {
    // previous slices' sum, 16 groups at a time
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      float4 prev[16];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) prev[nb * 4 + q] = sum[((mb * 4 + nb) * 4 + q) * 64];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 p = prev[nb * 4 + q];
          acc[mb][nb][4 * q] += p.x;
          acc[mb][nb][4 * q + 1] += p.y;
          acc[mb][nb][4 * q + 2] += p.z;
          acc[mb][nb][4 * q + 3] += p.w;
        }
    }
  }
  if constexpr (!kLast) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sum[((mb * 4 + nb) * 4 + q) * 64] = float4{acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1],
                                                     acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]};
  } else {
    // The finished tile goes through LDS (free again once gemm_tile returns)
    // in two halves of 128 tokens, so each dX row leaves in whole 512-byte
    // (bf16) pieces, scattered back to the row it was packed from.
    const float scale = a.ctl->scale;
    float* sm = reinterpret_cast<float*>(lds);
    const int64_t tok0 = nt * tile::kN, d0 = dt * tile::kM;
    const int chunk = tid & 63, row0 = tid >> 6;
    const bool cols_ok = d0 + 4 * chunk < a.d;          // d is a multiple of 8
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int32_t dst_row[32];   // the row of dX each packed row goes to
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int64_t tok = tok0 + h * 128 + row0 + 4 * i;
        dst_row[i] = tok < nv ? a.rows[tok] : 0;
      }
      if (wn == h) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int dl = wm * 128 + mb * 32 + 8 * q + 4 * (lane >> 5);
              *reinterpret_cast<float4*>(sm + (nb * 32 + (lane & 31)) * kDxPitch + dl) =
                  float4{scale * acc[mb][nb][4 * q], scale * acc[mb][nb][4 * q + 1],
                         scale * acc[mb][nb][4 * q + 2], scale * acc[mb][nb][4 * q + 3]};
            }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int row = row0 + 4 * i;
        const int64_t tok = tok0 + h * 128 + row;
        if (tok < nv && cols_ok) {
          const float4 v = *reinterpret_cast<const float4*>(sm + row * kDxPitch + 4 * chunk);
          store4(a.dx + static_cast<int64_t>(dst_row[i]) * a.d + d0 + 4 * chunk, v.x, v.y, v.z, v.w);
        }
      }
      __syncthreads();
    }
  }
}

// Each XCD walks a contiguous range of dW tiles; all 16 x 32 tiles of a slice
// at the headline shape run as two lock-step rounds whose concurrent tiles
// share their K = N operand panels in L2 (interleaving them with dX tiles in
// one launch desynchronised them and made the slice 1.8x slower).
template <typename T, typename DW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_dw(DwArgs<T, DW> a) {
  __shared__ __attribute__((aligned(16))) char lds[tile::kLdsBytes];
  int64_t L;
  if (!xcd_logical_n(blockIdx.x, a.d_tiles * a.s_tiles, L)) return;
  dw_tile(a, L, lds);
}

template <typename T, bool kLast>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_dx(DxArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char lds[tile::kLdsBytes];
  if (a.queue_next && blockIdx.x == 0 && threadIdx.x < 8) a.queue_next[threadIdx.x] = 0;
  const int64_t nv = chunk_valid(a.ctl, a.row0, a.n);
  const int64_t n_tiles = (nv + tile::kN - 1) / tile::kN;   // valid rows only
  int64_t L;
  if (!claim_tile(blockIdx.x, a.d_tiles * n_tiles, a.queue, lds, L)) return;
  dx_tile<T, kLast>(a, L, nv, n_tiles, lds);
}

// db[v0 + v] = scale sum_n G^T[v, n]: one wave per vocabulary row, lanes
// striding over the tokens, then a fixed-order wave reduction.
// accumulate: add to db (a later token chunk); n, row0: the chunk's capacity
// and first packed row.
template <typename T>
__global__ __launch_bounds__(256) void k_db(const T* __restrict__ gt, int64_t ldt, int64_t n,
                                            int64_t v0, int64_t slice_len,
                                            const Ctl* __restrict__ ctl, float* __restrict__ db,
                                            int64_t row0, int32_t accumulate) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (v >= slice_len) return;
  const int lane = threadIdx.x & 63;
  const T* row = gt + v * ldt;
  const int64_t nv = chunk_valid(ctl, row0, n);
  float s = 0.f;
  for (int64_t i = lane; i < nv; i += 64) s += ld_elem(row, i);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) db[v0 + v] = ctl->scale * s + (accumulate ? db[v0 + v] : 0.f);
}

#ifdef FLCE_HOST_KERNELS
static __global__ __launch_bounds__(256) void k_fill(float* __restrict__ p, int64_t count, float value) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < count) p[i] = value;
}
#endif  // FLCE_HOST_KERNELS

}  // namespace flce
