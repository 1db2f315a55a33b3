// Cross-entropy on logits given directly, [N, V] row-major in bf16 or fp32:
// the workload of the cross-entropy kernels of "Add efficient Cross-Entropy by
// cuda kernel" (TransformerEngine PR #995, Changes: a forward that reduces each
// row to its maximum and sum of exponentials, and a backward that writes
// softmax - onehot with the smoothing term), with the option set of the fused
// path (ignore_index, label smoothing, z-loss, softcap, mean / sum / none).
//
//   k_ce_fwd       one workgroup per row: online (max, sum-exp, sum-z) over the
//                  row in 16-byte vectors, lse, row loss
//   k_ce_bwd       one workgroup per row: dL/dr from the saved lse, written in
//                  the logits' dtype (in place allowed)
//   k_ce_fused     both in one kernel, one 768-thread workgroup per row whose
//                  registers hold the row between the two passes
//
// Streaming and HBM-bound: each element is read once per pass and the
// gradient written once; nothing is staged.  A row whose base address is not
// 16-byte aligned (V * sizeof(T) not a multiple of 16) is split into a short
// unaligned head, a vectorised body and a short tail, so any V works.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce_kernels.hpp"

namespace flce {

template <typename T>
struct CeArgs {
  const T* logits;          // [n, v] pre-softcap logits
  const int32_t* targets;   // [n]
  int64_t n, v;
  int32_t ignore_index;
  float softcap, inv_softcap;
  float keep_target;        // 1 - eps
  float eps;                // eps
  float eps_over_v;         // eps / V
  float zloss;              // s
  float two_s;              // 2 s
  const Ctl* ctl;           // n_valid and the gradient scale (k_prep)
  float* lse;               // [n] out (forward), 0 on ignored rows
  const float* lse_in;      // [n] in (backward)
  float* row_loss_ws;       // [n] per-row losses for the fixed-order reduction
  float* row_loss;          // [n] or null: per-row losses for the caller
  float* loss_rows;         // [n] or null: reduction 'none'
  T* grad;                  // [n, v] dL/dr (may be `logits`)
  int32_t* pred;            // [n] predicted token, -1 on ignored rows (forward with metrics)
  float* hits;              // [n] 1 where the prediction is the target
};

// 16 bytes of a row as floats, and back (bf16 with round to nearest even).
template <typename T> struct CeVec;
template <> struct CeVec<uint16_t> {
  static constexpr int n = 8;
  static __device__ __forceinline__ void load(const uint16_t* p, float (&z)[8]) {
    unpack(*reinterpret_cast<const uint4*>(p), z);
  }
  static __device__ __forceinline__ void unpack(const uint4& u, float (&z)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[2 * i] = __uint_as_float(w[i] << 16);
      z[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float (&g)[8]) {
    *reinterpret_cast<uint4*>(p) = uint4{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]),
                                         pack_bf16x2(g[4], g[5]), pack_bf16x2(g[6], g[7])};
  }
};
template <> struct CeVec<float> {
  static constexpr int n = 4;
  static __device__ __forceinline__ void load(const float* p, float (&z)[4]) {
    unpack(*reinterpret_cast<const uint4*>(p), z);
  }
  static __device__ __forceinline__ void unpack(const uint4& u, float (&z)[4]) {
    z[0] = __uint_as_float(u.x); z[1] = __uint_as_float(u.y);
    z[2] = __uint_as_float(u.z); z[3] = __uint_as_float(u.w);
  }
  static __device__ __forceinline__ void store(float* p, const float (&g)[4]) {
    *reinterpret_cast<float4*>(p) = float4{g[0], g[1], g[2], g[3]};
  }
};

// Split of row r into [0, head) unaligned, [head, body_end) whole 16-byte
// vectors, [body_end, v) unaligned (head and tail each shorter than a vector).
template <typename T>
struct RowSplit {
  int64_t head, body_end;
  int n_scalar;             // head + tail elements
};
template <typename T>
__device__ __forceinline__ RowSplit<T> row_split(const T* row, int64_t v) {
  constexpr int kVec = CeVec<T>::n;
  const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row) & 15u);
  int64_t head = mis ? static_cast<int64_t>((16u - mis) / sizeof(T)) : 0;
  head = head < v ? head : v;
  const int64_t body_end = head + (v - head) / kVec * kVec;
  return RowSplit<T>{head, body_end, static_cast<int>(head + (v - body_end))};
}
// element index of scalar slot i (0 <= i < n_scalar)
template <typename T>
__device__ __forceinline__ int64_t scalar_index(const RowSplit<T>& sp, int i) {
  return i < sp.head ? i : sp.body_end + (i - sp.head);
}

__device__ __forceinline__ float softcapped(float r, float c, float inv_c, bool on) {
  return on ? c * fast_tanh(r * inv_c) : r;
}

// Running row statistics of one thread: m = max z, d = sum of e^(z - m)
// (see lse_merge), s = sum z (online-softmax recurrence, page "Cutting LLM
// Memory by 84%", "Definition and Forward Pass").
struct RowStats {
  float m, d, s;
};

// maximum of N (a power of two) values as a tree of v_max_f32
template <int N>
__device__ __forceinline__ float tree_max(const float (&z)[N]) {
  if constexpr (N == 1) {
    return z[0];
  } else {
    float h[N / 2];
#pragma unroll
    for (int k = 0; k < N / 2; ++k) h[k] = __builtin_fmaxf(z[2 * k], z[2 * k + 1]);
    return tree_max<N / 2>(h);
  }
}

template <int N, bool kSumZ>
__device__ __forceinline__ void stats_add(RowStats& st, const float (&z)[N]) {
  const float mx = tree_max<N>(z);
  if (kSumZ) {
#pragma unroll
    for (int i = 0; i < N; ++i) st.s += z[i];
  }
  if (mx == -INFINITY) return;          // only masked (-inf) logits here
  const float m_new = fmax_fast(st.m, mx);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) sum += fast_exp2((z[i] - m_new) * kLog2e);
  st.d = rescale_add(st.d, (st.m - m_new) * kLog2e, sum);   // st.m = -inf: the old sum is 0
  st.m = m_new;
}

// Whole-workgroup merge of the per-thread statistics in a fixed order; every
// thread gets the row's result.  `sm` holds 3 kWaves floats of LDS.
template <int kWaves = 4>
__device__ __forceinline__ RowStats block_stats(RowStats st, float* sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(st.m, off), d2 = __shfl_xor(st.d, off), s2 = __shfl_xor(st.s, off);
    lse_merge(st.m, st.d, m2, d2);
    st.s += s2;
  }
  if (lane == 0) {
    sm[wave] = st.m;
    sm[kWaves + wave] = st.d;
    sm[2 * kWaves + wave] = st.s;
  }
  __syncthreads();
  RowStats r{-INFINITY, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    lse_merge(r.m, r.d, sm[w], sm[kWaves + w]);
    r.s += sm[2 * kWaves + w];
  }
  return r;
}

// Largest logit of a thread's elements and its lowest index.
struct RowArgmax {
  float b;
  int32_t i;
};

template <int N>
__device__ __forceinline__ void argmax_add(RowArgmax& am, const float (&z)[N], int64_t e0) {
#pragma unroll
  for (int k = 0; k < N; ++k) argmax_merge(am.b, am.i, z[k], static_cast<int32_t>(e0 + k));
}

// Whole-workgroup argmax in a fixed order (4 waves); `sm` holds 8 floats.
__device__ __forceinline__ RowArgmax block_argmax(RowArgmax am, float* sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
    argmax_merge(am.b, am.i, __shfl_xor(am.b, off), __shfl_xor(am.i, off));
  __syncthreads();                       // sm may still be read by block_stats
  if (lane == 0) {
    sm[wave] = am.b;
    sm[4 + wave] = __int_as_float(am.i);
  }
  __syncthreads();
  RowArgmax r{-INFINITY, 0x7fffffff};
#pragma unroll
  for (int w = 0; w < 4; ++w) argmax_merge(r.b, r.i, sm[w], __float_as_int(sm[4 + w]));
  return r;
}

// Statistics of row `row` (all 256 threads); returns the merged result.
// kArgmax: also the row's argmax into *am (thread-local; merged by the caller).
template <typename T, bool kSoftcap, bool kSumZ, bool kArgmax = false>
__device__ __forceinline__ RowStats row_stats(const CeArgs<T>& a, const T* row, const RowSplit<T>& sp,
                                              float* sm, RowArgmax* am = nullptr) {
  constexpr int kVec = CeVec<T>::n;
  constexpr int kUnroll = 4;
  const int tid = threadIdx.x;
  RowStats st{-INFINITY, 0.f, 0.f};
  if (tid < sp.n_scalar) {
    const int64_t e = scalar_index(sp, tid);
    float z[1] = {softcapped(ld_elem(row, e), a.softcap, a.inv_softcap, kSoftcap)};
    stats_add<1, kSumZ>(st, z);
    if (kArgmax) argmax_add(*am, z, e);
  }
  const int64_t nvec = (sp.body_end - sp.head) / kVec;
  const T* body = row + sp.head;
  int64_t j = tid;
  // kUnroll vectors in flight per thread
  for (; j + (kUnroll - 1) * 256 < nvec; j += kUnroll * 256) {
    float z[kUnroll][kVec];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) CeVec<T>::load(body + (j + u * 256) * kVec, z[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (kSoftcap) {
#pragma unroll
        for (int i = 0; i < kVec; ++i) z[u][i] = softcapped(z[u][i], a.softcap, a.inv_softcap, true);
      }
      stats_add<kVec, kSumZ>(st, z[u]);
      if (kArgmax) argmax_add(*am, z[u], sp.head + (j + u * 256) * kVec);
    }
  }
  for (; j < nvec; j += 256) {
    float z[kVec];
    CeVec<T>::load(body + j * kVec, z);
    if (kSoftcap) {
#pragma unroll
      for (int i = 0; i < kVec; ++i) z[i] = softcapped(z[i], a.softcap, a.inv_softcap, true);
    }
    stats_add<kVec, kSumZ>(st, z);
    if (kArgmax) argmax_add(*am, z, sp.head + j * kVec);
  }
  return block_stats(st, sm);
}

// dL/dr of one logit: scale [p (1 + 2 s lse) - (1-eps) [v = t] - eps/V] (1 - (z/c)^2)
template <bool kSoftcap>
__device__ __forceinline__ float ce_grad(float r, bool is_t, float lse2, float zfac, float scale,
                                         float keep, float eps_v, float c, float inv_c) {
  float z = r, dz = 1.f;
  if (kSoftcap) {
    const float x = r * inv_c;
    const float q = tanh_q(x);
    z = c * tanh_from_q(x, q);
    dz = q * (2.0f - q);          // 1 - tanh^2, accurate where tanh saturates
  }
  const float p = fast_exp2(__builtin_fmaf(z, kLog2e, -lse2));
  float g = __builtin_fmaf(p, zfac, -(is_t ? keep + eps_v : eps_v));
  if (kSoftcap) g *= dz;
  return scale * g;
}

// Gradient pass over row `row` given its lse; `t` < 0 writes zeros.
template <typename T, bool kSoftcap>
__device__ __forceinline__ void row_grad(const CeArgs<T>& a, const T* row, T* grow,
                                         const RowSplit<T>& sp, int64_t t, float lse, float scale) {
  constexpr int kVec = CeVec<T>::n;
  constexpr int kUnroll = 4;
  const int tid = threadIdx.x;
  const bool live = t >= 0;
  const float lse2 = lse * kLog2e, zfac = 1.f + a.two_s * lse;
  const float sc = live ? scale : 0.f;
  if (tid < sp.n_scalar) {
    const int64_t e = scalar_index(sp, tid);
    const float g = live ? ce_grad<kSoftcap>(ld_elem(row, e), e == t, lse2, zfac, sc, a.keep_target,
                                             a.eps_over_v, a.softcap, a.inv_softcap)
                         : 0.f;
    store1(grow + e, g);
  }
  const int64_t nvec = (sp.body_end - sp.head) / kVec;
  const T* body = row + sp.head;
  T* gbody = grow + sp.head;
  const int64_t t_rel = t - sp.head;      // target position within the body
  int64_t j = tid;
  for (; j + (kUnroll - 1) * 256 < nvec; j += kUnroll * 256) {
    float z[kUnroll][kVec];
    if (live) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) CeVec<T>::load(body + (j + u * 256) * kVec, z[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t e0 = (j + u * 256) * kVec;
#pragma unroll
      for (int i = 0; i < kVec; ++i)
        z[u][i] = live ? ce_grad<kSoftcap>(z[u][i], e0 + i == t_rel, lse2, zfac, sc, a.keep_target,
                                           a.eps_over_v, a.softcap, a.inv_softcap)
                       : 0.f;
      CeVec<T>::store(gbody + e0, z[u]);
    }
  }
  for (; j < nvec; j += 256) {
    float z[kVec];
    const int64_t e0 = j * kVec;
    if (live) CeVec<T>::load(body + e0, z);
#pragma unroll
    for (int i = 0; i < kVec; ++i)
      z[i] = live ? ce_grad<kSoftcap>(z[i], e0 + i == t_rel, lse2, zfac, sc, a.keep_target,
                                      a.eps_over_v, a.softcap, a.inv_softcap)
                  : 0.f;
    CeVec<T>::store(gbody + e0, z);
  }
}

// Per-row forward results from the merged statistics (thread 0 only).
template <typename T, bool kSoftcap>
__device__ __forceinline__ float row_finish(const CeArgs<T>& a, const T* row, int64_t r, int64_t t,
                                            const RowStats& st) {
  // a target outside [0, V) is reported by the status word; never read past the row
  const float zt = (t >= 0 && t < a.v) ? softcapped(ld_elem(row, t), a.softcap, a.inv_softcap, kSoftcap)
                                       : 0.f;
  const RowResult res = finish_row(st.m, st.d, zt, st.s, a.keep_target, a.eps, a.eps_over_v, a.zloss);
  const float lse = res.lse, rl = res.loss;
  a.lse[r] = lse;
  a.row_loss_ws[r] = rl;
  if (a.row_loss) a.row_loss[r] = rl;
  if (a.loss_rows) a.loss_rows[r] = rl;
  return lse;
}

template <typename T>
__device__ __forceinline__ void row_ignored(const CeArgs<T>& a, int64_t r) {
  a.lse[r] = 0.f;
  a.row_loss_ws[r] = 0.f;
  if (a.row_loss) a.row_loss[r] = 0.f;
  if (a.loss_rows) a.loss_rows[r] = 0.f;
}

// kArgmax: also the predicted token and whether it is the target.
template <typename T, bool kSoftcap, bool kSumZ, bool kArgmax>
__global__ __launch_bounds__(256) void k_ce_fwd(CeArgs<T> a) {
  __shared__ float sm[12];
  const int64_t r = blockIdx.x;
  const int32_t t = a.targets[r];
  if (t == a.ignore_index) {       // zero loss, row never read
    if (threadIdx.x == 0) {
      row_ignored(a, r);
      if (kArgmax) {
        a.pred[r] = -1;
        a.hits[r] = 0.f;
      }
    }
    return;
  }
  const T* row = a.logits + r * a.v;
  const RowSplit<T> sp = row_split(row, a.v);
  RowArgmax am{-INFINITY, 0x7fffffff};
  const RowStats st = row_stats<T, kSoftcap, kSumZ, kArgmax>(a, row, sp, sm, &am);
  if (kArgmax) am = block_argmax(am, sm);
  if (threadIdx.x == 0) {
    row_finish<T, kSoftcap>(a, row, r, t, st);
    if (kArgmax) {
      a.pred[r] = am.i;
      a.hits[r] = am.i == t ? 1.f : 0.f;
    }
  }
}

template <typename T, bool kSoftcap>
__global__ __launch_bounds__(256) void k_ce_bwd(CeArgs<T> a) {
  const int64_t r = blockIdx.x;
  const int32_t t = a.targets[r];
  const bool live = t != a.ignore_index;
  const T* row = a.logits + r * a.v;
  const RowSplit<T> sp = row_split(row, a.v);
  row_grad<T, kSoftcap>(a, row, a.grad + r * a.v, sp, live ? t : -1, live ? a.lse_in[r] : 0.f,
                        a.ctl->scale);
}

// Fused forward + backward, one 768-thread workgroup per row.  The first
// kCeCache vectors of each thread (a whole 128 Ki-entry bf16 row) stay in
// registers between the statistics pass and the gradient pass, so the row is
// read from memory once; only a longer row's remainder is read twice.
// A copy of v the compiler cannot see through: keeps a cached vector packed
// (4 registers) until the point of use instead of unpacking every cached
// vector right after its load.
__device__ __forceinline__ uint4 opaque(uint4 v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
  return v;
}

constexpr int kCeThreads = 768;   // 3 waves per SIMD: 170 registers each
constexpr int kCeCache = 21;      // 21 x 768 x 8 = 129024 bf16 entries per row

template <typename T, bool kSoftcap, bool kSumZ>
__global__ __launch_bounds__(kCeThreads) void k_ce_fused(CeArgs<T> a) {
  constexpr int kVec = CeVec<T>::n;
  constexpr int kWaves = kCeThreads / 64;
  __shared__ float sm[3 * kWaves + 1];
  const int64_t r = blockIdx.x;
  const int32_t t = a.targets[r];
  const int tid = threadIdx.x;
  const T* row = a.logits + r * a.v;
  T* grow = a.grad + r * a.v;
  const RowSplit<T> sp = row_split(row, a.v);
  // offsets within one row fit in 32 bits (V < 2^31)
  const int nvec = static_cast<int>((sp.body_end - sp.head) / kVec);
  const uint4* body = reinterpret_cast<const uint4*>(row + sp.head);
  uint4* gbody = reinterpret_cast<uint4*>(grow + sp.head);
  if (t == a.ignore_index) {          // zero loss, zero gradient row, row never read
    if (tid == 0) row_ignored(a, r);
    if (tid < sp.n_scalar) store1(grow + scalar_index(sp, tid), 0.f);
    for (int j = tid; j < nvec; j += kCeThreads) gbody[j] = uint4{0u, 0u, 0u, 0u};
    return;
  }
  // pass 1: statistics, the cached vectors all requested up front
  RowStats st{-INFINITY, 0.f, 0.f};
  if (tid < sp.n_scalar) {
    float z[1] = {softcapped(ld_elem(row, scalar_index(sp, tid)), a.softcap, a.inv_softcap, kSoftcap)};
    stats_add<1, kSumZ>(st, z);
  }
  uint4 cache[kCeCache];
#pragma unroll
  for (int c = 0; c < kCeCache; ++c) {
    const int j = tid + c * kCeThreads;
    cache[c] = j < nvec ? body[j] : uint4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int c = 0; c < kCeCache; ++c) {
    if (tid + c * kCeThreads < nvec) {
      float z[kVec];
      CeVec<T>::unpack(opaque(cache[c]), z);
      if (kSoftcap) {
#pragma unroll
        for (int i = 0; i < kVec; ++i) z[i] = softcapped(z[i], a.softcap, a.inv_softcap, true);
      }
      stats_add<kVec, kSumZ>(st, z);
    }
  }
  for (int j = tid + kCeCache * kCeThreads; j < nvec; j += kCeThreads) {
    float z[kVec];
    CeVec<T>::unpack(body[j], z);
    if (kSoftcap) {
#pragma unroll
      for (int i = 0; i < kVec; ++i) z[i] = softcapped(z[i], a.softcap, a.inv_softcap, true);
    }
    stats_add<kVec, kSumZ>(st, z);
  }
  st = block_stats<kWaves>(st, sm);
  if (tid == 0) sm[3 * kWaves] = row_finish<T, kSoftcap>(a, row, r, t, st);
  __syncthreads();
  // pass 2: gradient; each thread overwrites only elements it has read, so
  // the output may be the logits themselves
  const float lse = sm[3 * kWaves];
  const float lse2 = lse * kLog2e, zfac = 1.f + a.two_s * lse, scale = a.ctl->scale;
  const int t_rel = t - static_cast<int>(sp.head);    // target's offset in the body
  if (tid < sp.n_scalar) {
    const int64_t e = scalar_index(sp, tid);
    store1(grow + e, ce_grad<kSoftcap>(ld_elem(row, e), e == t, lse2, zfac, scale, a.keep_target,
                                       a.eps_over_v, a.softcap, a.inv_softcap));
  }
  auto grad_vec = [&](const uint4& raw, int j) {
    float z[kVec];
    CeVec<T>::unpack(raw, z);
    const int e0 = j * kVec;
#pragma unroll
    for (int i = 0; i < kVec; ++i)
      z[i] = ce_grad<kSoftcap>(z[i], e0 + i == t_rel, lse2, zfac, scale, a.keep_target, a.eps_over_v,
                               a.softcap, a.inv_softcap);
    CeVec<T>::store(reinterpret_cast<T*>(gbody + j), z);
  };
#pragma unroll
  for (int c = 0; c < kCeCache; ++c) {
    const int j = tid + c * kCeThreads;
    if (j < nvec) grad_vec(opaque(cache[c]), j);
  }
  for (int j = tid + kCeCache * kCeThreads; j < nvec; j += kCeThreads) grad_vec(body[j], j);
}

}  // namespace flce
