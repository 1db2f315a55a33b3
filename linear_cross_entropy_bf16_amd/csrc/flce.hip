// libflce.so: host side of the C ABI declared in include/flce.h.
//
// Validation happens entirely on the host before the first HIP call; then the
// kernels of flce_kernels.hpp are enqueued on the caller's stream in a fixed
// sequence.  The library allocates nothing: every buffer, the workspace
// included, belongs to the caller.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "flce.h"
// the small kernels of flce_kernels.hpp are compiled in this file only
#define FLCE_HOST_KERNELS 1
#include "flce_launch.hpp"

namespace {

using flce::Ctl;
namespace tile = flce::tile;

constexpr int64_t kAlign = 256;
constexpr int64_t kMaxSlice = 8192;          // default backward vocabulary slice width ...
constexpr int64_t kSliceBytes = 1ll << 30;   // ... shrunk until one G slice fits in 1 GiB.
// Every slice re-reads and re-writes the fp32 dX accumulator, so wider slices
// cut that traffic: at 65536 x 4096 x 128256 a 8192-wide slice (G and G^T
// 1 GiB each) makes the step 4.5% faster than 4096, 16384 only 1% more.
constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
// Output tiles per raster group along the token dimension: consecutive
// workgroups on one XCD share W tiles in that XCD's L2.  Measured at
// 65536 x 4096 x 128256 on one box: the G kernel is fastest with 4 (8: 2.7%
// slower; 16 and 32 far slower), the forward with 8 (1.8% faster than 4).
constexpr int kRasterGroup = 4;
constexpr int kFwdRasterGroup = 8;
// Extra elements in the row pitch of the backward's internal K-major buffers.
// A 256-row slab read with a pitch of a large power of two (N = 65536 tokens:
// 128 KiB) lands on few L2 channels; 256 more bytes per row spread it (the
// weight-gradient GEMM at 4096 x 4096 x 65536 runs 12% faster).
constexpr int64_t kPitchPad = 128;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// blocks of the target scan and the bytes of their partials
int64_t prep_blocks(int64_t n) { return n > 0 ? cdiv(n, flce::kPrepRows) : 1; }
int64_t prep_bytes(int64_t n) { return prep_blocks(n) * static_cast<int64_t>(sizeof(flce::PrepPart)); }

// ----------------------------------------------------------------- layout
struct Layout {
  int64_t elem;           // bytes per X/W element
  int64_t v_tiles, n_tiles, tiles_per_chunk, n_chunks;
  int64_t v_full, main_chunks;   // whole vocabulary tiles; chunks of the unmasked launch
  int64_t slice, ldg;     // backward slice width (multiple of 256) and G row pitch
  int64_t chunk, n_tok_chunks;   // backward token chunk (multiple of 256) and their count
  int64_t ldt;            // token pitch of X^T and G^T (chunk, plus kPitchPad)
  int64_t n_merge_blocks;
  // byte offsets from the workspace base
  int64_t ctl, prep, rows, tc, xc;   // shared by forward and backward
  int64_t zt, part_m, part_d, part_s, block_sums;
  int64_t part_b, part_i, pred, hits, hit_sums, fwd_end;   // predicted tokens / accuracy
  int64_t g, gt, xt, wt, dx_acc, lsep, bwd_end;
};

Layout make_layout(const flce_params& p) {
  Layout L{};
  L.elem = p.dtype == FLCE_DTYPE_BF16 ? 2 : 4;
  L.v_tiles = cdiv(p.v, tile::kM);
  L.n_tiles = cdiv(p.n, tile::kN);
  // Enough workgroups to fill 256 CUs several times over, and at most 4
  // vocabulary tiles per workgroup so the partials stay small (measured at
  // 65536 x 4096 x 128256: 1, 2, 4 and 8 tiles per workgroup lie within 4%,
  // 4 is the fastest).
  const int64_t tiles = L.v_tiles * L.n_tiles;
  int64_t tpc = tiles / 4096;
  tpc = tpc < 1 ? 1 : (tpc > 4 ? 4 : tpc);
  L.tiles_per_chunk = tpc;
  // Whole vocabulary tiles go to one launch; a partial last tile (V mod 256
  // rows) gets its own chunk and launch.
  L.v_full = p.v / tile::kM;
  L.main_chunks = cdiv(L.v_full, tpc);
  L.n_chunks = L.main_chunks + (L.v_full < L.v_tiles ? 1 : 0);
  int64_t slice = p.vocab_slice;
  if (slice <= 0) {
    slice = kMaxSlice;
    while (slice > tile::kM && p.n * slice * L.elem > kSliceBytes) slice /= 2;
  }
  L.slice = round_up(slice < p.v ? slice : p.v, tile::kM);
  L.ldg = L.slice + kPitchPad;
  // the backward works on at most `chunk` packed rows at a time; one chunk
  // (the whole batch) unless params.token_chunk asks for less
  const int64_t all = round_up(p.n > 0 ? p.n : 1, tile::kN);
  L.chunk = p.token_chunk > 0 ? round_up(p.token_chunk, tile::kN) : all;
  if (L.chunk > all) L.chunk = all;
  L.n_tok_chunks = p.n > 0 ? cdiv(p.n, L.chunk) : 1;
  L.ldt = L.chunk + kPitchPad;
  L.n_merge_blocks = cdiv(p.n, 256);

  int64_t off = 0;
  L.ctl = off;
  off += kAlign;
  L.prep = off;        off = round_up(off + prep_bytes(p.n), kAlign);
  // valid rows packed to the front: row map, targets and rows of X
  L.rows = off;        off = round_up(off + 4 * p.n, kAlign);
  L.tc = off;          off = round_up(off + 4 * p.n, kAlign);
  L.xc = off;          off = round_up(off + L.elem * p.n * p.d, kAlign);
  const int64_t base = off;
  L.zt = off;          off = round_up(off + 4 * p.n, kAlign);
  L.part_m = off;      off = round_up(off + 4 * p.n * L.n_chunks, kAlign);
  L.part_d = off;      off = round_up(off + 4 * p.n * L.n_chunks, kAlign);
  L.part_s = off;      off = round_up(off + 4 * p.n * L.n_chunks, kAlign);
  L.block_sums = off;  off = round_up(off + 8 * L.n_merge_blocks, kAlign);
  L.part_b = off;      off = round_up(off + 4 * p.n * L.n_chunks, kAlign);
  L.part_i = off;      off = round_up(off + 4 * p.n * L.n_chunks, kAlign);
  L.pred = off;        off = round_up(off + 4 * p.n, kAlign);
  L.hits = off;        off = round_up(off + 4 * p.n, kAlign);
  L.hit_sums = off;    off = round_up(off + 8 * L.n_merge_blocks, kAlign);
  L.fwd_end = off;
  // Backward region reuses the forward region (the forward's scratch is dead
  // once its loss is reduced).
  off = base;
  L.g = off;           off = round_up(off + L.elem * L.chunk * L.ldg, kAlign);
  L.gt = off;          off = round_up(off + L.elem * L.ldg * L.ldt, kAlign);
  L.xt = off;          off = round_up(off + L.elem * p.d * L.ldt, kAlign);
  L.wt = off;          off = round_up(off + L.elem * p.d * L.ldg, kAlign);
  const bool multi_slice = L.slice < p.v;
  L.dx_acc = off;   // one fp32 256 x 256 block per (token tile, d tile) of a chunk, in accumulator order
  if (multi_slice) off = round_up(off + 4 * L.chunk * round_up(p.d, tile::kM), kAlign);
  L.lsep = off;        off = round_up(off + 4 * p.n, kAlign);
  L.bwd_end = off;
  return L;
}

// ----------------------------------------------------------------- checks
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

flce_status check_shape(const flce_params* p) {
  if (!p) return FLCE_ERR_INVALID_ARGUMENT;
  if (p->n < 0 || p->n > kMaxDim) return FLCE_ERR_INVALID_ARGUMENT;
  if (p->d <= 0 || p->d > kMaxDim || p->d % 8 != 0) return FLCE_ERR_INVALID_ARGUMENT;
  if (p->v <= 0 || p->v > kMaxDim) return FLCE_ERR_INVALID_ARGUMENT;
  if (p->dtype != FLCE_DTYPE_BF16 && p->dtype != FLCE_DTYPE_F32) return FLCE_ERR_INVALID_ARGUMENT;
  if (p->reduction != FLCE_REDUCTION_MEAN && p->reduction != FLCE_REDUCTION_SUM &&
      p->reduction != FLCE_REDUCTION_NONE)
    return FLCE_ERR_INVALID_ARGUMENT;
  if (!(p->label_smoothing >= 0.f && p->label_smoothing <= 1.f)) return FLCE_ERR_INVALID_ARGUMENT;
  if (!(p->lse_square_scale >= 0.f) || !std::isfinite(p->lse_square_scale))
    return FLCE_ERR_INVALID_ARGUMENT;
  if (!(p->softcap >= 0.f) || !std::isfinite(p->softcap)) return FLCE_ERR_INVALID_ARGUMENT;
  if (p->vocab_slice < 0 || p->vocab_slice > (1 << 20)) return FLCE_ERR_INVALID_ARGUMENT;
  if (p->token_chunk < 0 || p->token_chunk > (1 << 22)) return FLCE_ERR_INVALID_ARGUMENT;
  if (p->dw_bf16 != 0 && p->dw_bf16 != 1) return FLCE_ERR_INVALID_ARGUMENT;
  if (p->class_weight && !aligned(p->class_weight, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  // per-tile buffer offsets are 32-bit: 256 rows of the widest K-major operand
  if (p->d > (1 << 20) || p->n > (1 << 22)) return FLCE_ERR_INVALID_ARGUMENT;
  // byte sizes of the largest tensors must fit comfortably in int64
  const double big = static_cast<double>(p->n) * static_cast<double>(p->v) + p->n * (double)p->d +
                     p->v * (double)p->d;
  if (big > 1e17) return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

// The fused path's launch grids fit in 31 bits; the largest is the forward's,
// one workgroup per token tile and vocabulary chunk (at most one per tile).
flce_status check_params(const flce_params* p) {
  const flce_status st = check_shape(p);
  if (st != FLCE_OK) return st;
  if (cdiv(p->n, 256) * cdiv(p->v, 256) > (int64_t{1} << 31) - 8) return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

// The bf16 tile engine addresses a 256-row slab of a K-major operand with
// 32-bit buffer offsets: row * pitch * 2 + 112 must stay below 2^31 for every
// row < 256 (rows past the operand use the out-of-range marker 2^31).  The
// library's own K-major buffers have pitches slice + 128 (G), N or the token
// chunk + 128 (X^T, G^T), and V rounded up to 256, + 128 (the stored-logits
// schedule's G and W^T); X and W have pitch D <= 2^20.
bool pitch_ok(const flce_params& p, int64_t pitch) {
  return p.dtype != FLCE_DTYPE_BF16 || 255 * pitch * 2 + 112 < (int64_t{1} << 31);
}

flce_status check_inputs(const flce_params& p, const void* x, const void* w, const void* bias,
                         const int32_t* targets) {
  if (!w || !aligned(w, 16)) return FLCE_ERR_INVALID_ARGUMENT;
  if (p.n > 0 && (!x || !aligned(x, 16) || !targets || !aligned(targets, 4)))
    return FLCE_ERR_INVALID_ARGUMENT;
  if (bias && !aligned(bias, 16)) return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

flce_status check_ws(const void* ws, size_t ws_bytes, int64_t need) {
  if (!ws || !aligned(ws, kAlign)) return FLCE_ERR_INVALID_ARGUMENT;
  if (static_cast<int64_t>(ws_bytes) < need) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  return FLCE_OK;
}

// The kernels are gfx950 code objects only.
flce_status check_device() {
  // per device: 0 unknown, 1 gfx950, 2 other (calls from several threads may
  // race to fill an entry; they all store the same value)
  static std::atomic<int> known[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FLCE_ERR_DEVICE;
  const int k = dev >= 0 && dev < 64 ? known[dev].load(std::memory_order_relaxed) : 0;
  if (k) return k == 1 ? FLCE_OK : FLCE_ERR_UNSUPPORTED;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FLCE_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) known[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FLCE_OK : FLCE_ERR_UNSUPPORTED;
}

// Last check before an entry point's launches: the device, then a reset of
// the thread's pending HIP error, so that launched() reports only the
// failures of this call's own launches.
flce_status ready_to_launch() {
  const flce_status st = check_device();
  if (st == FLCE_OK) (void)hipGetLastError();
  return st;
}

flce_status launched() { return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_DEVICE; }

char* at(void* ws, int64_t off) { return static_cast<char*>(ws) + off; }

// Work-queue counters in the control block, after the Ctl fields: the forward
// launches' (take_item) in bytes 64..127, the backward's (claim_tile: G
// launches 128..159, dX launches 160..191).
static_assert(sizeof(flce::Ctl) <= 64, "Ctl overlaps the queue counters");
static_assert(192 <= kAlign, "queue counters exceed the control block");
int32_t* fwd_queue(void* ws, const Layout& L) { return reinterpret_cast<int32_t*>(at(ws, L.ctl + 64)); }
int32_t* bwd_queue(void* ws, const Layout& L) { return reinterpret_cast<int32_t*>(at(ws, L.ctl + 128)); }

// 16 counters back to zero (one block of 16 threads).
__global__ void k_zero16(int32_t* q) { q[threadIdx.x] = 0; }

void fill(float* p, int64_t count, float value, hipStream_t s) {
  if (count <= 0) return;
  hipLaunchKernelGGL(flce::k_fill, dim3(static_cast<unsigned>(cdiv(count, 256))), dim3(256), 0, s,
                     p, count, value);
}

int64_t grid8(int64_t tiles) { return round_up(tiles, 8); }

// Target scan: range check, the ordered map of the valid rows, n_valid, the
// class-weight sums and the gradient scale in the control block.
void prep(const flce_params& p, void* ws, int64_t ctl_off, int64_t prep_off, int64_t rows_off,
          const int32_t* targets, const float* grad_output, const float* weight, hipStream_t s) {
  const unsigned nb = static_cast<unsigned>(prep_blocks(p.n));
  auto* part = reinterpret_cast<flce::PrepPart*>(at(ws, prep_off));
  hipLaunchKernelGGL(flce::k_prep_count, dim3(nb), dim3(flce::kPrepRows), 0, s, targets, p.n, p.v,
                     p.ignore_index, weight, part);
  hipLaunchKernelGGL(flce::k_prep_scatter, dim3(nb), dim3(flce::kPrepRows), 0, s, targets, p.n, p.v,
                     p.ignore_index, grad_output, p.reduction == FLCE_REDUCTION_MEAN ? 1 : 0, weight,
                     static_cast<const flce::PrepPart*>(part), reinterpret_cast<Ctl*>(at(ws, ctl_off)),
                     reinterpret_cast<int32_t*>(at(ws, rows_off)));
}

// ----------------------------------------------------------------- scratch
// Device memory for callers that cannot allocate any (code under HIP graph
// capture, serving loops or harnesses that forbid hipMalloc): a fixed array in
// this library's code object, used by flce_fused_fwd_bwd_noalloc in place of
// the caller's workspace.  Every GPU that loads the library holds its own copy
// until the process ends.  In host code `scratch` names only a host-side
// stand-in; its device address is looked up once per device (with that device
// current) and only that address is handed to kernels.  The fused path writes
// every byte of its workspace before reading it, so the array needs no
// clearing between calls; calls that overlap on one GPU share it and race.
constexpr size_t kScratchBytes = size_t{128} << 20;   // 128 MiB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mutex;
void* scratch_ptr[64];                                 // per device ordinal

flce_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FLCE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FLCE_ERR_DEVICE;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return FLCE_OK;
}

// ----------------------------------------------------------------- forward
flce::FwdGrid fwd_grid(const Layout& L) {
  return flce::FwdGrid{L.n_tiles, L.v_full, L.v_tiles, L.main_chunks, L.tiles_per_chunk};
}

// key: bit 0 bias, bit 1 softcap, bit 2 sum of z (label smoothing)
template <typename T>
void dispatch_fwd(const flce::FwdArgs<T>& a, const flce::FwdGrid& g, int key, flce::FwdMode mode,
                  hipStream_t s) {
  switch (key) {
    case 0: flce::launch_fwd<T, 0>(a, g, mode, s); break;
    case 1: flce::launch_fwd<T, 1>(a, g, mode, s); break;
    case 2: flce::launch_fwd<T, 2>(a, g, mode, s); break;
    case 3: flce::launch_fwd<T, 3>(a, g, mode, s); break;
    case 4: flce::launch_fwd<T, 4>(a, g, mode, s); break;
    case 5: flce::launch_fwd<T, 5>(a, g, mode, s); break;
    case 6: flce::launch_fwd<T, 6>(a, g, mode, s); break;
    default: flce::launch_fwd<T, 7>(a, g, mode, s); break;
  }
}

// pred / accuracy: predicted tokens and token accuracy (either may be null;
// both null is the plain forward).
template <typename T>
flce_status run_forward(const flce_params& p, const Layout& L, const void* x, const void* w,
                        const void* bias, const int32_t* targets, float* loss, float* lse,
                        float* row_loss, void* ws, hipStream_t s, int32_t* pred = nullptr,
                        float* accuracy = nullptr) {
  const bool metrics = pred != nullptr || accuracy != nullptr;
  Ctl* ctl = reinterpret_cast<Ctl*>(at(ws, L.ctl));
  const bool mean = p.reduction == FLCE_REDUCTION_MEAN;
  int32_t* rows = reinterpret_cast<int32_t*>(at(ws, L.rows));
  int32_t* tc = reinterpret_cast<int32_t*>(at(ws, L.tc));
  T* xc = reinterpret_cast<T*>(at(ws, L.xc));
  prep(p, ws, L.ctl, L.prep, L.rows, targets, nullptr, p.class_weight, s);
  if (p.n == 0) {
    if (p.reduction != FLCE_REDUCTION_NONE) fill(loss, 1, 0.f, s);
    if (accuracy) fill(accuracy, 1, 0.f, s);
    return launched();
  }
  hipLaunchKernelGGL((flce::k_gather_rows<T>), dim3(static_cast<unsigned>(p.n)), dim3(256), 0, s,
                     static_cast<const T*>(x), p.d, targets, static_cast<const int32_t*>(rows),
                     static_cast<const Ctl*>(ctl), xc, tc);
  flce::FwdArgs<T> a{};
  a.x = xc;
  a.w = static_cast<const T*>(w);
  a.bias = static_cast<const T*>(bias);
  a.targets = tc;
  a.ctl = ctl;
  a.n = p.n;
  a.d = p.d;
  a.v = p.v;
  a.softcap = p.softcap;
  a.inv_softcap = p.softcap > 0.f ? 1.0f / p.softcap : 0.f;
  a.group = kFwdRasterGroup;
  a.queue = fwd_queue(ws, L);
  a.part_m = reinterpret_cast<float*>(at(ws, L.part_m));
  a.part_d = reinterpret_cast<float*>(at(ws, L.part_d));
  a.part_s = reinterpret_cast<float*>(at(ws, L.part_s));
  a.zt = reinterpret_cast<float*>(at(ws, L.zt));
  a.part_b = reinterpret_cast<float*>(at(ws, L.part_b));
  a.part_i = reinterpret_cast<int32_t*>(at(ws, L.part_i));
  a.row0 = 0;
  a.cap = p.n;
  a.weight = p.class_weight;
  const bool b = bias != nullptr, c = p.softcap > 0.f, z = p.label_smoothing > 0.f;
  const int key = (b ? 1 : 0) | (c ? 2 : 0) | (z ? 4 : 0);
  dispatch_fwd<T>(a, fwd_grid(L), key, metrics ? flce::FwdMode::kArgmax : flce::FwdMode::kPlain, s);
  flce::MergeArgs m{};
  m.part_m = a.part_m;
  m.part_d = a.part_d;
  m.part_s = a.part_s;
  m.zt = a.zt;
  m.targets = targets;
  m.n = p.n;
  m.v = p.v;
  m.n_chunks = L.n_chunks;
  m.ignore_index = p.ignore_index;
  m.keep_target = 1.0f - p.label_smoothing;
  m.eps = p.label_smoothing;
  m.eps_over_v = static_cast<float>(static_cast<double>(p.label_smoothing) / static_cast<double>(p.v));
  m.zloss = p.lse_square_scale;
  m.lse = lse;
  m.row_loss = row_loss;
  m.loss_rows = p.reduction == FLCE_REDUCTION_NONE ? loss : nullptr;
  m.block_sums = reinterpret_cast<double*>(at(ws, L.block_sums));
  m.rows = rows;
  m.ctl = ctl;
  m.weight = p.class_weight;
  if (metrics) {
    m.part_b = a.part_b;
    m.part_i = a.part_i;
    m.pred = pred ? pred : reinterpret_cast<int32_t*>(at(ws, L.pred));
    m.hits = reinterpret_cast<float*>(at(ws, L.hits));
  }
  hipLaunchKernelGGL(flce::k_merge, dim3(static_cast<unsigned>(L.n_merge_blocks)), dim3(256), 0, s, m);
  if (p.reduction != FLCE_REDUCTION_NONE)
    hipLaunchKernelGGL(flce::k_loss_final, dim3(1), dim3(256), 0, s, m.block_sums, L.n_merge_blocks,
                       static_cast<const Ctl*>(ctl), mean ? 1 : 0, loss);
  if (accuracy) {
    double* hs = reinterpret_cast<double*>(at(ws, L.hit_sums));
    hipLaunchKernelGGL(flce::k_block_sums, dim3(static_cast<unsigned>(L.n_merge_blocks)), dim3(256), 0, s,
                       static_cast<const float*>(m.hits), p.n, hs);
    hipLaunchKernelGGL(flce::k_accuracy_final, dim3(1), dim3(256), 0, s, static_cast<const double*>(hs),
                       L.n_merge_blocks, static_cast<const Ctl*>(ctl), accuracy);
  }
  return launched();
}

// ----------------------------------------------------------------- backward
// key: bit 0 bias, bit 1 softcap, bit 2 class weights
template <typename T>
void dispatch_g(const flce::GArgs<T>& a, int64_t grid, bool bias, bool softcap, hipStream_t s) {
  switch ((bias ? 1 : 0) | (softcap ? 2 : 0) | (a.weight ? 4 : 0)) {
    case 0: flce::launch_g<T, 0>(a, grid, s); break;
    case 1: flce::launch_g<T, 1>(a, grid, s); break;
    case 2: flce::launch_g<T, 2>(a, grid, s); break;
    case 3: flce::launch_g<T, 3>(a, grid, s); break;
    case 4: flce::launch_g<T, 4>(a, grid, s); break;
    case 5: flce::launch_g<T, 5>(a, grid, s); break;
    case 6: flce::launch_g<T, 6>(a, grid, s); break;
    default: flce::launch_g<T, 7>(a, grid, s); break;
  }
}

template <typename T>
void transpose(const T* in, int64_t rows, int64_t cols, int64_t ld_in, T* out, int64_t out_rows,
               int64_t ld_out_used, int64_t ld_out, hipStream_t s, const Ctl* row_bound = nullptr,
               int64_t row0 = 0) {
  const int64_t gx = cdiv(ld_out_used, 64), gy = cdiv(out_rows, 64);
  if (gx <= 0 || gy <= 0) return;
  hipLaunchKernelGGL((flce::k_transpose<T>), dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                     dim3(256), 0, s, in, rows, cols, ld_in, out, out_rows, ld_out, row_bound, row0);
}

template <typename T, typename DW>
void run_dw(const T* xt, const T* gt, const flce_params& p, const Layout& L, int64_t v0, int64_t len,
               int64_t gcols, int64_t d_tiles, int64_t s_tiles, int64_t c0, bool accumulate,
               const Ctl* ctl, DW* dw, hipStream_t s) {
  flce::DwArgs<T, DW> wa{};
  wa.xt = xt;
  wa.gt = gt;
  wa.d = p.d;
  wa.v0 = v0;
  wa.slice_len = len;
  wa.ldt = L.ldt;
  wa.gcols = gcols;
  wa.ctl = ctl;
  wa.dw = dw;
  wa.d_tiles = d_tiles;
  wa.s_tiles = s_tiles;
  wa.row0 = c0;
  wa.cap = L.chunk;
  wa.accumulate = accumulate ? 1 : 0;
  flce::launch_dw<T, DW>(wa, grid8(d_tiles * s_tiles), s);
}

template <typename T>
flce_status run_backward(const flce_params& p, const Layout& L, const void* x, const void* w,
                         const void* bias, const int32_t* targets, const float* lse,
                         const float* grad_output, void* dx, void* dw, float* dbias, void* ws,
                         hipStream_t s, bool packed) {
  Ctl* ctl = reinterpret_cast<Ctl*>(at(ws, L.ctl));
  int32_t* rows = reinterpret_cast<int32_t*>(at(ws, L.rows));
  int32_t* tc = reinterpret_cast<int32_t*>(at(ws, L.tc));
  T* xc = reinterpret_cast<T*>(at(ws, L.xc));
  // the fused call reuses the forward's scan (grad_output 1 there as well) and packed rows
  if (!packed) {
    prep(p, ws, L.ctl, L.prep, L.rows, targets, grad_output, p.class_weight, s);
    if (p.n > 0)
      hipLaunchKernelGGL((flce::k_gather_rows<T>), dim3(static_cast<unsigned>(p.n)), dim3(256), 0, s,
                         static_cast<const T*>(x), p.d, targets, static_cast<const int32_t*>(rows),
                         static_cast<const Ctl*>(ctl), xc, tc);
  }
  T* g = reinterpret_cast<T*>(at(ws, L.g));
  T* gt = reinterpret_cast<T*>(at(ws, L.gt));
  T* xt = reinterpret_cast<T*>(at(ws, L.xt));
  T* wt = reinterpret_cast<T*>(at(ws, L.wt));
  float* dx_acc = reinterpret_cast<float*>(at(ws, L.dx_acc));
  float* lsep = reinterpret_cast<float*>(at(ws, L.lsep));
  if (p.n > 0)
    hipLaunchKernelGGL(flce::k_pack_lse, dim3(static_cast<unsigned>(cdiv(p.n, 256))), dim3(256), 0, s,
                       lse, static_cast<const int32_t*>(rows), static_cast<const Ctl*>(ctl), lsep);
  const T* W = static_cast<const T*>(w);
  const int64_t n_slices = cdiv(p.v, L.slice);
  const int64_t d_tiles = cdiv(p.d, tile::kM);
  const int64_t c_tiles = L.chunk / tile::kN;   // token tiles of a chunk (upper bound)
  const bool has_bias = bias != nullptr;
  // Tail counters of the G and dX launches: each launch's workgroup 0 zeroes
  // the other kernel's set, which runs next in stream order; the first G
  // launch's set is zeroed here.
  int32_t* q_g = bwd_queue(ws, L);
  int32_t* q_dx = q_g + 8;
  if (p.n > 0) hipLaunchKernelGGL(k_zero16, dim3(1), dim3(16), 0, s, q_g);
  // Token chunks outer, vocabulary slices inner: dX of a chunk is finished
  // within its pass; dW and db of every slice accumulate over the chunks.
  for (int64_t ci = 0; ci < L.n_tok_chunks; ++ci) {
    const int64_t c0 = ci * L.chunk;              // first packed row of the chunk
    // X^T of the chunk's packed valid rows [d][ldt], tokens past them zero
    transpose<T>(xc + c0 * p.d, L.chunk, p.d, p.d, xt, p.d, L.chunk, L.ldt, s, ctl, c0);
    for (int64_t si = 0; si < n_slices; ++si) {
      const int64_t v0 = si * L.slice;
      const int64_t len = (p.v - v0) < L.slice ? (p.v - v0) : L.slice;
      const int64_t s_tiles = cdiv(len, tile::kM);
      const int64_t gcols = s_tiles * tile::kM;
      // W^T of the slice [d][ldg], vocabulary >= len zero
      transpose<T>(W + v0 * p.d, len, p.d, p.d, wt, p.d, gcols, L.ldg, s);
      if (p.n > 0) {
        flce::GArgs<T> ga{};
        ga.x = xc + c0 * p.d;
        ga.w = W;
        ga.bias = static_cast<const T*>(bias);
        ga.targets = tc + c0;
        ga.ctl = ctl;
        ga.lsep = lsep + c0;
        ga.n = L.chunk;
        ga.row0 = c0;
        ga.d = p.d;
        ga.v = p.v;
        ga.ignore_index = p.ignore_index;
        ga.softcap = p.softcap;
        ga.inv_softcap = p.softcap > 0.f ? 1.0f / p.softcap : 0.f;
        ga.keep_target = 1.0f - p.label_smoothing;
        ga.eps_over_v = static_cast<float>(static_cast<double>(p.label_smoothing) / static_cast<double>(p.v));
        ga.two_s = 2.0f * p.lse_square_scale;
        ga.v0 = v0;
        ga.slice_len = len;
        ga.ldg = L.ldg;
        ga.ldt = L.ldt;
        ga.g = g;
        ga.gt = gt;
        ga.s_tiles = s_tiles;
        const int64_t g_grid = flce::queue_grid(c_tiles * s_tiles);   // upper bound: all rows valid
        ga.group = kRasterGroup;
        ga.weight = p.class_weight;
        ga.queue = q_g;
        ga.queue_next = q_dx;
        dispatch_g<T>(ga, g_grid, has_bias, p.softcap > 0.f, s);
      }
      if (p.dw_bf16)
        run_dw<T, uint16_t>(xt, gt, p, L, v0, len, gcols, d_tiles, s_tiles, c0, ci > 0, ctl,
                               static_cast<uint16_t*>(dw), s);
      else
        run_dw<T, float>(xt, gt, p, L, v0, len, gcols, d_tiles, s_tiles, c0, ci > 0, ctl,
                            static_cast<float*>(dw), s);
      if (p.n > 0) {
        flce::DxArgs<T> xa{};
        xa.wt = wt;
        xa.g = g;
        xa.n = L.chunk;
        xa.row0 = c0;
        xa.d = p.d;
        xa.kdim = gcols;
        xa.ldg = L.ldg;
        xa.ctl = ctl;
        xa.acc_buf = dx_acc;
        xa.rows = rows + c0;
        xa.dx = static_cast<T*>(dx);
        xa.first = si == 0;
        xa.d_tiles = d_tiles;
        xa.queue = q_dx;
        xa.queue_next = q_g;
        const int64_t x_grid = flce::queue_grid(d_tiles * c_tiles);   // upper bound: all rows valid
        flce::launch_dx<T>(xa, x_grid, si + 1 == n_slices, s);
      }
      if (has_bias)
        hipLaunchKernelGGL((flce::k_db<T>), dim3(static_cast<unsigned>(cdiv(len, 4))), dim3(256), 0, s,
                           static_cast<const T*>(gt), L.ldt, L.chunk, v0, len,
                           static_cast<const Ctl*>(ctl), dbias, c0, ci > 0 ? 1 : 0);
    }
  }
  // rows of dX with an ignored target (never written by k_dx) are zero
  if (p.n > 0)
    hipLaunchKernelGGL((flce::k_zero_ignored_rows<T>), dim3(static_cast<unsigned>(p.n)), dim3(256), 0,
                       s, static_cast<T*>(dx), p.d, targets, p.ignore_index);
  return launched();
}

// ------------------------------------------------- stored-logits variant
// Forward and backward with three contractions instead of four: each token
// chunk's raw logits are kept (fp32, register order) by the forward GEMM and
// read back by the G kernel instead of being recomputed; dX then contracts
// over the whole vocabulary at once.  6 N D V FLOPs, at the price of the
// chunk's logits in the workspace (C x V x 4 bytes).
constexpr int64_t kStoredChunk = 8192;   // default token chunk of the stored variant

struct StoredLayout {
  Layout base;             // ctl, rows, tc, xc, forward partials (shared with the other calls)
  int64_t chunk, n_tok_chunks, v_tiles, vpad, ldg, ldt;
  int64_t zs, g, gt, xt, wt, lsep, end;
};

StoredLayout make_stored_layout(const flce_params& p) {
  StoredLayout S{};
  S.base = make_layout(p);
  const Layout& L = S.base;
  const int64_t all = round_up(p.n > 0 ? p.n : 1, tile::kN);
  S.chunk = round_up(p.token_chunk > 0 ? p.token_chunk : kStoredChunk, tile::kN);
  if (S.chunk > all) S.chunk = all;
  S.n_tok_chunks = p.n > 0 ? cdiv(p.n, S.chunk) : 1;
  S.v_tiles = L.v_tiles;
  S.vpad = L.v_tiles * tile::kM;
  S.ldg = S.vpad + kPitchPad;
  S.ldt = S.chunk + kPitchPad;
  int64_t off = L.fwd_end;
  S.zs = off;    off = round_up(off + 4 * S.chunk * S.vpad, kAlign);
  S.g = off;     off = round_up(off + L.elem * S.chunk * S.ldg, kAlign);
  S.gt = off;    off = round_up(off + L.elem * S.vpad * S.ldt, kAlign);
  S.xt = off;    off = round_up(off + L.elem * p.d * S.ldt, kAlign);
  S.wt = off;    off = round_up(off + L.elem * p.d * S.ldg, kAlign);
  S.lsep = off;  off = round_up(off + 4 * p.n, kAlign);
  S.end = off;
  return S;
}

template <typename T>
flce_status run_fused_stored(const flce_params& p, const StoredLayout& S, const void* x, const void* w,
                             const void* bias, const int32_t* targets, float* loss, float* lse, void* dx,
                             void* dw, float* dbias, void* ws, hipStream_t s) {
  const Layout& L = S.base;
  Ctl* ctl = reinterpret_cast<Ctl*>(at(ws, L.ctl));
  const bool mean = p.reduction == FLCE_REDUCTION_MEAN;
  int32_t* rows = reinterpret_cast<int32_t*>(at(ws, L.rows));
  int32_t* tc = reinterpret_cast<int32_t*>(at(ws, L.tc));
  T* xc = reinterpret_cast<T*>(at(ws, L.xc));
  float* zs = reinterpret_cast<float*>(at(ws, S.zs));
  T* g = reinterpret_cast<T*>(at(ws, S.g));
  T* gt = reinterpret_cast<T*>(at(ws, S.gt));
  T* xt = reinterpret_cast<T*>(at(ws, S.xt));
  T* wt = reinterpret_cast<T*>(at(ws, S.wt));
  float* lsep = reinterpret_cast<float*>(at(ws, S.lsep));
  const T* W = static_cast<const T*>(w);
  prep(p, ws, L.ctl, L.prep, L.rows, targets, nullptr, p.class_weight, s);
  if (p.n > 0)
    hipLaunchKernelGGL((flce::k_gather_rows<T>), dim3(static_cast<unsigned>(p.n)), dim3(256), 0, s,
                       static_cast<const T*>(x), p.d, targets, static_cast<const int32_t*>(rows),
                       static_cast<const Ctl*>(ctl), xc, tc);
  // W^T of the whole vocabulary [d][ldg], once
  transpose<T>(W, p.v, p.d, p.d, wt, p.d, S.vpad, S.ldg, s);
  const int64_t d_tiles = cdiv(p.d, tile::kM);
  const int64_t c_tiles = S.chunk / tile::kN;
  const bool has_bias = bias != nullptr, c = p.softcap > 0.f, z = p.label_smoothing > 0.f;
  const int fkey = (has_bias ? 1 : 0) | (c ? 2 : 0) | (z ? 4 : 0);
  double* block_sums = reinterpret_cast<double*>(at(ws, L.block_sums));
  for (int64_t ci = 0; ci < S.n_tok_chunks; ++ci) {
    const int64_t c0 = ci * S.chunk;
    if (p.n > 0) {
      // forward of the chunk, keeping its raw logits
      flce::FwdArgs<T> a{};
      a.x = xc + c0 * p.d;
      a.w = W;
      a.bias = static_cast<const T*>(bias);
      a.targets = tc + c0;
      a.ctl = ctl;
      a.n = p.n;
      a.d = p.d;
      a.v = p.v;
      a.softcap = p.softcap;
      a.inv_softcap = p.softcap > 0.f ? 1.0f / p.softcap : 0.f;
      a.group = kFwdRasterGroup;
      a.queue = fwd_queue(ws, L);
      a.part_m = reinterpret_cast<float*>(at(ws, L.part_m)) + c0;
      a.part_d = reinterpret_cast<float*>(at(ws, L.part_d)) + c0;
      a.part_s = reinterpret_cast<float*>(at(ws, L.part_s)) + c0;
      a.zt = reinterpret_cast<float*>(at(ws, L.zt)) + c0;
      a.row0 = c0;
      a.cap = S.chunk;
      a.zs = zs;
      a.zs_vt = S.v_tiles;
      a.weight = p.class_weight;
      Layout Lc = L;                     // the chunk's token tiles only
      Lc.n_tiles = c_tiles;
      dispatch_fwd<T>(a, fwd_grid(Lc), fkey, flce::FwdMode::kStore, s);
      // lse, packed lse and row losses of the chunk's rows
      flce::MergeArgs m{};
      m.part_m = reinterpret_cast<float*>(at(ws, L.part_m));
      m.part_d = reinterpret_cast<float*>(at(ws, L.part_d));
      m.part_s = reinterpret_cast<float*>(at(ws, L.part_s));
      m.zt = reinterpret_cast<float*>(at(ws, L.zt));
      m.targets = targets;
      m.n = p.n;
      m.v = p.v;
      m.n_chunks = L.n_chunks;
      m.ignore_index = p.ignore_index;
      m.keep_target = 1.0f - p.label_smoothing;
      m.eps = p.label_smoothing;
      m.eps_over_v = static_cast<float>(static_cast<double>(p.label_smoothing) / static_cast<double>(p.v));
      m.zloss = p.lse_square_scale;
      m.lse = lse;
      m.block_sums = block_sums;
      m.rows = rows;
      m.ctl = ctl;
      m.row0 = c0;
      m.lsep = lsep;
      m.weight = p.class_weight;
      hipLaunchKernelGGL(flce::k_merge, dim3(static_cast<unsigned>(c_tiles)), dim3(256), 0, s, m);
      // G of the chunk over the whole vocabulary, from the kept logits
      flce::GArgs<T> ga{};
      ga.x = xc + c0 * p.d;
      ga.w = W;
      ga.bias = static_cast<const T*>(bias);
      ga.targets = tc + c0;
      ga.ctl = ctl;
      ga.lsep = lsep + c0;
      ga.n = S.chunk;
      ga.row0 = c0;
      ga.d = p.d;
      ga.v = p.v;
      ga.ignore_index = p.ignore_index;
      ga.softcap = p.softcap;
      ga.inv_softcap = a.inv_softcap;
      ga.keep_target = m.keep_target;
      ga.eps_over_v = m.eps_over_v;
      ga.two_s = 2.0f * p.lse_square_scale;
      ga.v0 = 0;
      ga.slice_len = p.v;
      ga.ldg = S.ldg;
      ga.ldt = S.ldt;
      ga.g = g;
      ga.gt = gt;
      ga.s_tiles = S.v_tiles;
      ga.group = kRasterGroup;
      ga.zs = zs;
      ga.zs_vt = S.v_tiles;
      const int64_t g_grid = grid8(c_tiles * S.v_tiles);
      ga.weight = p.class_weight;
      dispatch_g<T>(ga, g_grid, has_bias, c, s);
    }
    // X^T of the chunk; dW over the whole vocabulary, accumulated over chunks
    transpose<T>(xc + c0 * p.d, S.chunk, p.d, p.d, xt, p.d, S.chunk, S.ldt, s, ctl, c0);
    Layout Lw = L;
    Lw.ldt = S.ldt;
    Lw.chunk = S.chunk;
    if (p.dw_bf16)
      run_dw<T, uint16_t>(xt, gt, p, Lw, 0, p.v, S.vpad, d_tiles, S.v_tiles, c0, ci > 0, ctl,
                             static_cast<uint16_t*>(dw), s);
    else
      run_dw<T, float>(xt, gt, p, Lw, 0, p.v, S.vpad, d_tiles, S.v_tiles, c0, ci > 0, ctl,
                          static_cast<float*>(dw), s);
    if (p.n > 0) {
      // dX of the chunk in one contraction over the whole vocabulary
      flce::DxArgs<T> xa{};
      xa.wt = wt;
      xa.g = g;
      xa.n = S.chunk;
      xa.row0 = c0;
      xa.d = p.d;
      xa.kdim = S.vpad;
      xa.ldg = S.ldg;
      xa.ctl = ctl;
      xa.acc_buf = nullptr;              // first and last slice: no running sum
      xa.rows = rows + c0;
      xa.dx = static_cast<T*>(dx);
      xa.first = 1;
      xa.d_tiles = d_tiles;
      flce::launch_dx<T>(xa, grid8(d_tiles * c_tiles), true, s);
    }
    if (has_bias)
      hipLaunchKernelGGL((flce::k_db<T>), dim3(static_cast<unsigned>(cdiv(p.v, 4))), dim3(256), 0, s,
                         static_cast<const T*>(gt), S.ldt, S.chunk, int64_t{0}, p.v,
                         static_cast<const Ctl*>(ctl), dbias, c0, ci > 0 ? 1 : 0);
  }
  if (p.n == 0) {
    fill(loss, 1, 0.f, s);
    return launched();
  }
  hipLaunchKernelGGL(flce::k_loss_final, dim3(1), dim3(256), 0, s, static_cast<const double*>(block_sums),
                     L.n_merge_blocks, static_cast<const Ctl*>(ctl), mean ? 1 : 0, loss);
  hipLaunchKernelGGL((flce::k_zero_ignored_rows<T>), dim3(static_cast<unsigned>(p.n)), dim3(256), 0, s,
                     static_cast<T*>(dx), p.d, targets, p.ignore_index);
  return launched();
}

// ------------------------------------------------- cross-entropy on logits
struct CeLayout {
  int64_t elem;
  int64_t ctl, prep, rows, row_loss, block_sums, pred, hits, hit_sums, end;
  int64_t n_blocks;
};

CeLayout make_ce_layout(const flce_params& p) {
  CeLayout L{};
  L.elem = p.dtype == FLCE_DTYPE_BF16 ? 2 : 4;
  L.n_blocks = cdiv(p.n, 256);
  int64_t off = 0;
  L.ctl = off;         off += kAlign;
  L.prep = off;        off = round_up(off + prep_bytes(p.n), kAlign);
  L.rows = off;        off = round_up(off + 4 * p.n, kAlign);
  L.row_loss = off;    off = round_up(off + 4 * p.n, kAlign);
  L.block_sums = off;  off = round_up(off + 8 * L.n_blocks, kAlign);
  L.pred = off;        off = round_up(off + 4 * p.n, kAlign);
  L.hits = off;        off = round_up(off + 4 * p.n, kAlign);
  L.hit_sums = off;    off = round_up(off + 8 * L.n_blocks, kAlign);
  L.end = off;
  return L;
}

// flce_params without the hidden size: d and vocab_slice are ignored.
flce_status check_ce_params(const flce_params* p) {
  if (!p) return FLCE_ERR_INVALID_ARGUMENT;
  flce_params q = *p;
  q.d = 8;
  q.vocab_slice = 0;
  const flce_status st = check_shape(&q);
  if (st != FLCE_OK) return st;
  if (p->class_weight) return FLCE_ERR_UNSUPPORTED;   // class weights: fused path only
  if (static_cast<double>(p->n) * static_cast<double>(p->v) > 1e17) return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

// logits and the gradient: element-aligned, and equally misaligned to 16
// bytes so both split every row the same way
flce_status check_ce_ptrs(const flce_params& p, const void* logits, const int32_t* targets,
                          const void* grad) {
  const uintptr_t e = p.dtype == FLCE_DTYPE_BF16 ? 2 : 4;
  if (p.n == 0) return FLCE_OK;
  if (!logits || !aligned(logits, e) || !targets || !aligned(targets, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if (grad && (!aligned(grad, e) || ((reinterpret_cast<uintptr_t>(grad) -
                                      reinterpret_cast<uintptr_t>(logits)) & 15u) != 0))
    return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

template <typename T>
flce::CeArgs<T> ce_args(const flce_params& p, const CeLayout& L, const void* logits,
                        const int32_t* targets, void* ws) {
  flce::CeArgs<T> a{};
  a.logits = static_cast<const T*>(logits);
  a.targets = targets;
  a.n = p.n;
  a.v = p.v;
  a.ignore_index = p.ignore_index;
  a.softcap = p.softcap;
  a.inv_softcap = p.softcap > 0.f ? 1.0f / p.softcap : 0.f;
  a.keep_target = 1.0f - p.label_smoothing;
  a.eps = p.label_smoothing;
  a.eps_over_v = static_cast<float>(static_cast<double>(p.label_smoothing) / static_cast<double>(p.v));
  a.zloss = p.lse_square_scale;
  a.two_s = 2.0f * p.lse_square_scale;
  a.ctl = reinterpret_cast<const Ctl*>(at(ws, L.ctl));
  a.row_loss_ws = reinterpret_cast<float*>(at(ws, L.row_loss));
  return a;
}

void ce_prep(const flce_params& p, const CeLayout& L, const int32_t* targets,
             const float* grad_output, void* ws, hipStream_t s) {
  prep(p, ws, L.ctl, L.prep, L.rows, targets, grad_output, nullptr, s);
}

void ce_reduce(const flce_params& p, const CeLayout& L, float* loss, void* ws, hipStream_t s) {
  if (p.reduction == FLCE_REDUCTION_NONE) return;
  double* sums = reinterpret_cast<double*>(at(ws, L.block_sums));
  if (L.n_blocks > 0)
    hipLaunchKernelGGL(flce::k_block_sums, dim3(static_cast<unsigned>(L.n_blocks)), dim3(256), 0, s,
                       static_cast<const float*>(reinterpret_cast<float*>(at(ws, L.row_loss))), p.n, sums);
  hipLaunchKernelGGL(flce::k_loss_final, dim3(1), dim3(256), 0, s, static_cast<const double*>(sums),
                     L.n_blocks, reinterpret_cast<const Ctl*>(at(ws, L.ctl)),
                     p.reduction == FLCE_REDUCTION_MEAN ? 1 : 0, loss);
}

template <typename T>
flce_status run_ce(const flce_params& p, const CeLayout& L, const void* logits, const int32_t* targets,
                   float* loss, float* lse, float* row_loss, const float* lse_in,
                   const float* grad_output, void* grad, void* ws, hipStream_t s, int mode,
                   int32_t* pred = nullptr, float* accuracy = nullptr) {
  // mode 0: forward, 1: backward, 2: fused; pred / accuracy: forward metrics
  ce_prep(p, L, targets, grad_output, ws, s);
  flce::CeArgs<T> a = ce_args<T>(p, L, logits, targets, ws);
  a.lse = lse;
  a.lse_in = lse_in;
  a.row_loss = row_loss;
  a.loss_rows = (mode == 0 && p.reduction == FLCE_REDUCTION_NONE) ? loss : nullptr;
  a.grad = static_cast<T*>(grad);
  if (pred || accuracy) {
    a.pred = pred ? pred : reinterpret_cast<int32_t*>(at(ws, L.pred));
    a.hits = reinterpret_cast<float*>(at(ws, L.hits));
  }
  const bool c = p.softcap > 0.f, z = p.label_smoothing > 0.f;
  if (p.n > 0) {
    flce::launch_ce<T>(a, mode, (c ? 1 : 0) | (z ? 2 : 0), a.pred != nullptr, s);
    if (mode == 1) return launched();
  } else if (mode == 1) {
    return launched();
  }
  ce_reduce(p, L, loss, ws, s);
  if (accuracy) {
    double* hs = reinterpret_cast<double*>(at(ws, L.hit_sums));
    if (L.n_blocks > 0)
      hipLaunchKernelGGL(flce::k_block_sums, dim3(static_cast<unsigned>(L.n_blocks)), dim3(256), 0, s,
                         static_cast<const float*>(a.hits), p.n, hs);
    hipLaunchKernelGGL(flce::k_accuracy_final, dim3(1), dim3(256), 0, s, static_cast<const double*>(hs),
                       L.n_blocks, a.ctl, accuracy);
  }
  return launched();
}

}  // namespace

// =================================================================== C ABI
extern "C" {

size_t flce_workspace_size(const flce_params* params, int with_backward) {
  if (check_params(params) != FLCE_OK) return 0;
  const Layout L = make_layout(*params);
  if (!pitch_ok(*params, L.ldg) || !pitch_ok(*params, L.ldt)) return 0;
  const int64_t need = with_backward ? (L.bwd_end > L.fwd_end ? L.bwd_end : L.fwd_end) : L.fwd_end;
  return static_cast<size_t>(need);
}

flce_status flce_forward(const flce_params* params, const void* x, const void* w, const void* bias,
                         const int32_t* targets, float* loss, float* lse, float* row_loss, void* ws,
                         size_t ws_bytes, void* stream) {
  flce_status st = check_params(params);
  if (st != FLCE_OK) return st;
  const flce_params& p = *params;
  if ((st = check_inputs(p, x, w, bias, targets)) != FLCE_OK) return st;
  if (!loss || !aligned(loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if (p.n > 0 && (!lse || !aligned(lse, 4))) return FLCE_ERR_INVALID_ARGUMENT;
  if (row_loss && !aligned(row_loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  const Layout L = make_layout(p);
  if ((st = check_ws(ws, ws_bytes, L.fwd_end)) != FLCE_OK) return st;
  if ((st = ready_to_launch()) != FLCE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.dtype == FLCE_DTYPE_BF16)
    return run_forward<uint16_t>(p, L, x, w, bias, targets, loss, lse, row_loss, ws, s);
  return run_forward<float>(p, L, x, w, bias, targets, loss, lse, row_loss, ws, s);
}

flce_status flce_forward_metrics(const flce_params* params, const void* x, const void* w,
                                 const void* bias, const int32_t* targets, float* loss, float* lse,
                                 float* row_loss, int32_t* pred, float* accuracy, void* ws,
                                 size_t ws_bytes, void* stream) {
  flce_status st = check_params(params);
  if (st != FLCE_OK) return st;
  const flce_params& p = *params;
  if ((st = check_inputs(p, x, w, bias, targets)) != FLCE_OK) return st;
  if (!loss || !aligned(loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if (p.n > 0 && (!lse || !aligned(lse, 4))) return FLCE_ERR_INVALID_ARGUMENT;
  if (row_loss && !aligned(row_loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if ((pred && !aligned(pred, 4)) || (accuracy && !aligned(accuracy, 4))) return FLCE_ERR_INVALID_ARGUMENT;
  const Layout L = make_layout(p);
  if ((st = check_ws(ws, ws_bytes, L.fwd_end)) != FLCE_OK) return st;
  if ((st = ready_to_launch()) != FLCE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.dtype == FLCE_DTYPE_BF16)
    return run_forward<uint16_t>(p, L, x, w, bias, targets, loss, lse, row_loss, ws, s, pred, accuracy);
  return run_forward<float>(p, L, x, w, bias, targets, loss, lse, row_loss, ws, s, pred, accuracy);
}

static flce_status check_backward_outputs(const flce_params& p, const Layout& L, const float* lse,
                                          void* dx, void* dw, float* dbias, const void* bias) {
  if (p.reduction == FLCE_REDUCTION_NONE) return FLCE_ERR_UNSUPPORTED;
  if (p.n > 0 && (!lse || !aligned(lse, 4) || !dx || !aligned(dx, 16))) return FLCE_ERR_INVALID_ARGUMENT;
  if (!dw || !aligned(dw, 16)) return FLCE_ERR_INVALID_ARGUMENT;
  if (bias && (!dbias || !aligned(dbias, 4))) return FLCE_ERR_INVALID_ARGUMENT;
  if (!pitch_ok(p, L.ldg) || !pitch_ok(p, L.ldt)) return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

static flce_status check_backward_args(const flce_params& p, const Layout& L, const float* lse,
                                       void* dx, void* dw, float* dbias, const void* bias,
                                       const void* ws, size_t ws_bytes) {
  const flce_status st = check_backward_outputs(p, L, lse, dx, dw, dbias, bias);
  if (st != FLCE_OK) return st;
  const int64_t need = L.bwd_end > L.fwd_end ? L.bwd_end : L.fwd_end;
  return check_ws(ws, ws_bytes, need);
}

flce_status flce_backward(const flce_params* params, const void* x, const void* w, const void* bias,
                          const int32_t* targets, const float* lse, const float* grad_output, void* dx,
                          void* dw, float* dbias, void* ws, size_t ws_bytes, void* stream) {
  flce_status st = check_params(params);
  if (st != FLCE_OK) return st;
  const flce_params& p = *params;
  if ((st = check_inputs(p, x, w, bias, targets)) != FLCE_OK) return st;
  if (grad_output && !aligned(grad_output, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  const Layout L = make_layout(p);
  if ((st = check_backward_args(p, L, lse, dx, dw, dbias, bias, ws, ws_bytes)) != FLCE_OK) return st;
  if ((st = ready_to_launch()) != FLCE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.dtype == FLCE_DTYPE_BF16)
    return run_backward<uint16_t>(p, L, x, w, bias, targets, lse, grad_output, dx, dw, dbias, ws, s,
                                  false);
  return run_backward<float>(p, L, x, w, bias, targets, lse, grad_output, dx, dw, dbias, ws, s, false);
}

static flce_status run_fused(const flce_params& p, const Layout& L, const void* x, const void* w,
                             const void* bias, const int32_t* targets, float* loss, float* lse,
                             void* dx, void* dw, float* dbias, void* ws, hipStream_t s) {
  flce_status st;
  if (p.dtype == FLCE_DTYPE_BF16) {
    st = run_forward<uint16_t>(p, L, x, w, bias, targets, loss, lse, nullptr, ws, s);
    if (st != FLCE_OK) return st;
    return run_backward<uint16_t>(p, L, x, w, bias, targets, lse, nullptr, dx, dw, dbias, ws, s, true);
  }
  st = run_forward<float>(p, L, x, w, bias, targets, loss, lse, nullptr, ws, s);
  if (st != FLCE_OK) return st;
  return run_backward<float>(p, L, x, w, bias, targets, lse, nullptr, dx, dw, dbias, ws, s, true);
}

flce_status flce_fused_fwd_bwd(const flce_params* params, const void* x, const void* w,
                               const void* bias, const int32_t* targets, float* loss, float* lse,
                               void* dx, void* dw, float* dbias, void* ws, size_t ws_bytes,
                               void* stream) {
  flce_status st = check_params(params);
  if (st != FLCE_OK) return st;
  const flce_params& p = *params;
  if ((st = check_inputs(p, x, w, bias, targets)) != FLCE_OK) return st;
  if (!loss || !aligned(loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  const Layout L = make_layout(p);
  if ((st = check_backward_args(p, L, lse, dx, dw, dbias, bias, ws, ws_bytes)) != FLCE_OK) return st;
  if ((st = ready_to_launch()) != FLCE_OK) return st;
  return run_fused(p, L, x, w, bias, targets, loss, lse, dx, dw, dbias, ws, static_cast<hipStream_t>(stream));
}

flce_status flce_fused_fwd_bwd_noalloc(const flce_params* params, const void* x, const void* w,
                                       const void* bias, const int32_t* targets, float* loss,
                                       float* lse, void* dx, void* dw, float* dbias, void* stream) {
  flce_status st = check_params(params);
  if (st != FLCE_OK) return st;
  const flce_params& p = *params;
  if ((st = check_inputs(p, x, w, bias, targets)) != FLCE_OK) return st;
  if (!loss || !aligned(loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  const Layout L = make_layout(p);
  if ((st = check_backward_outputs(p, L, lse, dx, dw, dbias, bias)) != FLCE_OK) return st;
  const int64_t need = L.bwd_end > L.fwd_end ? L.bwd_end : L.fwd_end;
  if (need > static_cast<int64_t>(kScratchBytes)) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device()) != FLCE_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != FLCE_OK) return st;
  if ((st = ready_to_launch()) != FLCE_OK) return st;
  return run_fused(p, L, x, w, bias, targets, loss, lse, dx, dw, dbias, ws, static_cast<hipStream_t>(stream));
}

size_t flce_stored_workspace_size(const flce_params* params) {
  if (check_params(params) != FLCE_OK) return 0;
  const StoredLayout S = make_stored_layout(*params);
  if (!pitch_ok(*params, S.ldg) || !pitch_ok(*params, S.ldt)) return 0;
  return static_cast<size_t>(S.end);
}

flce_status flce_fused_fwd_bwd_stored(const flce_params* params, const void* x, const void* w,
                                      const void* bias, const int32_t* targets, float* loss, float* lse,
                                      void* dx, void* dw, float* dbias, void* ws, size_t ws_bytes,
                                      void* stream) {
  flce_status st = check_params(params);
  if (st != FLCE_OK) return st;
  const flce_params& p = *params;
  if ((st = check_inputs(p, x, w, bias, targets)) != FLCE_OK) return st;
  if (!loss || !aligned(loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if (p.reduction == FLCE_REDUCTION_NONE) return FLCE_ERR_UNSUPPORTED;
  if (p.n > 0 && (!lse || !aligned(lse, 4) || !dx || !aligned(dx, 16))) return FLCE_ERR_INVALID_ARGUMENT;
  if (!dw || !aligned(dw, 16)) return FLCE_ERR_INVALID_ARGUMENT;
  if (bias && (!dbias || !aligned(dbias, 4))) return FLCE_ERR_INVALID_ARGUMENT;
  const StoredLayout S = make_stored_layout(p);
  if (!pitch_ok(p, S.ldg) || !pitch_ok(p, S.ldt)) return FLCE_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(ws, ws_bytes, S.end)) != FLCE_OK) return st;
  if ((st = ready_to_launch()) != FLCE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.dtype == FLCE_DTYPE_BF16)
    return run_fused_stored<uint16_t>(p, S, x, w, bias, targets, loss, lse, dx, dw, dbias, ws, s);
  return run_fused_stored<float>(p, S, x, w, bias, targets, loss, lse, dx, dw, dbias, ws, s);
}

flce_status flce_check_status(const void* ws, void* stream) {
  if (!ws || !aligned(ws, kAlign)) return FLCE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return FLCE_ERR_DEVICE;
  Ctl host{};
  if (hipMemcpy(&host, ws, sizeof(Ctl), hipMemcpyDeviceToHost) != hipSuccess) return FLCE_ERR_DEVICE;
  return host.status ? FLCE_ERR_TARGET_OUT_OF_RANGE : FLCE_OK;
}

size_t flce_ce_workspace_size(const flce_params* params) {
  if (check_ce_params(params) != FLCE_OK) return 0;
  return static_cast<size_t>(make_ce_layout(*params).end);
}

flce_status flce_ce_forward(const flce_params* params, const void* logits, const int32_t* targets,
                            float* loss, float* lse, float* row_loss, void* ws, size_t ws_bytes,
                            void* stream) {
  flce_status st = check_ce_params(params);
  if (st != FLCE_OK) return st;
  const flce_params& p = *params;
  if ((st = check_ce_ptrs(p, logits, targets, nullptr)) != FLCE_OK) return st;
  if (!loss || !aligned(loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if (p.n > 0 && (!lse || !aligned(lse, 4))) return FLCE_ERR_INVALID_ARGUMENT;
  if (row_loss && !aligned(row_loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  const CeLayout L = make_ce_layout(p);
  if ((st = check_ws(ws, ws_bytes, L.end)) != FLCE_OK) return st;
  if ((st = ready_to_launch()) != FLCE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.dtype == FLCE_DTYPE_BF16)
    return run_ce<uint16_t>(p, L, logits, targets, loss, lse, row_loss, nullptr, nullptr, nullptr, ws, s, 0);
  return run_ce<float>(p, L, logits, targets, loss, lse, row_loss, nullptr, nullptr, nullptr, ws, s, 0);
}

flce_status flce_ce_forward_metrics(const flce_params* params, const void* logits,
                                    const int32_t* targets, float* loss, float* lse, float* row_loss,
                                    int32_t* pred, float* accuracy, void* ws, size_t ws_bytes,
                                    void* stream) {
  flce_status st = check_ce_params(params);
  if (st != FLCE_OK) return st;
  const flce_params& p = *params;
  if ((st = check_ce_ptrs(p, logits, targets, nullptr)) != FLCE_OK) return st;
  if (!loss || !aligned(loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if (p.n > 0 && (!lse || !aligned(lse, 4))) return FLCE_ERR_INVALID_ARGUMENT;
  if (row_loss && !aligned(row_loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if ((pred && !aligned(pred, 4)) || (accuracy && !aligned(accuracy, 4))) return FLCE_ERR_INVALID_ARGUMENT;
  const CeLayout L = make_ce_layout(p);
  if ((st = check_ws(ws, ws_bytes, L.end)) != FLCE_OK) return st;
  if ((st = ready_to_launch()) != FLCE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.dtype == FLCE_DTYPE_BF16)
    return run_ce<uint16_t>(p, L, logits, targets, loss, lse, row_loss, nullptr, nullptr, nullptr, ws, s, 0,
                            pred, accuracy);
  return run_ce<float>(p, L, logits, targets, loss, lse, row_loss, nullptr, nullptr, nullptr, ws, s, 0,
                       pred, accuracy);
}

flce_status flce_ce_backward(const flce_params* params, const void* logits, const int32_t* targets,
                             const float* lse, const float* grad_output, void* dlogits, void* ws,
                             size_t ws_bytes, void* stream) {
  flce_status st = check_ce_params(params);
  if (st != FLCE_OK) return st;
  const flce_params& p = *params;
  if (p.reduction == FLCE_REDUCTION_NONE) return FLCE_ERR_UNSUPPORTED;
  if (p.n > 0 && !dlogits) return FLCE_ERR_INVALID_ARGUMENT;
  if ((st = check_ce_ptrs(p, logits, targets, dlogits)) != FLCE_OK) return st;
  if (p.n > 0 && (!lse || !aligned(lse, 4))) return FLCE_ERR_INVALID_ARGUMENT;
  if (grad_output && !aligned(grad_output, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  const CeLayout L = make_ce_layout(p);
  if ((st = check_ws(ws, ws_bytes, L.end)) != FLCE_OK) return st;
  if ((st = ready_to_launch()) != FLCE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.dtype == FLCE_DTYPE_BF16)
    return run_ce<uint16_t>(p, L, logits, targets, nullptr, nullptr, nullptr, lse, grad_output, dlogits, ws,
                            s, 1);
  return run_ce<float>(p, L, logits, targets, nullptr, nullptr, nullptr, lse, grad_output, dlogits, ws, s, 1);
}

flce_status flce_ce_fused_fwd_bwd(const flce_params* params, const void* logits, const int32_t* targets,
                                  float* loss, float* lse, void* dlogits, void* ws, size_t ws_bytes,
                                  void* stream) {
  flce_status st = check_ce_params(params);
  if (st != FLCE_OK) return st;
  const flce_params& p = *params;
  if (p.reduction == FLCE_REDUCTION_NONE) return FLCE_ERR_UNSUPPORTED;
  if (p.n > 0 && !dlogits) return FLCE_ERR_INVALID_ARGUMENT;
  if ((st = check_ce_ptrs(p, logits, targets, dlogits)) != FLCE_OK) return st;
  if (!loss || !aligned(loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if (p.n > 0 && (!lse || !aligned(lse, 4))) return FLCE_ERR_INVALID_ARGUMENT;
  const CeLayout L = make_ce_layout(p);
  if ((st = check_ws(ws, ws_bytes, L.end)) != FLCE_OK) return st;
  if ((st = ready_to_launch()) != FLCE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.dtype == FLCE_DTYPE_BF16)
    return run_ce<uint16_t>(p, L, logits, targets, loss, lse, nullptr, nullptr, nullptr, dlogits, ws, s, 2);
  return run_ce<float>(p, L, logits, targets, loss, lse, nullptr, nullptr, nullptr, dlogits, ws, s, 2);
}

const char* flce_status_string(flce_status status) {
  switch (status) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FLCE_ERR_UNSUPPORTED: return "unsupported";
    case FLCE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FLCE_ERR_TARGET_OUT_OF_RANGE: return "target out of range";
    case FLCE_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

int flce_version(void) { return 10100; }

}  // extern "C"
