/*
 * flce.h - fused linear cross-entropy (FLCE) for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libflce.so.  The library computes, for hidden states X [N, D],
 * an LM-head weight W [V, D] (nn.Linear layout, i.e. the logical [D, V]
 * matrix of the page "Cutting LLM Memory by 84%: A Deep Dive into Fused
 * Kernels", section "The Logit Bottleneck", stored transposed), an optional
 * bias b [V] and int32 targets t [N]:
 *
 *   r     = X W^T + b                       (logits, never stored)
 *   z     = c tanh(r / c)   if softcap c > 0, else r
 *   lse_n = log sum_v exp(z_nv)
 *   row_n = lse_n - (1-eps) z_{n,t_n} - (eps/V) sum_v z_nv + s lse_n^2
 *   loss  = sum over valid rows of row_n, divided by n_valid for 'mean'
 *
 * Rows with t_n == ignore_index are not valid: their loss and lse are 0 and
 * their gradient rows are 0 (page "Cutting LLM Memory by 84%", "Kernel
 * Implementation", step 1).  They take no part in any contraction: the valid
 * rows are packed (in order) into the workspace first and every GEMM runs on
 * those only.  The backward recomputes softmax tiles from the
 * saved LSE and forms G = [softmax(z)(1 + 2 s lse) - (1-eps) onehot - eps/V]
 * (times 1 - (z/c)^2 under the softcap), then dX = scale G W and
 * dW = scale G^T X, db = scale sum_n G, with scale = g / n_valid ('mean') or g
 * ('sum') for the upstream gradient g (same page, "Backward Pass" and
 * "Fused Linear Cross-Entropy"; the option set follows the page
 * "[CuteDSL] FLCE: 2-SM online-softmax fast path (Blackwell)", Summary).
 * No [N, V] buffer is ever allocated: the forward keeps only per-row
 * online-softmax partials, the backward works one vocabulary slice at a time.
 *
 * Conventions for every entry point:
 *  - Device pointers are plain HIP device addresses; the caller owns every
 *    buffer, including the workspace.  The library never allocates or frees
 *    device memory and never synchronises, except flce_check_status().
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    runs asynchronously; results are valid once that stream has reached the
 *    end of the call.  Kernels run on the calling thread's current HIP
 *    device: every pointer and the stream must belong to it (hipSetDevice
 *    first when several devices are visible).
 *  - Tensors are dense row-major.  X, W, dX, bias must be 16-byte aligned;
 *    D must be a multiple of 8.  N and V are arbitrary (ragged tails are
 *    handled in the kernels).  N <= 2^22, D <= 2^20, V < 2^31, and for the
 *    fused path ceil(N/256) * ceil(V/256) < 2^31 (one forward tile each).
 *    In bf16 every K-major buffer the backward builds must have a row pitch
 *    p with 510 p + 112 < 2^31 (the tile engine's 32-bit buffer offsets):
 *    vocab_slice <= 2^20 and N <= 2^22 always satisfy it; the stored-logits
 *    schedule, whose G rows span the whole vocabulary, needs V <= 4210432.
 *  - Element type of X, W, bias and dX is params->dtype (bf16 or fp32).
 *    Loss, lse, row_loss, dW and db are always fp32.  Accumulation is fp32.
 *  - Every argument is validated on the host before any HIP call, so invalid
 *    calls return an error without touching the GPU.  Nothing aborts or
 *    throws across this interface.  Just before its launches an entry point
 *    clears the calling thread's pending HIP error (hipGetLastError), so
 *    FLCE_ERR_DEVICE reports a failure of its own launches.
 *  - Results are deterministic: every reduction has a fixed order and no
 *    value is accumulated with atomics.  The only atomics are work counters
 *    in the workspace that decide which workgroup computes which tile; a
 *    tile's result does not depend on that.
 *  - Concurrent calls that share a workspace race; give each in-flight call
 *    its own workspace.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum flce_status {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARGUMENT = 1,   /* bad size, pointer, alignment or option */
  FLCE_ERR_UNSUPPORTED = 2,        /* reduction NONE with a backward; device is not gfx950 */
  FLCE_ERR_WORKSPACE_TOO_SMALL = 3,
  FLCE_ERR_TARGET_OUT_OF_RANGE = 4,/* a target outside [0, V) that is not ignore_index
                                      (reported by flce_check_status) */
  FLCE_ERR_DEVICE = 5              /* a HIP call or kernel launch failed */
} flce_status;

typedef enum flce_dtype {
  FLCE_DTYPE_BF16 = 0,
  FLCE_DTYPE_F32 = 1
} flce_dtype;

typedef enum flce_reduction {
  FLCE_REDUCTION_MEAN = 0,         /* sum of valid row losses / n_valid (0 if n_valid == 0) */
  FLCE_REDUCTION_SUM = 1,
  FLCE_REDUCTION_NONE = 2          /* per-row losses; forward only */
} flce_reduction;

typedef struct flce_params {
  int64_t n;                 /* tokens (rows of X), >= 0 */
  int64_t d;                 /* hidden size, > 0, multiple of 8 */
  int64_t v;                 /* vocabulary size, > 0 */
  int32_t dtype;             /* flce_dtype of X, W, bias and dX */
  int32_t ignore_index;      /* rows with this target are skipped (usually -100) */
  float label_smoothing;     /* eps in [0, 1] */
  float lse_square_scale;    /* z-loss weight s >= 0 */
  float softcap;             /* c; 0 = off, > 0 caps logits to (-c, c) */
  int32_t reduction;         /* flce_reduction */
  int32_t vocab_slice;       /* backward vocabulary slice width; 0 = library default.
                                Rounded up to a multiple of 256. */
  int32_t token_chunk;       /* backward token chunk: 0 = the whole batch in one pass;
                                else the packed valid rows are processed this many at a
                                time (rounded up to 256), so the backward workspace (G
                                slices, X^T, the dX running sum) is sized by the chunk,
                                not by N, and dW / db accumulate over the chunks */
  int32_t dw_bf16;           /* 0: dW is fp32; 1: dW is bf16 (half the memory; rounded
                                once per token chunk, as it accumulates in its own dtype) */
  const float* class_weight; /* NULL, or fp32 [v] per-class weights on the device (the
                                ce_weight option of the page "[CuteDSL] FLCE", Summary),
                                with torch's weighted cross-entropy meaning: row loss
                                (1-eps) w_t (lse - z_t) + (eps/V) sum_v w_v (lse - z_v)
                                + s w_t lse^2, 'mean' divided by the valid rows' sum of
                                w_t.  Fused-path calls only; the flce_ce_* calls return
                                FLCE_ERR_UNSUPPORTED with weights. */
} flce_params;

/* Bytes of workspace the calls need for these parameters.  with_backward = 0
 * sizes flce_forward only; 1 sizes flce_backward and flce_fused_fwd_bwd (and
 * also covers flce_forward).  Returns 0 for invalid parameters.  The size is
 * O(N (V/256 + D) + C * (vocab_slice + D)), far below the N x V logits: the
 * packed valid rows of X, per-row forward partials, and for the backward one
 * G slice in both orientations, X^T and an fp32 dX accumulator, for C = N
 * tokens or the token chunk (page "Cutting LLM Memory by 84%", "Path to
 * Production": processing the tokens in blocks along N keeps the memory
 * constant in the sequence length). */
size_t flce_workspace_size(const flce_params* params, int with_backward);

/* Forward: loss and per-row LSE.  The cross-entropy of a one-hot target
 * reduces to the row's log-sum-exp minus its target logit, evaluated with the
 * running row maximum subtracted (page "Cutting LLM Memory by 84%",
 * "Definition and Forward Pass"); the logits GEMM keeps only per-row
 * online-softmax partials and the target logit, never the logits (page
 * "[CuteDSL] FLCE", Summary: a store-free forward).  The row loss is formed as
 * (m - z_t) + ln sum_v e^(z_v - m) with m the row maximum, so a confidently
 * predicted row keeps the accuracy of that sum (a few ulp of 1) whatever |z|.
 *  x        [n, d] dtype          w   [v, d] dtype        bias [v] dtype or NULL
 *  targets  [n] int32
 *  loss     fp32 [1] for MEAN/SUM, fp32 [n] (per-row losses) for NONE
 *  lse      fp32 [n], required: log-sum-exp of each valid row, 0 on ignored rows
 *           (flce_backward needs it)
 *  row_loss fp32 [n] or NULL: per-row losses (0 on ignored rows)
 *  ws       workspace of at least flce_workspace_size(params, 0) bytes,
 *           256-byte aligned
 * Targets are range-checked on the device; call flce_check_status to read the
 * result. */
flce_status flce_forward(const flce_params* params, const void* x, const void* w,
                         const void* bias, const int32_t* targets, float* loss,
                         float* lse, float* row_loss, void* ws, size_t ws_bytes,
                         void* stream);

/* Forward plus the predicted-token and token-accuracy outputs of the option
 * set (page "[CuteDSL] FLCE", Summary; the pages give no formula, so the plain
 * reading): the predicted token of a row is the argmax over the vocabulary of
 * its final logit z (after bias and softcap; the lowest index among equal
 * maxima), and the token accuracy is the fraction of valid rows whose
 * predicted token is the target (0 if no row is valid).  The argmax is
 * tracked in the same GEMM epilogue as the LSE, in fp32.
 *  pred      int32 [n] or NULL: predicted token, -1 on ignored rows
 *  accuracy  fp32 [1] or NULL
 * Other arguments and the workspace size as for flce_forward (both NULL is
 * flce_forward). */
flce_status flce_forward_metrics(const flce_params* params, const void* x, const void* w,
                                 const void* bias, const int32_t* targets, float* loss,
                                 float* lse, float* row_loss, int32_t* pred, float* accuracy,
                                 void* ws, size_t ws_bytes, void* stream);

/* Backward from the saved LSE (page "[CuteDSL] FLCE", Summary: the backward
 * recomputes the masked softmax tile by tile over the vocabulary; dW is
 * contracted over all tokens and written once per vocabulary slice).
 *  lse          fp32 [n] from flce_forward with the same inputs and options
 *  grad_output  fp32 [1] device scalar g (d total / d loss), or NULL for 1.0
 *  dx           [n, d] dtype, overwritten
 *  dw           [v, d] fp32 (bf16 with params->dw_bf16), overwritten
 *  dbias        fp32 [v], overwritten; may be NULL only when bias is NULL
 *  ws           at least flce_workspace_size(params, 1) bytes
 * reduction NONE returns FLCE_ERR_UNSUPPORTED (a per-token upstream gradient
 * cannot be folded into the vocabulary-sliced weight-gradient contraction). */
flce_status flce_backward(const flce_params* params, const void* x, const void* w,
                          const void* bias, const int32_t* targets, const float* lse,
                          const float* grad_output, void* dx, void* dw, float* dbias,
                          void* ws, size_t ws_bytes, void* stream);

/* Forward and backward in one call with grad_output = 1.0 (the fwd+bwd
 * benchmark convention of the page "[CuteDSL] FLCE", Benchmarks).  Outputs as
 * in flce_forward and flce_backward; lse is still required (it is written and
 * then consumed).  reduction NONE returns FLCE_ERR_UNSUPPORTED. */
flce_status flce_fused_fwd_bwd(const flce_params* params, const void* x, const void* w,
                               const void* bias, const int32_t* targets, float* loss,
                               float* lse, void* dx, void* dw, float* dbias, void* ws,
                               size_t ws_bytes, void* stream);

/* flce_fused_fwd_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and results without the
 * workspace arguments.  Its workspace is a 128 MiB array inside the library
 * (one per GPU, held until the process ends); the call allocates nothing.
 * Parameters whose flce_workspace_size(params, 1) exceeds 128 MiB return
 * FLCE_ERR_WORKSPACE_TOO_SMALL before any HIP call (a smaller
 * params->vocab_slice or params->token_chunk reduces the size).  Every call
 * on one GPU uses the same array: calls that overlap on a GPU (other streams,
 * other threads) race and must be serialised by the caller. */
flce_status flce_fused_fwd_bwd_noalloc(const flce_params* params, const void* x, const void* w,
                                       const void* bias, const int32_t* targets, float* loss,
                                       float* lse, void* dx, void* dw, float* dbias, void* stream);

/* ---------------------------------------------------------------------------
 * Cross-entropy on logits given directly (no linear layer): the workload of
 * the cross-entropy kernels of the page "Add efficient Cross-Entropy by cuda
 * kernel" (TransformerEngine PR #995, Changes: a forward that reduces each row
 * to its maximum and sum of exponentials, and a backward that writes the
 * softmax minus the one-hot target, less a uniform smoothing term), with the
 * option set and definitions above applied to r = logits:
 *
 *   z = c tanh(r / c) (softcap c > 0) or r;  lse, row_n and loss as above;
 *   dL/dr = scale [softmax(z)(1 + 2 s lse) - (1-eps) onehot - eps/V] (1 - (z/c)^2)
 *
 * eps is the PyTorch smoothing; the Megatron form that page's kernels follow
 * (smoothing = eps_M V / (V - 1), i.e. 1 - eps_M on the target and
 * eps_M / (V - 1) on every other class) is eps = eps_M V / (V - 1) here.
 * params->d and params->vocab_slice are ignored.  The logits are [n, v]
 * row-major in params->dtype, element-aligned; V is arbitrary (a row that does
 * not start on 16 bytes is read as an unaligned head, 16-byte vectors and an
 * unaligned tail).  Streaming kernels, one workgroup per row: the forward
 * reads the logits once; the backward reads them once and writes dL/dr once.
 * Rows whose target is ignore_index are not read; their gradient rows are 0.
 * Targets are range-checked on the device (flce_check_status); an
 * out-of-range target never causes an out-of-bounds access.
 * ------------------------------------------------------------------------- */

/* Workspace bytes of the flce_ce_* calls: O(N) (status word, row map, per-row
 * losses, block sums).  0 for invalid parameters. */
size_t flce_ce_workspace_size(const flce_params* params);

/* Forward on logits.  loss, lse and row_loss as for flce_forward. */
flce_status flce_ce_forward(const flce_params* params, const void* logits,
                            const int32_t* targets, float* loss, float* lse,
                            float* row_loss, void* ws, size_t ws_bytes, void* stream);

/* Forward on logits with the predicted tokens and token accuracy defined at
 * flce_forward_metrics (pred int32 [n] or NULL, accuracy fp32 [1] or NULL). */
flce_status flce_ce_forward_metrics(const flce_params* params, const void* logits,
                                    const int32_t* targets, float* loss, float* lse,
                                    float* row_loss, int32_t* pred, float* accuracy, void* ws,
                                    size_t ws_bytes, void* stream);

/* Backward on logits from the saved lse.
 *  grad_output  fp32 [1] device scalar, or NULL for 1.0
 *  dlogits      [n, v] dtype, overwritten with dL/dr; may be `logits` itself
 *               (in place), else it must be misaligned to 16 bytes exactly as
 *               much as `logits` (both 16-byte aligned is the usual case)
 * reduction NONE returns FLCE_ERR_UNSUPPORTED. */
flce_status flce_ce_backward(const flce_params* params, const void* logits,
                             const int32_t* targets, const float* lse,
                             const float* grad_output, void* dlogits, void* ws,
                             size_t ws_bytes, void* stream);

/* Forward and backward in one pass per row with grad_output = 1.0: each row
 * is reduced to its lse, then its gradient is written (dlogits may be
 * `logits`, as for flce_ce_backward).  reduction NONE returns
 * FLCE_ERR_UNSUPPORTED. */
flce_status flce_ce_fused_fwd_bwd(const flce_params* params, const void* logits,
                                  const int32_t* targets, float* loss, float* lse,
                                  void* dlogits, void* ws, size_t ws_bytes, void* stream);

/* Forward and backward with three contractions instead of four (the
 * chunked-store schedule the page "[CuteDSL] FLCE" compares against: 6 N D V
 * FLOPs instead of 8 N D V, more memory): the packed valid rows go in token
 * chunks of params->token_chunk rows (0 = 8192); the forward GEMM of a chunk
 * keeps its raw logits (fp32, C x V x 4 bytes of workspace) next to the
 * online-softmax partials, the G kernel reads them back instead of
 * recomputing them, dX of the chunk contracts over the whole vocabulary at
 * once, and dW / db accumulate over the chunks.  Same arguments, outputs and
 * options as flce_fused_fwd_bwd (params->vocab_slice is unused); the
 * workspace is flce_stored_workspace_size(params). */
size_t flce_stored_workspace_size(const flce_params* params);

flce_status flce_fused_fwd_bwd_stored(const flce_params* params, const void* x, const void* w,
                                      const void* bias, const int32_t* targets, float* loss,
                                      float* lse, void* dx, void* dw, float* dbias, void* ws,
                                      size_t ws_bytes, void* stream);

/* The host-side validation contract of the page "[CuteDSL] FLCE",
 * Correctness, for the one check that needs the targets' values: synchronises
 * `stream`, then reports the device-side target check of the last call that
 * used this workspace: FLCE_OK or FLCE_ERR_TARGET_OUT_OF_RANGE
 * (FLCE_ERR_DEVICE if the synchronisation or copy fails).  When it reports an
 * out-of-range target, that call's numeric results are undefined. */
flce_status flce_check_status(const void* ws, void* stream);

/* Static, human-readable name of a status code: the reason a call was
 * refused (the host-side validation and by-design refusal contracts of the
 * page "[CuteDSL] FLCE", Correctness, e.g. reduction NONE with a backward). */
const char* flce_status_string(flce_status status);

/* Library version as major * 10000 + minor * 100 + patch.  Not an operation
 * of the method: it names the build of the option set above (page
 * "[CuteDSL] FLCE", Summary); 1.1.0 forms the row loss from the row maximum
 * (see flce_forward). */
int flce_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
