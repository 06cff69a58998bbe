/*
 * cce.h — C ABI of libcce, a fused linear cross-entropy ("Cut Cross-Entropy")
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For token rows e_i (i < N, length D), classifier rows c_j
 * (j < V, length D) and integer targets y_i:
 *
 *     LSE_i  = log sum_j exp(e_i . c_j)
 *     loss_i = LSE_i - e_i . c_{y_i}
 *
 * as stated in Wijmans et al., "Cut Your Losses in Large-Vocabulary Language
 * Models" (abstract: only the correct token's logit and a log-sum-exp over all
 * logits evaluated on the fly) and in the blog "Cut Cross Entropy from first
 * principles" (loss = LSE minus the correct-token logit).  The [N, V] logit
 * matrix is never written to device memory (mlx-cross-entropy README, "The
 * problem" and "How it works").  Rows whose target equals ignore_index give
 * loss 0 and gradient 0 and are not counted; reductions are none / sum / mean
 * over the non-ignored rows (README "API" table; tirogla "Loss functions",
 * "How it works" step 4 and the "Code" section, which floors the count at 1).
 * The backward returns dE = G C and dC = G^T E with
 * G = (softmax - onehot(y)) * scale ("Loss functions" step 2: the fused gradient p - y),
 * dropping G on (32 token rows, 32 vocab entries) blocks on which every
 * softmax value is below 2^-12 and that hold no target (README "How it
 * works" items 1-2: 32x32 tiles, skipped below 2^-12; Wijmans et al.
 * abstract): whole 256x256 gradient tiles are skipped from the forward's
 * per-block maxima, and inside kept tiles the contractions skip the MFMAs of
 * dropped blocks.
 *
 * Two optional loss terms follow tirogla "Loss functions": label smoothing
 * eps ("How it works" step 3) replaces the one-hot target by the soft target
 * T_i = (1 - eps) onehot(y_i) + eps / V (over all V classes, the true one
 * included), so loss_i = -sum_j T_ij log softmax_ij and G = (softmax - T) *
 * scale; the z-loss lam ("Implementation notes") adds lam * LSE_i^2 to
 * loss_i, which adds 2 lam LSE_i softmax_ij to G.  Filtering still decides on
 * the softmax and drops only its part of G: the uniform -eps/V * scale_i part
 * is applied to every entry (as a rank-one term of dE, dC and dbias).
 *
 * Logit soft-capping s > 0 is not defined on those pages: it takes the form
 * Gemma 2 uses, z' = s tanh(z / s) after the bias, in place of z everywhere
 * (LSE, the correct-token logit, the filter's softmax), and multiplies G by
 * dz'/dz = 1 - (z' / s)^2.  It cannot be combined with label smoothing (the
 * smoothing part of G is then no longer the same for every entry):
 * CCE_ERR_UNSUPPORTED.  It is built for bf16 operands only: with float32
 * operands a softcap > 0 is CCE_ERR_UNSUPPORTED.
 *
 * Conventions for every call:
 *  - Pointers marked (device) are device memory on the current HIP device;
 *    (host) are host memory.  The library never allocates, frees or
 *    synchronises in cce_forward / cce_backward: it enqueues kernels on
 *    `stream` and returns.  The caller owns every buffer, including the two
 *    that carry the library's own data: the forward state (written by
 *    cce_forward, read by cce_backward: O(N + N*V/128 + 512*D) floats, the
 *    per-block partials the backward's filter reuses) and the backward
 *    workspace (scratch of one cce_backward call: the gradient tiles of a
 *    vocabulary chunk, e transposed, dE accumulation), and keeps them alive
 *    until the stream work completes.  Between forward and backward only the
 *    state needs to be kept (about 41 MB at N = 4096, D = 4096, V = 128256,
 *    against 2.1 GB of fp32 logits); the workspace can be allocated for the
 *    backward and freed after it.
 *  - Layout: row-major, contiguous, base pointers 16-byte aligned.  e is
 *    [N, D], c is [V, D] (D contiguous); e and c share one dtype; outputs are
 *    float32 (dE, dC: see cce_backward).  D must be a multiple of 8 (bf16)
 *    or 4 (float32); D and V are positive.
 *  - An empty batch (N = 0) is valid: e, targets, lse, a per-row loss, dE and
 *    grad_loss have no elements and may be NULL; the forward writes n_valid 0
 *    and a sum or mean of 0 (the mean's count is floored at 1), the backward
 *    writes dC and dbias as zeros.
 *  - Errors: argument and size faults are reported synchronously, before any
 *    launch, as a negative cce_status (label_smoothing outside [0, 1] or a
 *    negative or non-finite z_loss is CCE_ERR_INVALID_ARG).  A target outside [0, V) that is not
 *    ignore_index is not a host-visible fault: its row's loss is NaN (so a
 *    mean or sum is NaN), its gradient row is NaN, and cce_read_stats
 *    reports it in bad_targets.  No exception crosses the ABI.
 *  - Reentrancy: apart from the measurement hook at the end of this header
 *    (and the no-allocation forward, which shares one device array), the
 *    library keeps no global mutable state; calls on different states and
 *    workspaces may run concurrently.  Two calls sharing a state or a
 *    workspace must be ordered on one stream.
 */
#ifndef CCE_H_
#define CCE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same object as hipStream_t; NULL is the default stream. */
typedef struct ihipStream_t* cce_stream_t;

typedef enum {
  CCE_OK = 0,
  CCE_ERR_INVALID_ARG = -1, /* null pointer, negative N or non-positive D / V, bad enum, misalignment */
  CCE_ERR_UNSUPPORTED = -2, /* softcap with label smoothing, D not a multiple of the vector width, size limits */
  CCE_ERR_WORKSPACE = -3,   /* state or workspace smaller than cce_state_size() / cce_workspace_size() */
  CCE_ERR_HIP = -4          /* a HIP launch or copy reported an error */
} cce_status;

typedef enum { CCE_DTYPE_BF16 = 0, CCE_DTYPE_F32 = 1 } cce_dtype;
typedef enum { CCE_REDUCTION_NONE = 0, CCE_REDUCTION_SUM = 1, CCE_REDUCTION_MEAN = 2 } cce_reduction;
typedef enum { CCE_ACCUM_DETERMINISTIC = 0, CCE_ACCUM_ATOMIC = 1 } cce_accum;
/* Element type of dE and dC: float32, or the operands' dtype (bf16 for bf16
 * operands; rounded to nearest even from the fp32 accumulation). */
typedef enum { CCE_GRAD_FLOAT32 = 0, CCE_GRAD_OPERAND = 1 } cce_grad_dtype;

typedef struct {
  int64_t n_valid;      /* rows whose target != ignore_index (last forward)        */
  int64_t bad_targets;  /* non-ignored targets outside [0, V)  (last forward)      */
  int64_t tiles_total;  /* gradient tiles of the last backward: ceil(N/Bn)*ceil(V/Bv) */
  int64_t tiles_kept;   /* tiles the last backward computed (filter decision)      */
  int64_t filter_rows;  /* Bn: token rows per gradient tile                        */
  int64_t filter_vocab; /* Bv: vocabulary entries per gradient tile                */
  int64_t blocks_total; /* 32x32 blocks of the last backward: ceil(N/32)*ceil(V/32)  */
  int64_t blocks_kept;  /* blocks of kept tiles whose G the last backward kept     */
  int64_t block_rows;   /* 32: token rows per block                                */
  int64_t block_vocab;  /* 32: vocabulary entries per block                        */
} cce_stats;

/*
 * Bytes of the forward state for this problem: the int32 counters, the
 * per-(row, 128-vocab block) (max, sum-exp) partials, the per-row loss and,
 * for label smoothing, the classifier column sum and its row-block partials.
 * Returns 0 for invalid arguments.
 */
size_t cce_state_size(int64_t N, int64_t D, int64_t V, int dtype);

/*
 * Bytes of the backward workspace for this problem and vocab_chunk.
 * vocab_chunk = 0 picks the library default.  The backward forms the
 * gradient tiles G one vocabulary chunk at a time and keeps that chunk's G
 * in the workspace: with bf16 operands only the kept 256x256 tiles, one
 * 128 KB slot each, room for the tiles of a chunk vocab_chunk wide (rounded
 * up to 8 tiles) when every tile is kept, and the chunks are cut by kept
 * tiles, so a filtered backward covers the vocabulary in as few chunks as
 * that room allows (one at the pages' Gemma-2-2B head); with fp32 operands G
 * and G^T of a chunk exactly vocab_chunk wide.  The default room is at most
 * 256 MiB but never fewer than 8192 columns (the vocabulary cut into nearly
 * equal chunks of whole 256-wide tiles: 4 chunks at N = 4096, V = 128256, 16
 * at N = 16384, when nothing is filtered).  Plus e transposed (N*D
 * elements), an fp32 [N, D] accumulation of dE for bf16 gradients that more
 * than one pass adds up, and the compaction, keep-map and chunk arrays:
 * about 0.38 GB at N = 4096, D = 4096, V = 128256 (1.2 GB with the whole
 * vocabulary in one chunk).  A positive value (a multiple of 256) sets the
 * chunk width, trading workspace for launches.  Returns 0 for invalid
 * arguments.
 */
size_t cce_workspace_size(int64_t N, int64_t D, int64_t V, int dtype, int64_t vocab_chunk);

/*
 * Vocabulary entries per chunk that cce_backward sizes its gradient tiles for,
 * for this problem and vocab_chunk argument (the default when vocab_chunk = 0;
 * the value passed, clamped to the vocabulary, otherwise): the chunk width
 * when every tile is kept.  The backward launches its gradient kernels once
 * per chunk.  A chunk's classifier rows stay under 2^31 bytes, the reach of
 * one buffer descriptor, so a classifier of any size (V * D elements) is
 * taken in chunks.  Returns 0 for invalid arguments.
 */
int64_t cce_vocab_chunk(int64_t N, int64_t D, int64_t V, int dtype, int64_t vocab_chunk);

/*
 * Forward.  e (device) [N, D], c (device) [V, D] of `dtype`; bias (device)
 * [V] of `dtype` or NULL: the optional classifier bias of the mlx-cross-entropy
 * README ("API" table), added to every row of the logits, z = e c^T + b;
 * targets (device) int64 [N].  label_smoothing (eps in [0, 1]) and z_loss (lam >= 0)
 * are the optional terms above, 0 for the plain loss; eps > 0 adds two
 * HBM-bound passes (a column sum of c over the vocabulary, and of the bias).
 * reduction: CCE_REDUCTION_NONE writes loss[N] (0 on ignored rows);
 * SUM / MEAN write loss[0] (MEAN divides by max(n_valid, 1)).  lse (device)
 * float [N] receives every row's LSE (ignored rows included).  n_valid
 * (device) int32 [1] receives the non-ignored count; may be NULL.  softcap: 0 for
 * none, s > 0 (finite) for s tanh(z / s); negative or non-finite values are
 * CCE_ERR_INVALID_ARG.  state (device) of state_bytes >= cce_state_size(N, D,
 * V, dtype) receives the forward state (the per-block partials the backward's
 * filter reads, the counters cce_read_stats reports): keep it unmodified
 * between this call and cce_backward.  A state smaller than that is
 * CCE_ERR_WORKSPACE.
 */
cce_status cce_forward(const void* e, const void* c, const void* bias, const int64_t* targets, int64_t N,
                       int64_t D, int64_t V, int dtype, int64_t ignore_index, int reduction, float softcap,
                       float label_smoothing, float z_loss, float* loss, float* lse, int32_t* n_valid, void* state,
                       size_t state_bytes, cce_stream_t stream);

/*
 * Forward without a state buffer, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments as cce_forward, minus the state: the state
 * lives in one static device array of CCE_NOALLOC_SCRATCH_BYTES per GPU (the
 * library's own, held by each GPU the library runs on until the process
 * ends), so no cce_backward or cce_read_stats can follow this call.  Problems
 * whose cce_state_size exceeds CCE_NOALLOC_SCRATCH_BYTES (64 MiB: e.g.
 * N = 4096 tokens at V = 128256, or N = 2048 at V = 256000) return
 * CCE_ERR_WORKSPACE before any HIP call.  It allocates, frees and
 * synchronises nothing (the array's device address is looked up once per
 * device, on the first call with that device current).  Every call on a GPU
 * shares that GPU's array, which keeps the last call's contents: calls that
 * overlap on one GPU (two streams, two threads) race and must be ordered by
 * the caller.
 */
#define CCE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
cce_status cce_forward_noalloc(const void* e, const void* c, const void* bias, const int64_t* targets, int64_t N,
                               int64_t D, int64_t V, int dtype, int64_t ignore_index, int reduction, float softcap,
                               float label_smoothing, float z_loss, float* loss, float* lse, int32_t* n_valid,
                               cce_stream_t stream);

/*
 * Backward.  Same e, c, bias, targets, sizes, dtype, ignore_index, reduction,
 * softcap, label_smoothing and z_loss as the forward; lse (device) float [N] is
 * the forward's output and state is the forward's state, unmodified (with
 * label smoothing it also holds the forward's column sum of c; the backward
 * only updates its counters).  ws (device) of ws_bytes >=
 * cce_workspace_size(N, D, V, dtype, vocab_chunk) is this call's scratch (its
 * contents on entry do not matter).  grad_loss (device) float is the
 * upstream gradient: [N] for NONE, [1] otherwise.  filter = 1 drops G on
 * the 32x32 blocks whose softmax is below 2^-12 everywhere (and that hold no
 * target), skipping 256x256 tiles made only of such blocks; 0 computes every
 * tile and block.  accum = CCE_ACCUM_DETERMINISTIC gives run-to-run
 * bitwise-identical results (fixed-order split reduction);
 * CCE_ACCUM_ATOMIC accumulates dE with fp32 atomics.  grad_dtype
 * (cce_grad_dtype) picks the element type of dE (device) [N, D] and dC
 * (device) [V, D], both overwritten: float32, or the operand dtype (bf16
 * gradients written by the kernels themselves, every accumulation still
 * fp32, so a caller training in bf16 needs no conversion pass).  dE or dC
 * may be NULL: that gradient is not formed and its contraction does not run
 * (a frozen classifier or frozen inputs); at least one of dE, dC and dbias
 * must be given.  dbias (device) float
 * [V] or NULL: when given, overwritten with the bias gradient db_j =
 * sum_i G_ij (column sums of the filtered gradient tiles, in a fixed order
 * in both accum modes); it is defined with or without a bias.  vocab_chunk as
 * in cce_workspace_size.  A state or workspace smaller than its size is
 * CCE_ERR_WORKSPACE.
 */
cce_status cce_backward(const void* e, const void* c, const void* bias, const int64_t* targets, int64_t N,
                        int64_t D, int64_t V, int dtype, int64_t ignore_index, int reduction, float softcap,
                        float label_smoothing, float z_loss, const float* lse, const float* grad_loss, int filter,
                        int accum, int64_t vocab_chunk, int grad_dtype, void* dE, void* dC, float* dbias,
                        void* state, size_t state_bytes, void* ws, size_t ws_bytes, cce_stream_t stream);

/*
 * Copies the state's counters to `out` (host) after the work queued on
 * `stream` so far; the one call here that synchronises (the stream).  N, V
 * describe the problem the state was used for (for tiles_total).
 */
cce_status cce_read_stats(const void* state, size_t state_bytes, int64_t N, int64_t V, cce_stream_t stream,
                          cce_stats* out);

/*
 * Copies the tile keep map of the last cce_backward that used `ws` (device) to
 * `out` (host), ceil(N/256) x ceil(V/256) bytes, row-major: 1 where that
 * backward computed the gradient tile, 0 where the filter dropped it.  Row
 * block b is the b-th group of 256 non-ignored rows in order (ignored rows
 * belong to no block; blocks past the non-ignored rows are 0).  N, D, V,
 * dtype and vocab_chunk are those of the backward (they fix the layout of
 * ws).  Synchronises `stream`.  A test and measurement aid.
 */
cce_status cce_read_keep_map(const void* ws, size_t ws_bytes, int64_t N, int64_t D, int64_t V, int dtype,
                             int64_t vocab_chunk, uint8_t* out, cce_stream_t stream);

/*
 * Copies the 32x32 block keep map of the last cce_backward that used `ws`
 * (device) to `out` (host), ceil(N/32) x ceil(V/32) bytes, row-major: 1 where
 * that backward kept the block's gradient entries (a block of a kept tile on
 * which some softmax value reaches 2^-12 or that holds a target), 0 where it
 * zeroed them.  Row block b is the b-th group of 32 non-ignored rows in order.
 * Arguments and synchronisation as cce_read_keep_map.
 */
cce_status cce_read_block_map(const void* ws, size_t ws_bytes, int64_t N, int64_t D, int64_t V, int dtype,
                              int64_t vocab_chunk, uint8_t* out, cce_stream_t stream);

/* Static description of a status code. */
const char* cce_status_string(int status);

/* Tile geometry: gradient tile Bn x Bv and the forward partial width. */
void cce_tile_shape(int* filter_rows, int* filter_vocab, int* partial_vocab);

/*
 * Measurement hook.  Between cce_profile_start(k, n) and cce_profile_stop(k,
 * ...), every launch of kernel k by cce_forward / cce_backward (at most n
 * launches) is bracketed by two HIP events recorded on the launch stream.
 * cce_profile_stop waits for those events and returns the summed elapsed time
 * (host double, ms) and the number of launches timed (host int).  The hook
 * holds process-wide state: it is meant for benchmarks and is not
 * thread-safe.  Kernel ids 0..16 are fwd_tile, rows, reduce, bwd_prep, filter,
 * grad_tile, dC_gemm, dE_gemm, dE_reduce, fill_zero, transpose_e, db_reduce,
 * colsum, colsum_reduce, vec_sum, fill_rank1, tile_list (cce_kernel_name).
 */
cce_status cce_profile_start(int kernel_id, int max_launches);
cce_status cce_profile_stop(int kernel_id, double* total_ms, int* launches);
const char* cce_kernel_name(int kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* CCE_H_ */
