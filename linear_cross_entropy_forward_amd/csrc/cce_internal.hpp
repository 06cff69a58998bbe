// Internal constants, problem description and workspace layout shared by the
// C-ABI host code and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cce {

// Tile geometry.  The forward and gradient tiles are kTileV vocab x kTileN
// tokens; every wave of the forward owns kPartialWidth vocab rows and writes
// one (max, sum-exp) partial per (token, kPartialWidth-block).  The gradient
// filter decides per (kTileN tokens, kTileV vocab) tile.
constexpr int kTileV = 256;
constexpr int kTileN = 256;
constexpr int kPartialWidth = 128;
// The filter's finer level: within a kept tile, 32 token rows x 32 vocab
// entries, the MFMA output block; the gradient kernel zeroes G on blocks whose
// softmax stays below 2^-12 (and that hold no target) and the two gradient
// contractions skip their MFMAs there.
constexpr int kBlock = 32;
constexpr int kBlocksPerTile = kTileV / kBlock;  // 8 along either side
constexpr int kMaxBlocks = 1024;  // K blocks one contraction tile can list
// Compact gradient storage: one 256 x 256 tile per slot, rows of 256
// elements (token-major); slot j starts at row j * kSlotRows.
constexpr int kSlotRows = 256;
// Row blocks of the column-sum kernel (partials [kColBlocks][D] in the
// workspace) and the fewest rows one block takes.
constexpr int kColBlocks = 512;
constexpr int kColMinRows = 64;

constexpr int kDtypeBf16 = 0;
constexpr int kDtypeF32 = 1;
constexpr int kReductionNone = 0;
constexpr int kReductionSum = 1;
constexpr int kReductionMean = 2;
constexpr int kAccumDeterministic = 0;
constexpr int kAccumAtomic = 1;

// int32 counters at the start of the workspace.
constexpr int kHdrNValid = 0;
constexpr int kHdrBadTargets = 1;
constexpr int kHdrTilesKept = 2;
constexpr int kHdrNValidBwd = 3;
constexpr int kHdrBlocksKept = 4;
constexpr int kHdrWords = 64;  // 256 bytes

// Default byte budget of one vocabulary chunk's gradient tiles (G, and for
// fp32 operands G^T as well): 256 MiB, but never narrower than
// kMinChunkTiles vocabulary tiles (so that each chunk's contractions keep
// K long enough to outweigh the fp32 read-modify-write of dE that every
// further chunk costs; at N = 16384 both give 8192 columns).  Chunks are
// balanced: the vocabulary is cut into ceil(V / widest) nearly equal
// chunks of whole tiles.
constexpr size_t kDefaultGBudget = size_t(256) << 20;
constexpr int kMinChunkTiles = 32;
// Extra elements per row of the transposed gradient tiles (row pitch
// Npad + kGtPad).  Zero: measured no faster with a padded pitch.
constexpr int kGtPad = 0;
// Work-groups that run at once with one per CU (256 CUs).
constexpr int kWaveSlots = 256;


struct Problem {
  const void* e;
  const void* c;
  const void* bias;  // [V] operand type, or null
  const int64_t* targets;
  int N, D, V;
  int dtype;
  int64_t ignore_index;
  int reduction;
  float label_smoothing;  // eps in [0, 1]: soft target (1 - eps) onehot + eps / V
  float z_loss;           // lam >= 0: loss_i += lam * LSE_i^2
  float softcap;          // s >= 0: logits s tanh(z / s) when s > 0
  // forward outputs / backward inputs
  float* loss;
  float* lse;
  int32_t* n_valid;
  // backward
  const float* grad_loss;
  int filter;
  int accum;
  void* dE;          // [N][D], float or (grad_bf16) bf16
  void* dC;          // [V][D], float or (grad_bf16) bf16
  float* dbias;      // [V] or null
  int grad_bf16;     // dE and dC in bf16 (bf16 operands, grad_dtype = operand dtype)
};

// Two device buffers, both owned by the caller.  The forward state is what
// cce_forward writes and cce_backward reads (O(N + N V / 128 + 512 D)
// floats: the per-block partials, the counters, the classifier column sum);
// the backward workspace is scratch of one cce_backward call (the vocabulary
// chunk's gradient tiles, e^T, the compaction arrays, dE accumulation).
struct Layout {
  size_t state_total;  // bytes of the forward state
  size_t total;        // bytes of the backward workspace
  // -- forward state
  int32_t* hdr;
  float2* part;     // [N][nVB]
  float* nll_out;   // [N] per-row loss (the caller's loss buffer for 'none')
  float* csum;      // [D] sum over the vocabulary of the classifier rows (label smoothing)
  float* aux;       // [0] sum of the bias (label smoothing with a bias)
  float* colpart;   // [kColBlocks][D] column-sum partials of the forward
  // -- backward workspace
  float* scale;     // [Npad] per token row (original order), 0 past N
  int* rowmap;      // [Npad] token row of each compacted slot: valid rows, ignored rows, -1
  float* scale_c;   // [Npad] scale per compacted slot (0 for ignored rows and padding)
  float* lse_c;     // [Npad] LSE per compacted slot (+inf for ignored rows and padding)
  int* tgt_c;       // [Npad] target per compacted slot (-1 for ignored rows and padding)
  float* db_part;   // [Npad/256][V] per token block column sums of G (bias gradient)
  float* r1c;       // [D] -eps/V * sum_i scale_i e_i: the smoothing term of every dC row
  float* ssum;      // [1] sum_i scale_i (label smoothing's share of db)
  float* bcolpart;  // [bcol_blocks][D] column-sum partials of the backward
  uint8_t* keep;    // [nb][nvb_t]
  uint8_t* bmask;   // [nb][nvg] per 32-vocab group, bit t: 32-row group t of the token block kept
  int* tlist;       // [nchunks][list_stride] per chunk, its kept gradient tiles in launch order
  int* tcount;      // [nchunks] kept gradient tiles per chunk
  int* ch_vb;       // [nchunks + 1] first vocab tile of each chunk (chunk ch: [ch_vb[ch], ch_vb[ch + 1]))
  int* slot;        // [nb][nvb_t] compact: slot of each kept tile in its chunk's G
  // G, bf16 (compact): cap slots of one 256 x 256 tile each ([256 tokens][256
  // vocab], 128 KB), the kept tiles of one chunk in list order; fp32: [Npad][Vc],
  // the chunk's tiles in place
  void* G;
  void* Gt;         // [Vc][gt_ld] the same tiles transposed, fp32 only (columns past Npad unused)
  void* Et;         // [D][Npad] e transposed (zero rows past N)
  size_t g_bytes;   // bytes of G
  size_t gt_bytes;  // bytes of Gt
  int gt_ld;        // row pitch of Gt in elements: Npad + kGtPad
  float* dE_part;   // [splits-1][N][D]
  float* dE_acc;    // [N][D] fp32 accumulation of dE when dE itself is bf16 and more than one pass adds to it
  int nVB, Npad, nb, nvb_t, nvg, Vc, nchunks, splits, splits_atomic, bcol_blocks;
  // compact gradient storage (bf16): chunks are packed from units of `unit`
  // vocab tiles, at most S kept tiles (cap slots, cap = S) and span_u units
  // each; dense (fp32): chunks of unit = Vc / 256 vocab tiles.
  // list_stride = per-chunk list length
  int compact, unit, S, cap, span_u, list_stride;
};


// Computes the layout for (N, D, V, dtype, vocab_chunk); the pointers of the
// forward state are set when `state` is given, those of the backward
// workspace when `ws` is given (sizes are always filled in).
Layout make_layout(int64_t N, int64_t D, int64_t V, int dtype, int64_t vocab_chunk, void* state, void* ws);
// Row blocks (the return value) and rows per block of the column sum over R
// rows.
int colsum_blocks(int64_t R, int& rows_per_block);

// Kernel ids of the profiling hook (cce_profile_start / cce_profile_stop).
enum KernelId {
  kKFwdTile = 0, kKRows, kKReduce, kKBwdPrep, kKFilter, kKGradTile, kKDC, kKDE, kKDEReduce, kKFill,
  kKTransE, kKDbReduce, kKColSum, kKColReduce, kKVecSum, kKFillRank1, kKTileList, kNumKernels
};
// Records start/stop events around one launch of kernel `id` when profiling of
// that id is active (no-op otherwise).
void prof_before(int id, hipStream_t st);
void prof_after(int id, hipStream_t st);

hipError_t launch_forward(const Problem& P, const Layout& L, hipStream_t st);
// An empty batch (N = 0): zero counters, the reduced loss (when given), n_valid
// (when given), `gbytes` bytes at `g` (dC; a multiple of 16) and `nb` floats at
// `b` (db).
hipError_t launch_empty(const Layout& L, float* loss, int32_t* n_valid, void* g, size_t gbytes, float* b, size_t nb,
                        hipStream_t st);
hipError_t launch_backward(const Problem& P, const Layout& L, hipStream_t st);

}  // namespace cce
