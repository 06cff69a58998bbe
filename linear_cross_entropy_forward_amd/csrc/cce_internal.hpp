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
constexpr int kMaxBlocks = 4096;  // K blocks one contraction tile can list
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
constexpr int kHdrWords = 64;  // 256 bytes

// Default byte budget of the per-chunk gradient tile buffers G and G^T together
// (2 GiB: one chunk for the whole vocabulary at N = 4096; fewer, longer
// launches measured faster than 512 MiB chunks).
constexpr size_t kDefaultGBudget = size_t(2048) << 20;
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

struct Layout {
  size_t total;     // bytes
  int32_t* hdr;
  float2* part;     // [N][nVB]
  float* nll_out;   // [N] per-row loss (the caller's loss buffer for 'none')
  float* scale;     // [Npad] per token row (original order), 0 past N
  int* rowmap;      // [Npad] token row of each compacted slot: valid rows, ignored rows, -1
  float* scale_c;   // [Npad] scale per compacted slot (0 for ignored rows and padding)
  float* lse_c;     // [Npad] LSE per compacted slot (+inf for ignored rows and padding)
  int* tgt_c;       // [Npad] target per compacted slot (-1 for ignored rows and padding)
  float* db_part;   // [Npad/256][V] per token block column sums of G (bias gradient)
  float* csum;      // [D] sum over the vocabulary of the classifier rows (label smoothing)
  float* r1c;       // [D] -eps/V * sum_i scale_i e_i: the smoothing term of every dC row
  float* aux;       // [0] sum of the bias, [1] sum_i scale_i
  float* colpart;   // [kColBlocks][D] column-sum partials
  uint8_t* keep;    // [nb][nvb_t]
  int* tlist;       // per chunk, its kept gradient tiles in launch order (chunk ch at cvb0 * nb)
  int* tcount;      // [nchunks] kept gradient tiles per chunk
  void* G;          // [Npad][Vc] operand type: gradient tiles of one vocab chunk
  void* Gt;         // [Vc][gt_ld] the same tiles transposed, fp32 only (columns past Npad unused)
  void* Et;         // [D][Npad] e transposed (zero rows past N)
  size_t g_bytes;   // bytes of G
  size_t gt_bytes;  // bytes of Gt
  int gt_ld;        // row pitch of Gt in elements: Npad + kGtPad
  float* dE_part;   // [splits-1][N][D]
  float* dE_acc;    // [N][D] fp32 accumulation of dE when dE itself is bf16 and more than one pass adds to it
  int nVB, Npad, nb, nvb_t, Vc, nchunks, splits, splits_atomic;
};

// Computes the layout for (N, D, V, dtype, vocab_chunk); with base == nullptr
// only sizes are filled in.
Layout make_layout(int64_t N, int64_t D, int64_t V, int dtype, int64_t vocab_chunk, void* base);

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
