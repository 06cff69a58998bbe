// C ABI of libcce: argument validation, workspace layout and the launch
// sequence of the forward and backward.  Declarations and the contract of each
// call are in include/cce.h.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/cce.h"
#include "cce_internal.hpp"

namespace cce {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Column-sum row blocks for R rows: at least kColMinRows rows per block, at
// most kColBlocks blocks.
int colsum_blocks(int64_t R, int& rows_per_block) {
  const int64_t rpb = std::max<int64_t>(kColMinRows, (R + kColBlocks - 1) / kColBlocks);
  rows_per_block = (int)rpb;
  return (int)std::max<int64_t>(1, (R + rpb - 1) / rpb);
}

Layout make_layout(int64_t N, int64_t D, int64_t V, int dtype, int64_t vocab_chunk, void* state, void* ws) {
  Layout L{};
  if (N < 1) N = 1;  // an empty batch uses only the counters; sized like one row
  const size_t es = dtype == kDtypeBf16 ? 2 : 4;
  L.nVB = (int)((V + kPartialWidth - 1) / kPartialWidth);
  L.Npad = (int)((N + kTileN - 1) / kTileN * kTileN);
  L.nb = L.Npad / kTileN;
  L.nvb_t = (int)((V + kTileV - 1) / kTileV);
  L.nvg = L.nvb_t * kBlocksPerTile;
  const int64_t vmax = (int64_t)L.nvb_t * kTileV;
  int64_t vc;
  if (vocab_chunk > 0) {
    vc = vocab_chunk;
  } else {
    // bf16 keeps G only; fp32 both G and G^T.  The widest chunk within the
    // budget (but at least kMinChunkTiles tiles), each buffer below 2 GiB
    // (32-bit buffer offsets), and the chunk's classifier rows too (one
    // descriptor in the dE contraction); then the vocabulary cut into that
    // many nearly equal chunks of whole tiles.
    const size_t per_col = ((size_t)L.Npad + kGtPad) * es * (dtype == kDtypeBf16 ? 1 : 2);
    int64_t tiles = (int64_t)(kDefaultGBudget / (per_col * kTileV));
    if (tiles < kMinChunkTiles) tiles = kMinChunkTiles;
    const int64_t cap = (int64_t)((((size_t)1 << 31) - 1) / (((size_t)L.Npad + kGtPad) * es) / kTileV);
    const int64_t cap_c = (int64_t)((((size_t)1 << 31) - 1) / ((size_t)D * es) / kTileV);
    tiles = std::min(std::min(tiles, cap), std::min(cap_c, (int64_t)kMaxBlocks));
    if (tiles < 1) tiles = 1;
    const int64_t nch = (L.nvb_t + tiles - 1) / tiles;
    vc = (L.nvb_t + nch - 1) / nch * kTileV;
  }
  if (vc < kTileV) vc = kTileV;
  if (vc > vmax) vc = vmax;
  if (vc > (int64_t)kMaxBlocks * kTileV) vc = (int64_t)kMaxBlocks * kTileV;
  L.Vc = (int)vc;
  const int tiles_d = (int)((D + kTileV - 1) / kTileV);
  const int tiles_de = L.nb * tiles_d;
  const int cvb = (int)(vc / kTileV);
  // bf16: compact gradient storage.  The vocabulary is cut into units of
  // `unit` vocab tiles (8, one per XCD in dC's dealing, or fewer for narrow
  // chunks) and consecutive units are packed greedily into chunks of at most
  // S = nb * m * unit kept tiles (m = ceil(cvb / unit) units, the dense
  // chunk rounded up to whole units) and at most span_u units (the block
  // lists of the contractions, the chunk's classifier rows under one 32-bit
  // buffer offset).  On a dense keep map that gives the dense chunks; on a
  // sparse one, as few chunks as the slots allow.  Every chunk but the last
  // holds at least min(m, span_u) units (a chunk cut for its count holds
  // more than (m - 1) * nb * unit tiles), which bounds the chunk count.
  L.compact = dtype == kDtypeBf16;
  if (L.compact) {
    const int64_t span_c = (int64_t)((((size_t)1 << 31) - 1) / ((size_t)D * es) / kTileV);
    const int span = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxBlocks, span_c));
    L.unit = std::min(std::min(8, cvb), span);
    const int m = (cvb + L.unit - 1) / L.unit;
    L.S = L.nb * m * L.unit;
    L.cap = L.S;
    L.span_u = std::max(1, span / L.unit);
    const int nunits = (L.nvb_t + L.unit - 1) / L.unit;
    const int per_chunk = std::min(m, L.span_u);
    L.nchunks = (nunits + per_chunk - 1) / per_chunk;
    L.list_stride = L.cap;
  } else {
    L.unit = cvb;
    L.S = 0;
    L.cap = 0;
    L.span_u = 1;
    L.nchunks = (int)((V + vc - 1) / vc);
    L.list_stride = cvb * L.nb;
  }
  // dE work-groups: enough vocabulary splits to fill one round of the chip
  // (kWaveSlots work-groups, one per CU); each further split adds a partial
  // buffer that the epilogue writes and a final pass re-reads.  (Taking more
  // splits when padding rows empty some token blocks measured slower: the
  // extra epilogues and partial traffic outweigh the fuller chip.)
  int sp = (kWaveSlots + tiles_de - 1) / tiles_de;
  if (sp > 8) sp = 8;
  if (sp > cvb) sp = cvb;
  if (sp < 1) sp = 1;
  L.splits = sp;
  int spa = (2 * kWaveSlots + tiles_de - 1) / tiles_de;
  if (spa > 16) spa = 16;
  if (spa > cvb) spa = cvb;
  if (spa < 1) spa = 1;
  L.splits_atomic = spa;
  L.g_bytes = L.compact ? (size_t)L.cap * kSlotRows * kTileV * es : (size_t)L.Npad * (size_t)vc * es;
  L.gt_ld = L.Npad + kGtPad;
  L.gt_bytes = dtype == kDtypeBf16 ? 0 : (size_t)L.gt_ld * (size_t)vc * es;
  int rpb_unused;
  L.bcol_blocks = colsum_blocks(N, rpb_unused);

  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  // forward state
  const size_t o_hdr = take(kHdrWords * 4);
  const size_t o_part = take((size_t)N * L.nVB * sizeof(float2));
  const size_t o_nll = take((size_t)N * 4);
  const size_t o_csum = take((size_t)D * 4);
  const size_t o_aux = take(64);
  const size_t o_colp = take((size_t)kColBlocks * (size_t)D * 4);
  L.state_total = off;
  // backward workspace
  off = 0;
  const size_t o_scale = take((size_t)L.Npad * 4);
  const size_t o_rowmap = take((size_t)L.Npad * 4);
  const size_t o_scale_c = take((size_t)L.Npad * 4);
  const size_t o_lse_c = take((size_t)L.Npad * 4);
  const size_t o_tgt_c = take((size_t)L.Npad * 4);
  const size_t o_keep = take((size_t)L.nb * L.nvb_t);
  const size_t o_bmask = take((size_t)L.nb * L.nvg);
  const size_t o_tlist = take((size_t)L.nchunks * L.list_stride * 4);
  const size_t o_tcount = take((size_t)L.nchunks * 4);
  const size_t o_chvb = take((size_t)(L.nchunks + 1) * 4);
  const size_t o_slot = take(L.compact ? (size_t)L.nb * L.nvb_t * 4 : 0);
  const size_t o_r1c = take((size_t)D * 4);
  const size_t o_ssum = take(64);
  const size_t o_bcolp = take((size_t)L.bcol_blocks * (size_t)D * 4);
  const size_t o_g = take(L.g_bytes);
  const size_t o_gt = take(L.gt_bytes);
  const size_t o_et = take((size_t)D * (size_t)L.Npad * es);
  const size_t o_dep = take((size_t)(L.splits - 1) * (size_t)N * (size_t)D * 4);
  const size_t o_dbp = take((size_t)L.nb * (size_t)V * 4);
  const size_t o_dacc = take((size_t)N * (size_t)D * 4);
  L.total = off;
  if (state) {
    char* b = (char*)state;
    L.hdr = (int32_t*)(b + o_hdr);
    L.part = (float2*)(b + o_part);
    L.nll_out = (float*)(b + o_nll);
    L.csum = (float*)(b + o_csum);
    L.aux = (float*)(b + o_aux);
    L.colpart = (float*)(b + o_colp);
  }
  if (ws) {
    char* b = (char*)ws;
    L.scale = (float*)(b + o_scale);
    L.rowmap = (int*)(b + o_rowmap);
    L.scale_c = (float*)(b + o_scale_c);
    L.lse_c = (float*)(b + o_lse_c);
    L.tgt_c = (int*)(b + o_tgt_c);
    L.keep = (uint8_t*)(b + o_keep);
    L.bmask = (uint8_t*)(b + o_bmask);
    L.tlist = (int*)(b + o_tlist);
    L.tcount = (int*)(b + o_tcount);
    L.ch_vb = (int*)(b + o_chvb);
    L.slot = (int*)(b + o_slot);
    L.r1c = (float*)(b + o_r1c);
    L.ssum = (float*)(b + o_ssum);
    L.bcolpart = (float*)(b + o_bcolp);
    L.G = b + o_g;
    L.Gt = b + o_gt;
    L.Et = b + o_et;
    L.dE_part = (float*)(b + o_dep);
    L.db_part = (float*)(b + o_dbp);
    L.dE_acc = (float*)(b + o_dacc);
  }
  return L;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shared checks of forward and backward.  Returns CCE_OK or an error.
static cce_status check_common(const void* e, const void* c, const int64_t* targets, int64_t N, int64_t D,
                               int64_t V, int dtype, int reduction, float softcap, const void* state,
                               int64_t vocab_chunk) {
  // an empty batch (N = 0) may pass null e and targets
  if (!c || !state || (N > 0 && (!e || !targets))) return CCE_ERR_INVALID_ARG;
  if (N < 0 || D <= 0 || V <= 0) return CCE_ERR_INVALID_ARG;
  if (dtype != kDtypeBf16 && dtype != kDtypeF32) return CCE_ERR_INVALID_ARG;
  if (reduction != kReductionNone && reduction != kReductionSum && reduction != kReductionMean)
    return CCE_ERR_INVALID_ARG;
  if (vocab_chunk < 0 || vocab_chunk % kTileV != 0) return CCE_ERR_INVALID_ARG;
  if (!aligned16(e) || !aligned16(c) || !aligned16(state) || ((uintptr_t)targets & 7u)) return CCE_ERR_INVALID_ARG;
  if (!(softcap >= 0.0f && softcap <= 3.0e38f)) return CCE_ERR_INVALID_ARG;
  // soft-capping is built for bf16 operands only (the fp32 variant is off)
  if (softcap > 0.0f && dtype != kDtypeBf16) return CCE_ERR_UNSUPPORTED;
  const int64_t es = dtype == kDtypeBf16 ? 2 : 4;
  if (D % (16 / es) != 0) return CCE_ERR_UNSUPPORTED;
  // 32-bit buffer offsets: every operand a kernel addresses from one base
  // stays below 2 GiB; the contraction tiles list at most kMaxBlocks blocks.
  const int64_t lim = (int64_t)1 << 31;
  if ((N + kTileN) * D * es >= lim || N > (int64_t)kMaxBlocks * kTileN || V >= lim / 2 || D >= lim / 2)
    return CCE_ERR_UNSUPPORTED;
  Layout L = make_layout(N, D, V, dtype, vocab_chunk, nullptr, nullptr);
  // (compact storage keeps each chunk's classifier rows within `span`)
  if ((!L.compact && (int64_t)L.Vc * D * es >= lim) || (int64_t)L.g_bytes >= lim || (int64_t)L.gt_bytes >= lim)
    return CCE_ERR_UNSUPPORTED;
  return CCE_OK;
}

// ---------------------------------------------------------------------------
// Profiling hook: HIP events recorded on the launch stream around every launch
// of the kernels being profiled.  Measurement aid only; not thread-safe.
// ---------------------------------------------------------------------------
struct ProfSlot {
  bool active = false;
  int cap = 0, n = 0;
  std::vector<hipEvent_t> ev;  // start, stop per launch
};
static ProfSlot g_prof[kNumKernels];

void prof_before(int id, hipStream_t st) {
  ProfSlot& p = g_prof[id];
  if (p.active && p.n < p.cap) (void)hipEventRecord(p.ev[2 * p.n], st);
}
void prof_after(int id, hipStream_t st) {
  ProfSlot& p = g_prof[id];
  if (p.active && p.n < p.cap) {
    (void)hipEventRecord(p.ev[2 * p.n + 1], st);
    ++p.n;
  }
}

static void prof_release(ProfSlot& p) {
  for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
  p.ev.clear();
  p.active = false;
  p.cap = p.n = 0;
}

static const char* const kKernelNames[kNumKernels] = {
    "fwd_tile", "rows", "reduce", "bwd_prep", "filter", "grad_tile", "dC_gemm", "dE_gemm", "dE_reduce",
    "fill_zero", "transpose_e", "db_reduce", "colsum", "colsum_reduce", "vec_sum", "fill_rank1", "tile_list"};

}  // namespace cce

using namespace cce;

extern "C" {

size_t cce_state_size(int64_t N, int64_t D, int64_t V, int dtype) {
  if (N < 0 || D <= 0 || V <= 0 || (dtype != kDtypeBf16 && dtype != kDtypeF32)) return 0;
  return make_layout(N, D, V, dtype, 0, nullptr, nullptr).state_total;
}

size_t cce_workspace_size(int64_t N, int64_t D, int64_t V, int dtype, int64_t vocab_chunk) {
  if (N < 0 || D <= 0 || V <= 0 || (dtype != kDtypeBf16 && dtype != kDtypeF32)) return 0;
  if (vocab_chunk < 0 || vocab_chunk % kTileV != 0) return 0;
  return make_layout(N, D, V, dtype, vocab_chunk, nullptr, nullptr).total;
}

int64_t cce_vocab_chunk(int64_t N, int64_t D, int64_t V, int dtype, int64_t vocab_chunk) {
  if (N < 0 || D <= 0 || V <= 0 || (dtype != kDtypeBf16 && dtype != kDtypeF32)) return 0;
  if (vocab_chunk < 0 || vocab_chunk % kTileV != 0) return 0;
  return make_layout(N, D, V, dtype, vocab_chunk, nullptr, nullptr).Vc;
}

static bool bias_ok(const void* bias, int dtype) {
  return ((uintptr_t)bias & (dtype == kDtypeBf16 ? 1u : 3u)) == 0;
}

// eps in [0, 1] and lam >= 0, both finite (NaN fails every comparison)
static bool terms_ok(float label_smoothing, float z_loss) {
  return label_smoothing >= 0.0f && label_smoothing <= 1.0f && z_loss >= 0.0f && z_loss <= 3.0e38f;
}

cce_status cce_forward(const void* e, const void* c, const void* bias, const int64_t* targets, int64_t N,
                       int64_t D, int64_t V, int dtype, int64_t ignore_index, int reduction, float softcap,
                       float label_smoothing, float z_loss, float* loss, float* lse, int32_t* n_valid, void* state,
                       size_t state_bytes, cce_stream_t stream) {
  cce_status st = check_common(e, c, targets, N, D, V, dtype, reduction, softcap, state, 0);
  if (st != CCE_OK) return st;
  if (!bias_ok(bias, dtype) || !terms_ok(label_smoothing, z_loss)) return CCE_ERR_INVALID_ARG;
  if (softcap > 0.0f && label_smoothing > 0.0f) return CCE_ERR_UNSUPPORTED;
  // with N = 0, lse and a per-row loss have no elements (may be null)
  if ((N > 0 && !lse) || ((N > 0 || reduction != kReductionNone) && !loss)) return CCE_ERR_INVALID_ARG;
  Layout L = make_layout(N, D, V, dtype, 0, state, nullptr);
  if (state_bytes < L.state_total) return CCE_ERR_WORKSPACE;
  if (N == 0) {
    const hipError_t err = launch_empty(L, reduction == kReductionNone ? nullptr : loss, n_valid, nullptr, 0,
                                        nullptr, 0, (hipStream_t)stream);
    return err == hipSuccess ? CCE_OK : CCE_ERR_HIP;
  }
  if (reduction == kReductionNone) L.nll_out = loss;
  Problem P{};
  P.e = e;
  P.c = c;
  P.bias = bias;
  P.targets = targets;
  P.N = (int)N;
  P.D = (int)D;
  P.V = (int)V;
  P.dtype = dtype;
  P.ignore_index = ignore_index;
  P.reduction = reduction;
  P.label_smoothing = label_smoothing;
  P.z_loss = z_loss;
  P.softcap = softcap;
  P.loss = loss;
  P.lse = lse;
  P.n_valid = n_valid;
  hipError_t err = launch_forward(P, L, (hipStream_t)stream);
  return err == hipSuccess ? CCE_OK : CCE_ERR_HIP;
}

cce_status cce_backward(const void* e, const void* c, const void* bias, const int64_t* targets, int64_t N,
                        int64_t D, int64_t V, int dtype, int64_t ignore_index, int reduction, float softcap,
                        float label_smoothing, float z_loss, const float* lse, const float* grad_loss, int filter,
                        int accum, int64_t vocab_chunk, int grad_dtype, void* dE, void* dC, float* dbias,
                        void* state, size_t state_bytes, void* ws, size_t ws_bytes, cce_stream_t stream) {
  cce_status st = check_common(e, c, targets, N, D, V, dtype, reduction, softcap, state, vocab_chunk);
  if (st != CCE_OK) return st;
  if (!bias_ok(bias, dtype) || ((uintptr_t)dbias & 3u) || !terms_ok(label_smoothing, z_loss))
    return CCE_ERR_INVALID_ARG;
  if (softcap > 0.0f && label_smoothing > 0.0f) return CCE_ERR_UNSUPPORTED;
  // each gradient is optional (null: not formed), at least one is asked for
  if ((N > 0 && (!lse || !grad_loss)) || (!dE && !dC && !dbias)) return CCE_ERR_INVALID_ARG;
  if ((filter != 0 && filter != 1) || (accum != kAccumDeterministic && accum != kAccumAtomic))
    return CCE_ERR_INVALID_ARG;
  if (grad_dtype != CCE_GRAD_FLOAT32 && grad_dtype != CCE_GRAD_OPERAND) return CCE_ERR_INVALID_ARG;
  if ((dE && !aligned16(dE)) || (dC && !aligned16(dC)) || !ws || !aligned16(ws)) return CCE_ERR_INVALID_ARG;
  Layout L = make_layout(N, D, V, dtype, vocab_chunk, state, ws);
  if (state_bytes < L.state_total || ws_bytes < L.total) return CCE_ERR_WORKSPACE;
  if (N == 0) {
    // no rows: dC and db are zero (the smoothing term included), dE is empty
    const size_t ges = grad_dtype == CCE_GRAD_OPERAND && dtype == kDtypeBf16 ? 2 : 4;
    const hipError_t err =
        launch_empty(L, nullptr, nullptr, dC, dC ? (size_t)V * (size_t)D * ges : 0, dbias, (size_t)V,
                     (hipStream_t)stream);
    return err == hipSuccess ? CCE_OK : CCE_ERR_HIP;
  }
  Problem P{};
  P.e = e;
  P.c = c;
  P.bias = bias;
  P.targets = targets;
  P.N = (int)N;
  P.D = (int)D;
  P.V = (int)V;
  P.dtype = dtype;
  P.ignore_index = ignore_index;
  P.reduction = reduction;
  P.label_smoothing = label_smoothing;
  P.z_loss = z_loss;
  P.softcap = softcap;
  P.lse = (float*)lse;
  P.grad_loss = grad_loss;
  P.filter = filter;
  P.accum = accum;
  P.dE = dE;
  P.dC = dC;
  P.dbias = dbias;
  P.grad_bf16 = grad_dtype == CCE_GRAD_OPERAND && dtype == kDtypeBf16 ? 1 : 0;
  hipError_t err = launch_backward(P, L, (hipStream_t)stream);
  return err == hipSuccess ? CCE_OK : CCE_ERR_HIP;
}

cce_status cce_read_stats(const void* state, size_t state_bytes, int64_t N, int64_t V, cce_stream_t stream,
                          cce_stats* out) {
  if (!state || !out || state_bytes < (size_t)kHdrWords * 4 || N < 0 || V <= 0) return CCE_ERR_INVALID_ARG;
  int32_t h[kHdrWords];
  if (hipMemcpyAsync(h, state, sizeof(h), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess)
    return CCE_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return CCE_ERR_HIP;
  out->n_valid = h[kHdrNValid];
  out->bad_targets = h[kHdrBadTargets];
  out->tiles_total = ((N + kTileN - 1) / kTileN) * ((V + kTileV - 1) / kTileV);
  out->tiles_kept = h[kHdrTilesKept];
  out->filter_rows = kTileN;
  out->filter_vocab = kTileV;
  out->blocks_total = ((N + kBlock - 1) / kBlock) * ((V + kBlock - 1) / kBlock);
  out->blocks_kept = h[kHdrBlocksKept];
  out->block_rows = kBlock;
  out->block_vocab = kBlock;
  return CCE_OK;
}

cce_status cce_read_keep_map(const void* ws, size_t ws_bytes, int64_t N, int64_t D, int64_t V, int dtype,
                             int64_t vocab_chunk, uint8_t* out, cce_stream_t stream) {
  if (!ws || !out || N < 0 || D <= 0 || V <= 0 || (dtype != kDtypeBf16 && dtype != kDtypeF32) ||
      vocab_chunk < 0 || vocab_chunk % kTileV != 0)
    return CCE_ERR_INVALID_ARG;
  const Layout L = make_layout(N, D, V, dtype, vocab_chunk, nullptr, const_cast<void*>(ws));
  if (ws_bytes < L.total) return CCE_ERR_WORKSPACE;
  const size_t n = (size_t)((N + kTileN - 1) / kTileN) * (size_t)L.nvb_t;
  if (n == 0) return CCE_OK;
  if (hipMemcpyAsync(out, L.keep, n, hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess) return CCE_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return CCE_ERR_HIP;
  return CCE_OK;
}

cce_status cce_read_block_map(const void* ws, size_t ws_bytes, int64_t N, int64_t D, int64_t V, int dtype,
                              int64_t vocab_chunk, uint8_t* out, cce_stream_t stream) {
  if (!ws || !out || N < 0 || D <= 0 || V <= 0 || (dtype != kDtypeBf16 && dtype != kDtypeF32) ||
      vocab_chunk < 0 || vocab_chunk % kTileV != 0)
    return CCE_ERR_INVALID_ARG;
  const Layout L = make_layout(N, D, V, dtype, vocab_chunk, nullptr, const_cast<void*>(ws));
  if (ws_bytes < L.total) return CCE_ERR_WORKSPACE;
  const int64_t nrb = (N + kBlock - 1) / kBlock, nvg = (V + kBlock - 1) / kBlock;
  if (nrb == 0) return CCE_OK;
  const int64_t nbk = (N + kTileN - 1) / kTileN;
  std::vector<uint8_t> bytes((size_t)(nbk * L.nvg));
  if (hipMemcpyAsync(bytes.data(), L.bmask, bytes.size(), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess)
    return CCE_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return CCE_ERR_HIP;
  // byte (token block, vocab group) holds one bit per 32-row group of the block
  for (int64_t r = 0; r < nrb; ++r)
    for (int64_t g = 0; g < nvg; ++g)
      out[r * nvg + g] = (bytes[(size_t)((r / kBlocksPerTile) * L.nvg + g)] >> (r % kBlocksPerTile)) & 1u;
  return CCE_OK;
}

const char* cce_status_string(int status) {
  switch (status) {
    case CCE_OK: return "ok";
    case CCE_ERR_INVALID_ARG: return "invalid argument";
    case CCE_ERR_UNSUPPORTED: return "unsupported configuration";
    case CCE_ERR_WORKSPACE: return "workspace too small";
    case CCE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

cce_status cce_profile_start(int kernel_id, int max_launches) {
  if (kernel_id < 0 || kernel_id >= kNumKernels || max_launches <= 0) return CCE_ERR_INVALID_ARG;
  ProfSlot& p = g_prof[kernel_id];
  prof_release(p);
  p.ev.resize(2 * (size_t)max_launches);
  for (auto& e : p.ev)
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      prof_release(p);
      return CCE_ERR_HIP;
    }
  p.cap = max_launches;
  p.active = true;
  return CCE_OK;
}

cce_status cce_profile_stop(int kernel_id, double* total_ms, int* launches) {
  if (kernel_id < 0 || kernel_id >= kNumKernels || !total_ms || !launches) return CCE_ERR_INVALID_ARG;
  ProfSlot& p = g_prof[kernel_id];
  double tot = 0.0;
  cce_status st = CCE_OK;
  for (int i = 0; i < p.n; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(p.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]) != hipSuccess) {
      st = CCE_ERR_HIP;
      break;
    }
    tot += ms;
  }
  *total_ms = tot;
  *launches = p.n;
  prof_release(p);
  return st;
}

const char* cce_kernel_name(int kernel_id) {
  return (kernel_id >= 0 && kernel_id < kNumKernels) ? kKernelNames[kernel_id] : "unknown";
}

void cce_tile_shape(int* filter_rows, int* filter_vocab, int* partial_vocab) {
  if (filter_rows) *filter_rows = kTileN;
  if (filter_vocab) *filter_vocab = kTileV;
  if (partial_vocab) *partial_vocab = kPartialWidth;
}

}  // extern "C"
