// HIP kernels for the fused linear cross-entropy on gfx950.
//
// Method (Wijmans et al., "Cut Your Losses in Large-Vocabulary Language
// Models", abstract; mlx-cross-entropy README, "How it works"):
//   loss_i = LSE_j(e_i . c_j) - e_i . c_{y_i}, with the [N, V] logits formed
//   only tile by tile in registers, never in global memory.
//
// Forward:  fwd_tile      S^T tile = C_v E_b^T on MFMA, per (token, 128-vocab
//                         block) max m and sum-exp s written as partials
//           rows          correct-token gather-dot, LSE = combine of partials,
//                         per-row loss (ignore mask)
//           reduce        fixed-order mean / sum and the exact valid count
//           colsum(+reduce) with label smoothing: sum over the vocabulary of
//                         the classifier rows (and vec_sum of the bias), so
//                         that sum_j z_ij = e_i . csum + sum_j b_j
// Backward: bwd_prep      per-row gradient scale (mean/sum/none, ignore mask)
//                         and the compaction of the token rows: the backward
//                         works on the valid rows first, ignored rows after
//                         (whole blocks of them drop out), reading and writing
//                         token rows through that permutation
//           filter        tile keep map: a (token block, vocab block) tile is
//                         kept iff some valid row's softmax reaches 2^-12 on it
//                         (README "How it works" item 2, using the forward's
//                         per-block maxima) or holds a valid row's target
//           grad_tile     recompute S for kept tiles, G = (p - onehot) * scale
//                         rounded to the operand type, into a vocab chunk of G
//           dC_gemm       dC[v] = sum over kept token blocks of G^T E
//           dE_gemm       dE   += sum over kept vocab blocks of G C
//                         (split over vocab, fixed-order partial reduce, or
//                         fp32 atomics)
// Label smoothing eps makes the target (1 - eps) onehot + eps / V and z-loss
// lam adds lam LSE^2 (tirogla "Loss functions", step 3 and "Implementation
// notes"), so G = (p (1 + 2 lam LSE) - (1 - eps) onehot) * scale - eps / V *
// scale.  The last term is the same for every vocabulary entry of a row: the
// tiles carry the rest, and its rank-one share of dE, dC and db (a row scale
// times the classifier column sum, minus eps/V times sum_i scale_i e_i, minus
// eps/V times sum_i scale_i) is added in the epilogues, exactly, kept tile or
// not.
#include "cce_gemm.hpp"
#include "cce_internal.hpp"

namespace cce {

constexpr float kLog2e = 1.4426950408889634f;
// M tiles per group of the grouped tile order (see grouped_tile), per kernel:
// the forward and dE keep 8 (their groups share the classifier tiles / the G
// rows of 8 tiles), the gradient tiles and dC 4 (measured: 8 -> 4 made both
// about 1% faster at the 8B head, the forward and dE about 0.7% slower; 16
// was slower everywhere).
constexpr int kRasterFwd = 8;
constexpr int kRasterGrad = 4;
constexpr int kRasterDC = 4;
constexpr int kRasterDE = 8;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Logit soft-capping s tanh(z / s) (the Gemma 2 form; the pages do not define
// it), from tanh(x) = 1 - 2 / (exp(2x) + 1): s - 2s / (exp2(z k) + 1) with
// k = 2 log2(e) / s.  Saturates to +-s exactly (exp2 gives inf or 0); near 0
// the absolute error is a few ulp of s.
__device__ __forceinline__ float softcap_f(float z, float s, float k) {
  return __builtin_fmaf(-2.f * s, __builtin_amdgcn_rcpf(fast_exp2(z * k) + 1.f), s);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Work-groups are dispatched round-robin over the 8 XCDs (WG i on XCD i % 8).
// Give each XCD a contiguous run of logical tiles so that tiles sharing an
// operand block run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int i, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = i & 7, j = i >> 3;
  return x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

// Grouped ordering of an (tiles_m x tiles_n) tile grid: runs of `group`
// consecutive M tiles are visited for every N tile before the next run, so
// the ~32 work-groups an XCD holds at once cover about group x (32/group)
// tiles and re-use group A blocks and 32/group B blocks from its L2.
__device__ __forceinline__ void grouped_tile(int idx, int tiles_m, int tiles_n, int group, int& tm, int& tn) {
  const int per = group * tiles_n;
  const int g = idx / per;
  const int first = g * group;
  const int gm = min(tiles_m - first, group);
  const int r = idx - g * per;
  tm = first + r % gm;
  tn = r / gm;
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<uint16_t>(uint16_t v) {
  return __builtin_bit_cast(float, (uint32_t)v << 16);
}
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }

// The classifier bias of a 256-row vocabulary tile, as fp32, into LDS (rows
// past V, and every row without a bias, read 0).  Visible to the waves after
// the main loop's first barrier.
template <typename T, int ROWS>
__device__ __forceinline__ void stage_bias(float* sb, const T* __restrict__ bias, int v0, int V) {
  for (int i = threadIdx.x; i < ROWS; i += blockDim.x) sb[i] = (bias && v0 + i < V) ? to_f<T>(bias[v0 + i]) : 0.f;
}
// Bias of the four consecutive tile rows r..r+3 (r a multiple of 4).
__device__ __forceinline__ f32x4 bias4(const float* sb, int r) {
  return *(const __attribute__((address_space(3))) f32x4*)(
      (const __attribute__((address_space(3))) float*)sb + r);
}

// Four consecutive fp32 values in the operand type, packed for one store.
__device__ __forceinline__ void store4(rsrc_t r, uint32_t off, float a, float b, float c, float d,
                                       const uint16_t*) {
  __bf16 x0 = (__bf16)a, x1 = (__bf16)b, x2 = (__bf16)c, x3 = (__bf16)d;
  uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, x0) | ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
  uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, x2) | ((uint32_t)__builtin_bit_cast(uint16_t, x3) << 16);
  u32x2 v = {lo, hi};
  st64(r, off, v);
}
__device__ __forceinline__ void store4(rsrc_t r, uint32_t off, float a, float b, float c, float d,
                                       const float*) {
  u32x4 v = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
             __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// Lane-quad exchange (DPP quad_perm): value of lane (k ^ 2) or (k ^ 1).
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
}
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// 4x4 transpose of 32-bit values across a lane quad: on entry lane k holds
// d[u] = x[k][u] (in the accumulator layout: four consecutive rows u of the
// lane's own column k), on exit d[u] = x[u][k] (row k, four consecutive
// columns u), after two quad exchanges.
__device__ __forceinline__ void quad_transpose(uint32_t (&d)[4]) {
  const int k = threadIdx.x & 3;
  // rows {2,3} of lanes {0,1} <-> rows {0,1} of lanes {2,3}
  const bool k2 = (k & 2) != 0, k1 = (k & 1) != 0;
  {
    const uint32_t s0 = quad_xor2(k2 ? d[0] : d[2]);
    const uint32_t s1 = quad_xor2(k2 ? d[1] : d[3]);
    d[0] = k2 ? s0 : d[0];
    d[1] = k2 ? s1 : d[1];
    d[2] = k2 ? d[2] : s0;
    d[3] = k2 ? d[3] : s1;
  }
  // odd rows of even lanes <-> even rows of odd lanes
  {
    const uint32_t s0 = quad_xor1(k1 ? d[0] : d[1]);
    const uint32_t s1 = quad_xor1(k1 ? d[2] : d[3]);
    d[0] = k1 ? s0 : d[0];
    d[2] = k1 ? s1 : d[2];
    d[1] = k1 ? d[1] : s0;
    d[3] = k1 ? d[3] : s1;
  }
}

// Transposed store of the 4x4 fp32 block held by a lane quad (see
// quad_transpose): lane k writes row k, the quad's four columns, as one
// 16-byte store.  `off_row0` is the byte offset of (row 0, the quad's first
// column), `ld` the row pitch in bytes.
__device__ __forceinline__ void store_quad_t(rsrc_t r, uint32_t off_row0, uint32_t ld, const float (&x)[4],
                                             const float*) {
  uint32_t d[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) d[u] = __builtin_bit_cast(uint32_t, x[u]);
  quad_transpose(d);
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{d[0], d[1], d[2], d[3]}, r,
                                         off_row0 + (uint32_t)(threadIdx.x & 3) * ld, 0, 0);
}

// ============================================================================
// e^T [D][Npad] in compacted slot order (padding slots zero) for the dC
// contraction, via 64x64 LDS tiles.
// ============================================================================
template <typename T>
__global__ __launch_bounds__(256) void transpose_e_kernel(const T* __restrict__ e, const int* __restrict__ rowmap,
                                                          T* __restrict__ et, int N, int D, int Npad) {
  __shared__ T tile[64][65];
  const int d0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int n = n0 + r, d = d0 + tx;
    const int src = rowmap[n];  // token row of compacted slot n (-1: padding)
    tile[r][tx] = (src >= 0 && d < D) ? e[(size_t)src * D + d] : (T)0;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int d = d0 + r, n = n0 + tx;
    if (d < D && n < Npad) et[(size_t)d * Npad + n] = tile[tx][r];
  }
}

// ============================================================================
// Forward logit tile + per-block online LSE partials.
// Output tile rows are vocabulary entries, columns are tokens, so each lane
// holds 16 vocab values of one token per 32x32 block and the vocabulary
// reduction is mostly in-lane.
// ============================================================================
template <class C>
__global__ __launch_bounds__(C::NT, 1) void fwd_tile_kernel(const typename C::T* __restrict__ c,
                                                            const typename C::T* __restrict__ e,
                                                            const typename C::T* __restrict__ bias,
                                                            int N, int D, int V, float softcap,
                                                            float2* __restrict__ part, int nVB, int tiles_n,
                                                            int total) {
  using T = typename C::T;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_DMA_BYTES];
  __shared__ __attribute__((aligned(16))) float sbias[C::BM];
  int tv, tn;
  grouped_tile(xcd_remap(blockIdx.x, total), total / tiles_n, tiles_n, kRasterFwd, tv, tn);
  const int v0 = tv * C::BM, n0 = tn * C::BN;
  if (bias || softcap > 0.f) stage_bias<T, C::BM>(sbias, bias, v0, V);

  Operand A = make_operand(c + (size_t)v0 * D, (uint64_t)(V - v0) * D * sizeof(T), (uint32_t)D,
               min(C::BM, V - v0), D);
  Operand B = make_operand(e + (size_t)n0 * D, (uint64_t)(N - n0) * D * sizeof(T), (uint32_t)D,
               min(C::BN, N - n0), D);
  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};
  mainloop_dma<C, 1>(acc, A, B, (D + C::BK - 1) / C::BK, nullptr, smem);

  AccMap<C> am;
  const int lane = threadIdx.x & 63;
  const int wm = (threadIdx.x >> 6) / C::WAVES_N;
  const int vblk = (v0 + wm * C::WM) / C::WM;
  // logits of this lane's 64 rows of column fn (plus the rows' bias); rows
  // past V are left out only in the last vocab tile (ragged)
  auto emit = [&](auto has_bias, auto ragged) __attribute__((always_inline)) {
    f32x4 bz[C::FM][4];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int q = 0; q < 4; ++q) bz[fm][q] = decltype(has_bias)::value ? bias4(sbias, am.row(fm, 4 * q)) : f32x4{};
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int n = n0 + am.colj(fn);
      auto z = [&](int fm, int r) { return acc[fm][fn][r] + bz[fm][r >> 2][r & 3]; };
      auto in = [&](int fm, int r) { return !decltype(ragged)::value || v0 + am.row(fm, r) < V; };
      float mx = -INFINITY;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (in(fm, r)) mx = fmaxf(mx, z(fm, r));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mxl = mx * kLog2e;
      float s = 0.f;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (in(fm, r)) s += fast_exp2(__builtin_fmaf(z(fm, r), kLog2e, -mxl));
      s += __shfl_xor(s, 32, 64);
      if (lane < 32 && n < N && vblk < nVB) part[(size_t)n * nVB + vblk] = make_float2(mx, s);
    }
  };
  if (sizeof(T) == 2 && softcap > 0.f) {
    // capped logits (bias included) in place, then the plain epilogue (bf16
    // operands only: the host rejects soft-capping with fp32)
    const float kc = 2.f * kLog2e / softcap;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 bz = bias4(sbias, am.row(fm, 4 * q));
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            acc[fm][fn][4 * q + u] = softcap_f(acc[fm][fn][4 * q + u] + bz[u], softcap, kc);
      }
    if (v0 + C::BM <= V) emit(std::false_type{}, std::false_type{});
    else emit(std::false_type{}, std::true_type{});
  } else if (bias) {
    if (v0 + C::BM <= V) emit(std::true_type{}, std::false_type{});
    else emit(std::true_type{}, std::true_type{});
  } else {
    if (v0 + C::BM <= V) emit(std::false_type{}, std::false_type{});
    else emit(std::false_type{}, std::true_type{});
  }
}

// ============================================================================
// Per-row: correct-token logit (gather-dot), LSE from the partials, loss.
// One wave per row.
// ============================================================================
// With SMOOTH, also e_i . csum (plus the bias sum aux[0]) = sum_j z_ij, the
// smoothing term's logit sum.  loss_i = LSE - (1 - eps) z_y - eps / V sum_j
// z_ij + lam LSE^2 (the soft-target cross-entropy, since the target sums to 1).
template <typename T, bool SMOOTH>
__global__ __launch_bounds__(256) void rows_kernel(const T* __restrict__ e, const T* __restrict__ c,
                                                   const T* __restrict__ bias,
                                                   const int64_t* __restrict__ targets, int N, int D,
                                                   int V, int64_t ignore_index,
                                                   const float2* __restrict__ part, int nVB,
                                                   const float* __restrict__ csum, const float* __restrict__ aux,
                                                   float eps, float lam, float softcap,
                                                   float* __restrict__ lse_out, float* __restrict__ nll) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= N) return;
  const int64_t t = targets[i];
  const bool valid = t != ignore_index;
  const bool inrange = t >= 0 && t < V;
  constexpr int VEC = Elem<T>::VEC;

  float zy = 0.f, zs = 0.f;
  if (valid && inrange) {
    // plain global loads: the row pointers differ per wave, and the loop bound
    // keeps every 16-byte access inside the row
    const T* er = e + (size_t)i * D;
    const T* cr = c + (size_t)t * D;
    float acc = 0.f, accs = 0.f;
    for (int k = lane * VEC; k < D; k += 64 * VEC) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(er + k);
      const u32x4 b = *reinterpret_cast<const u32x4*>(cr + k);
      float cs[VEC];
      if constexpr (SMOOTH) {
#pragma unroll
        for (int h = 0; h < VEC / 4; ++h) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(csum + k + 4 * h);
#pragma unroll
          for (int u = 0; u < 4; ++u) cs[4 * h + u] = v[u];
        }
      }
      // (vector elements are copied to scalars before any bit cast: clang
      // mis-lowers a bit cast applied directly to a vector-element lvalue)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x = a[q], y = b[q];
        if constexpr (sizeof(T) == 2) {
          const float x0 = __builtin_bit_cast(float, x << 16), x1 = __builtin_bit_cast(float, x & 0xffff0000u);
          acc = __builtin_fmaf(x0, __builtin_bit_cast(float, y << 16), acc);
          acc = __builtin_fmaf(x1, __builtin_bit_cast(float, y & 0xffff0000u), acc);
          if constexpr (SMOOTH) {
            accs = __builtin_fmaf(x0, cs[2 * q], accs);
            accs = __builtin_fmaf(x1, cs[2 * q + 1], accs);
          }
        } else {
          const float x0 = __builtin_bit_cast(float, x);
          acc = __builtin_fmaf(x0, __builtin_bit_cast(float, y), acc);
          if constexpr (SMOOTH) accs = __builtin_fmaf(x0, cs[q], accs);
        }
      }
    }
    zy = wave_sum(acc);
    if (bias) zy += to_f<T>(bias[t]);
    if (softcap > 0.f) zy = softcap_f(zy, softcap, 2.f * kLog2e / softcap);
    if constexpr (SMOOTH) {
      zs = wave_sum(accs);
      if (bias) zs += aux[0];
    }
  }

  const float2* p = part + (size_t)i * nVB;
  float m = -INFINITY;
  for (int v = lane; v < nVB; v += 64) m = fmaxf(m, p[v].x);
  m = wave_max(m);
  const float ml = m * kLog2e;
  float s = 0.f;
  for (int v = lane; v < nVB; v += 64) {
    float2 q = p[v];
    s += q.y * fast_exp2(__builtin_fmaf(q.x, kLog2e, -ml));
  }
  s = wave_sum(s);
  const float lse = m + fast_log2(s) * kLn2;
  if (lane == 0) {
    lse_out[i] = lse;
    float l = lse - (1.f - eps) * zy + lam * lse * lse;
    if constexpr (SMOOTH) l -= eps / (float)V * zs;
    nll[i] = valid ? (inrange ? l : __builtin_nanf("")) : 0.f;
  }
}

// ============================================================================
// Fixed-order reduction of the per-row losses (one work-group), exact counts.
// ============================================================================
__global__ __launch_bounds__(1024) void reduce_kernel(const float* __restrict__ nll,
                                                      const int64_t* __restrict__ targets, int N, int V,
                                                      int64_t ignore_index, int reduction,
                                                      float* __restrict__ loss, int32_t* __restrict__ n_valid,
                                                      int32_t* __restrict__ hdr) {
  __shared__ double ssum[1024];
  __shared__ int scnt[1024], sbad[1024];
  const int tid = threadIdx.x;
  double acc = 0.0;
  int cnt = 0, bad = 0;
  for (int i = tid; i < N; i += 1024) {
    const int64_t t = targets[i];
    if (t != ignore_index) {
      ++cnt;
      if (t < 0 || t >= V) ++bad;
    }
    if (reduction != kReductionNone) acc += (double)nll[i];
  }
  ssum[tid] = acc;
  scnt[tid] = cnt;
  sbad[tid] = bad;
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
    if (tid < o) {
      ssum[tid] += ssum[tid + o];
      scnt[tid] += scnt[tid + o];
      sbad[tid] += sbad[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int nv = scnt[0];
    if (reduction == kReductionSum) loss[0] = (float)ssum[0];
    else if (reduction == kReductionMean) loss[0] = (float)(ssum[0] / (double)(nv > 0 ? nv : 1));
    if (n_valid) n_valid[0] = nv;
    hdr[kHdrNValid] = nv;
    hdr[kHdrBadTargets] = sbad[0];
  }
}

// ============================================================================
// Column sums for the label-smoothing term.  part[b][d] = sum over the rows r
// of row block b (rows [b rpb, (b + 1) rpb)) of w_r x[r][d], w = 1 when null;
// then out[d] = factor * sum_b part[b][d].  A thread owns one 16-byte column
// group and walks its block's rows in order, eight loads in flight; both
// passes add in a fixed order (deterministic).
// ============================================================================
template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(const T* __restrict__ x, const float* __restrict__ w, int R,
                                                     int D, int rpb, float* __restrict__ part) {
  constexpr int VEC = Elem<T>::VEC;
  const int d = (blockIdx.x * 256 + threadIdx.x) * VEC;
  if (d >= D) return;
  const int r0 = blockIdx.y * rpb, r1 = min(R, r0 + rpb);
  float acc[VEC] = {};
  auto add = [&](const u32x4& v, float wr) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t u = v[q];
      if constexpr (sizeof(T) == 2) {
        acc[2 * q] = __builtin_fmaf(wr, __builtin_bit_cast(float, u << 16), acc[2 * q]);
        acc[2 * q + 1] = __builtin_fmaf(wr, __builtin_bit_cast(float, u & 0xffff0000u), acc[2 * q + 1]);
      } else {
        acc[q] = __builtin_fmaf(wr, __builtin_bit_cast(float, u), acc[q]);
      }
    }
  };
  int r = r0;
  for (; r + 8 <= r1; r += 8) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const u32x4*>(x + (size_t)(r + k) * D + d);
#pragma unroll
    for (int k = 0; k < 8; ++k) add(v[k], w ? w[r + k] : 1.f);
  }
  for (; r < r1; ++r) add(*reinterpret_cast<const u32x4*>(x + (size_t)r * D + d), w ? w[r] : 1.f);
  float* o = part + (size_t)blockIdx.y * D + d;
#pragma unroll
  for (int h = 0; h < VEC / 4; ++h)
    *reinterpret_cast<f32x4*>(o + 4 * h) = f32x4{acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]};
}

// 64 columns per work-group: wave w adds the blocks [w nblk/16, (w+1) nblk/16)
// of its lane's column, then the 16 wave sums are added in wave order.
__global__ __launch_bounds__(1024) void colsum_reduce_kernel(const float* __restrict__ part, int nblk, int D,
                                                             float factor, float* __restrict__ out) {
  __shared__ float sw[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = blockIdx.x * 64 + lane;
  const int b0 = nblk * w / 16, b1 = nblk * (w + 1) / 16;
  float s = 0.f;
  if (d < D) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) s += part[(size_t)b * D + d];
  }
  sw[w][lane] = s;
  __syncthreads();
  if (w == 0 && d < D) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += sw[k][lane];
    out[d] = factor * t;
  }
}

// out[0] = sum of x[0..n) (one work-group, fixed order).
template <typename T>
__global__ __launch_bounds__(1024) void vec_sum_kernel(const T* __restrict__ x, int n, float* __restrict__ out) {
  __shared__ float s[1024];
  float a = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) a += to_f<T>(x[i]);
  s[threadIdx.x] = a;
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = s[0];
}

// ============================================================================
// Backward preparation (one work-group).  Per row, in the original order, the
// scale d(loss)/d(nll_i) times the upstream gradient: 0 if ignored, NaN for an
// out-of-range target, 0 past N.  The compaction of the token rows (the Loss
// functions page, "Efficiency": skip padded rows): slot n' of rowmap holds the
// valid rows in order, then the ignored rows in order, then -1 for the slots
// [N, Npad); per slot, scale_c, lse_c and tgt_c give the row's scale, LSE and
// target, with scale 0, LSE +inf and target -1 for ignored rows and padding,
// so that their gradient entries come out exactly 0.
// ============================================================================
__global__ __launch_bounds__(1024) void bwd_prep_kernel(const int64_t* __restrict__ targets, int N,
                                                        int Npad, int V, int64_t ignore_index,
                                                        int reduction, const float* __restrict__ grad_loss,
                                                        const float* __restrict__ lse,
                                                        float* __restrict__ scale, int* __restrict__ rowmap,
                                                        float* __restrict__ scale_c, float* __restrict__ lse_c,
                                                        int* __restrict__ tgt_c, int32_t* __restrict__ hdr,
                                                        float* __restrict__ scale_sum) {
  __shared__ int scnt[1024];
  __shared__ float ssum[1024];
  const int tid = threadIdx.x;
  // each thread owns a contiguous run of rows; an inclusive scan of the runs'
  // valid counts places them
  const int chunk = (N + 1023) / 1024;
  const int i0 = min(N, tid * chunk), i1 = min(N, i0 + chunk);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += targets[i] != ignore_index;
  scnt[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? scnt[tid - o] : 0;
    __syncthreads();
    scnt[tid] += v;
    __syncthreads();
  }
  const int nv = scnt[1023];
  int vslot = scnt[tid] - cnt;        // valid rows before this run
  int islot = nv + (i0 - vslot);      // slot of this run's first ignored row
  const float g0 = reduction == kReductionNone ? 0.f : grad_loss[0];
  const float gm = reduction == kReductionMean ? (float)((double)g0 / (double)(nv > 0 ? nv : 1)) : g0;
  float acc = 0.f;
  for (int i = i0; i < i1; ++i) {
    const int64_t t = targets[i];
    if (t != ignore_index) {
      const bool inrange = t >= 0 && t < V;
      float sv = reduction == kReductionNone ? grad_loss[i] : gm;
      if (!inrange) sv = __builtin_nanf("");
      scale[i] = sv;
      acc += sv;
      rowmap[vslot] = i;
      scale_c[vslot] = sv;
      lse_c[vslot] = lse[i];
      tgt_c[vslot] = inrange ? (int)t : -1;
      ++vslot;
    } else {
      scale[i] = 0.f;
      rowmap[islot] = i;
      scale_c[islot] = 0.f;
      lse_c[islot] = INFINITY;
      tgt_c[islot] = -1;
      ++islot;
    }
  }
  for (int n = N + tid; n < Npad; n += 1024) {
    scale[n] = 0.f;
    rowmap[n] = -1;
    scale_c[n] = 0.f;
    lse_c[n] = INFINITY;
    tgt_c[n] = -1;
  }
  if (tid == 0) {
    hdr[kHdrNValidBwd] = nv;
    hdr[kHdrTilesKept] = 0;
    hdr[kHdrBlocksKept] = 0;
  }
  if (scale_sum) {  // sum_i scale_i, fixed order (the smoothing share of db)
    ssum[tid] = acc;
    __syncthreads();
    for (int o = 512; o >= 1; o >>= 1) {
      if (tid < o) ssum[tid] += ssum[tid + o];
      __syncthreads();
    }
    if (tid == 0) scale_sum[0] = ssum[0];
  }
}

// ============================================================================
// Backward: tile keep map.  Work-group = one token block x 64 vocab blocks.
// ============================================================================
__global__ __launch_bounds__(1024) void filter_kernel(const int64_t* __restrict__ targets,
                                                     const float* __restrict__ lse,
                                                     const float2* __restrict__ part, const int* __restrict__ rowmap,
                                                     int N, int V, int nVB, int64_t ignore_index, int nvb_t,
                                                     int filter, uint8_t* __restrict__ keep,
                                                     uint8_t* __restrict__ bmask, int nvg,
                                                     int32_t* __restrict__ hdr) {
  constexpr int Bn = kTileN, PPB = kTileV / kPartialWidth;  // partial blocks per vocab tile
  __shared__ float s_lse[Bn];
  __shared__ int s_tb[Bn], s_row[Bn];
  __shared__ int s_any;
  constexpr int NW = 16;  // waves
  __shared__ uint8_t s_k[NW][64];
  const int b = blockIdx.y;  // block of compacted token slots
  const int tid = threadIdx.x;
  if (tid == 0) s_any = 0;
  __syncthreads();
  for (int r = tid; r < Bn; r += blockDim.x) {
    const int slot = b * Bn + r;
    const int i = slot < N ? rowmap[slot] : -1;
    float l = INFINITY;
    int tb = -1;
    if (i >= 0) {
      const int64_t t = targets[i];
      if (t != ignore_index) {
        s_any = 1;
        if (t >= 0 && t < V) {
          l = lse[i];
          tb = (int)(t / kTileV);
        }
      }
    }
    s_lse[r] = l;
    s_tb[r] = tb;
    s_row[r] = i;
  }
  __syncthreads();
  // lane = vocab block (a wave reads consecutive partials of one row), wave w
  // = rows w, w + 16, ...: all sixteen rows' loads in flight at once; the
  // sixteen waves' answers are then combined
  const int lane = tid & 63, w = tid >> 6;
  const int vb = blockIdx.x * 64 + lane;
  bool k = false;
  if (!filter) {
    k = s_any != 0;  // a block of ignored rows only has G = 0: never computed
  } else if (vb < nvb_t) {
    const float thr = -12.0f * kLn2;
    constexpr int U = Bn / NW;
    static_assert(Bn % NW == 0, "rows per wave");
    {
      const int r0 = w;
      float m[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + NW * u;
        m[u] = -INFINITY;
        if (r < Bn && s_tb[r] >= 0) {
          const float2* p = part + (size_t)s_row[r] * nVB + (size_t)vb * PPB;
#pragma unroll
          for (int q = 0; q < PPB; ++q)
            if (vb * PPB + q < nVB) m[u] = fmaxf(m[u], p[q].x);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + NW * u;
        if (r < Bn && s_tb[r] >= 0 && (s_tb[r] == vb || m[u] - s_lse[r] >= thr)) k = true;
      }
    }
  }
  s_k[w][lane] = k ? 1 : 0;
  __syncthreads();
  if (w == 0) {
    int any = 0;
#pragma unroll
    for (int x = 0; x < NW; ++x) any |= s_k[x][lane];
    const bool kk = any != 0 && vb < nvb_t;
    if (vb < nvb_t) {
      keep[(size_t)b * nvb_t + vb] = kk ? 1 : 0;
      // the tile's 32x32 block bits start cleared; the gradient kernel sets
      // those of the tiles it computes
      *reinterpret_cast<uint64_t*>(bmask + (size_t)b * nvg + (size_t)vb * kBlocksPerTile) = 0;
    }
    const uint64_t bal = __ballot(kk);
    if (lane == 0) atomicAdd(&hdr[kHdrTilesKept], (int)__popcll(bal));
  }
}

// ============================================================================
// Vocabulary chunks of the backward (one work-group): chunk ch covers vocab
// tiles [ch_vb[ch], ch_vb[ch + 1]).  Compact gradient storage (S > 0):
// units of `unit` vocab tiles are packed greedily, in order, into chunks of
// at most S kept tiles and span_u units (ucnt: scratch for the units' kept
// counts); dense storage (S = 0): chunks of `unit` vocab tiles.  Chunk
// numbers past the last chunk get empty ranges; ch_vb[nchunks] = nvb_t.
// ============================================================================
__global__ __launch_bounds__(1024) void chunk_plan_kernel(const uint8_t* __restrict__ keep, int nb, int nvb_t,
                                                          int unit, int S, int span_u, int nchunks,
                                                          int* __restrict__ ch_vb, int* __restrict__ ucnt) {
  const int tid = threadIdx.x;
  if (S == 0) {
    for (int c = tid; c <= nchunks; c += 1024) ch_vb[c] = min(c * unit, nvb_t);
    return;
  }
  // the units' kept counts: in LDS when they fit (the greedy pass below
  // reads them one by one), one (unit, token block) pair per thread;
  // else in the scratch, one unit per thread
  constexpr int kLdsUnits = 4096;
  __shared__ int lcnt[kLdsUnits];
  const int nunits = (nvb_t + unit - 1) / unit;
  const bool lds = nunits <= kLdsUnits;
  int* cnts = lds ? lcnt : ucnt;
  if (lds) {
    for (int u = tid; u < nunits; u += 1024) lcnt[u] = 0;
    __syncthreads();
    for (int w = tid; w < nunits * nb; w += 1024) {
      const int u = w % nunits, b = w / nunits;
      const uint8_t* kr = keep + (size_t)b * nvb_t;
      int k = 0;
      for (int v = u * unit; v < min(nvb_t, (u + 1) * unit); ++v) k += kr[v] != 0;
      if (k) atomicAdd(&lcnt[u], k);
    }
  } else {
    for (int u = tid; u < nunits; u += 1024) {
      int k = 0;
      for (int v = u * unit; v < min(nvb_t, (u + 1) * unit); ++v)
        for (int b = 0; b < nb; ++b) k += keep[(size_t)b * nvb_t + v] != 0;
      ucnt[u] = k;
    }
  }
  __syncthreads();
  if (tid == 0) {
    // each unit holds at most nb * unit <= S kept tiles: a chunk always
    // takes its first unit
    int c = 0, cnt = 0, u0 = 0;
    ch_vb[0] = 0;
    for (int u = 0; u < nunits; ++u) {
      const int k = cnts[u];
      if (u > u0 && (cnt + k > S || u + 1 - u0 > span_u) && c + 1 < nchunks) {
        ch_vb[++c] = u * unit;
        cnt = 0;
        u0 = u;
      }
      cnt += k;
    }
    for (int cc = c + 1; cc <= nchunks; ++cc) ch_vb[cc] = nvb_t;
  }
}

// ============================================================================
// Per vocabulary chunk (one work-group each): the chunk's kept gradient tiles,
// in the grouped order the gradient kernel would visit them, as a list and a
// count, and (compact storage) the slot of each kept tile: its position in
// the list.  The gradient kernel spreads the list evenly over the XCDs: with
// filtering the kept tiles gather where the frequent targets are, and a
// mapping over all tiles would hand most of them to one XCD.
// ============================================================================
__global__ __launch_bounds__(1024) void tile_list_kernel(const uint8_t* __restrict__ keep, int nvb_t, int tiles_n,
                                                         const int* __restrict__ ch_vb, int list_stride,
                                                         int* __restrict__ tlist, int* __restrict__ tcount,
                                                         int* __restrict__ slot) {
  __shared__ int scnt[1024];
  const int ch = blockIdx.x, tid = threadIdx.x;
  const int cvb0 = ch_vb[ch];
  const int cnvb = ch_vb[ch + 1] - cvb0;
  const int n = cnvb * tiles_n;
  const int run = (n + 1023) / 1024;
  const int i0 = min(n, tid * run), i1 = min(n, i0 + run);
  auto kept = [&](int idx) {
    int tvl, tn;
    grouped_tile(idx, cnvb, tiles_n, kRasterGrad, tvl, tn);
    return keep[(size_t)tn * nvb_t + cvb0 + tvl] != 0;
  };
  int cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += kept(i);
  scnt[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? scnt[tid - o] : 0;
    __syncthreads();
    scnt[tid] += v;
    __syncthreads();
  }
  int* out = tlist + (size_t)ch * list_stride;
  int pos = scnt[tid] - cnt;
  // (the plan keeps every chunk within list_stride tiles; the bound is
  // enforced here too so that no write leaves the chunk's list)
  for (int i = i0; i < i1 && pos < list_stride; ++i)
    if (kept(i)) {
      if (slot) {
        int tvl, tn;
        grouped_tile(i, cnvb, tiles_n, kRasterGrad, tvl, tn);
        slot[(size_t)tn * nvb_t + cvb0 + tvl] = pos;
      }
      out[pos++] = i;
    }
  if (tid == 1023) tcount[ch] = min(scnt[1023], list_stride);
}

// ============================================================================
// Backward: recompute kept logit tiles and write G = (p - onehot) * scale for
// one vocabulary chunk (vocab tiles [chv[0], chv[1])): bf16 (compact) one
// tile per slot, slot j = the tile's position in the chunk's list, as
// [256 tokens][256 vocab]; fp32 in place into G [Npad][Vc] (token-major) and
// G^T [Vc][gt_ld].
// ============================================================================
template <class C>
__global__ __launch_bounds__(C::NT, 1) void grad_tile_kernel(
    const typename C::T* __restrict__ c, const typename C::T* __restrict__ e, const typename C::T* __restrict__ bias,
    const int* __restrict__ rowmap, const int* __restrict__ tgt_c, const float* __restrict__ lse_c,
    const float* __restrict__ scale_c, float eps, float lam, float softcap, const int* __restrict__ tlist,
    const int* __restrict__ tcount, int N, int D, int V, const int* __restrict__ chv, int tiles_n, int Vc, int gt_ld,
    typename C::T* __restrict__ G, typename C::T* __restrict__ Gt, size_t g_bytes, size_t gt_bytes,
    float* __restrict__ db_part, uint8_t* __restrict__ bmask, int nvg, int32_t* __restrict__ hdr, int filter) {
  using T = typename C::T;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_DMA_BYTES];
  __shared__ __attribute__((aligned(16))) float sbias[C::BM];
  __shared__ uint32_t sbm[kBlocksPerTile];  // kept 32x32 blocks: per vocab group, one bit per row group
  __shared__ f32x4 scol[C::BN];             // per token column: lse, the coefficients, the target row
  // the chunk's kept tiles (listed in grouped order), XCD-contiguous runs of
  // the list: the same share of kept tiles on every XCD
  const int cnt = *tcount;
  if ((int)blockIdx.x >= cnt) return;
  if ((int)threadIdx.x < kBlocksPerTile) sbm[threadIdx.x] = 0;  // visible after the main loop's barriers
  const int cvb0 = chv[0], tiles_v = chv[1] - cvb0;
  const int li = xcd_remap(blockIdx.x, cnt);  // list position: the slot of the tile's G (bf16)
  int tvl, tn;
  grouped_tile(tlist[li], tiles_v, tiles_n, kRasterGrad, tvl, tn);
  const int tv = cvb0 + tvl;
  const int v0 = tv * C::BM, n0 = tn * C::BN;
  if (bias || softcap > 0.f) stage_bias<T, C::BM>(sbias, bias, v0, V);

  Operand A = make_operand(c + (size_t)v0 * D, (uint64_t)(V - v0) * D * sizeof(T), (uint32_t)D,
               min(C::BM, V - v0), D);
  // token rows of the tile's compacted slots n0.. through rowmap
  Operand B = make_operand(e, (uint64_t)N * D * sizeof(T), (uint32_t)D, C::BN, D);
  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};
  // per-column (slot) constants, staged in LDS before the main loop (one
  // column per thread, their latency hidden behind the loop; held in
  // registers across it they would be spilled): lse in log2 units, the
  // coefficients of p (scale times 1 + 2 lam LSE, the z-loss share) and of
  // the one-hot target (scale times 1 - eps), and the target's row in the
  // tile (outside the tile: -1024, below any lane's row offset).  Ignored
  // and padding slots have LSE +inf (p = 0) and scale 0: their G is exactly 0.
  for (int j = threadIdx.x; j < C::BN; j += C::NT) {
    const int n = n0 + j;  // < Npad: the grid covers the padded slots exactly
    const float l = lse_c[n];
    const float s = scale_c[n];
    const int tg = tgt_c[n];
    scol[j] = f32x4{l * kLog2e, s != 0.f ? s * (1.f + 2.f * lam * l) : 0.f, s * (1.f - eps),
                    __builtin_bit_cast(float, (tg >= v0 && tg < v0 + C::BM) ? tg - v0 : -1024)};
  }
  mainloop_dma<C, 1>(acc, A, B, (D + C::BK - 1) / C::BK, nullptr, smem, rowmap + n0);

  // this lane's columns' constants (the main loop's barriers order the
  // staging before these reads); trow: the target's row relative to the
  // lane's first accumulator row (outside [0, WM) when the target is not in
  // the wave's rows)
  AccMap<C> am;
  float lsel[C::FN], sc[C::FN], st[C::FN];
  int trow[C::FN];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    const f32x4 k = scol[am.colj(fn)];
    lsel[fn] = k[0];
    sc[fn] = k[1];
    st[fn] = k[2];
    // (the element is copied out first: a bit cast of a vector element
    // lvalue read element 0 in this compiler)
    const float k3 = k[3];
    trow[fn] = __builtin_bit_cast(int, k3) - am.row0;
  }
  rsrc_t rg = make_rsrc(G, g_bytes);
  rsrc_t rgt = make_rsrc(Gt, gt_bytes);
  const int vl0 = tvl * C::BM;  // chunk-local column of the tile
  // G = (softmax - onehot) * scale, rounded once to the operand type, handed
  // to `sink(fn, fm, q, rl, g)` four consecutive vocab rows (rl..rl+3,
  // tile-local) of one token column at a time.  Rows of the last tile past V
  // are zeroed (their logits read zero rows of c); all other tiles take the
  // branch-free path.
  // A column's target row lies in this wave's 128 rows for few tiles (about
  // 128 / V of them per column): a wave-uniform test skips the one-hot compare
  // everywhere else.
  // mode 0: plain logits; 1: plus the bias; 2: bias (zero without one), then
  // soft-capped, G scaled by the cap's derivative 1 - (z'/s)^2
  const float kcap = softcap > 0.f ? 2.f * kLog2e / softcap : 0.f;
  const float rcap = softcap > 0.f ? 1.f / softcap : 0.f;
  // The finer filter level (with filtering on): each 32x32 MFMA block (fm,
  // fn) of the tile (32 vocab rows x 32 token slots) is kept iff one of its
  // softmax values reaches 2^-12 (log2 argument >= -12) or it holds a target;
  // a dropped block's G is exactly 0: the bf16 contractions skip its MFMAs
  // and it is not written at all, the fp32 ones (dense) read stored zeros.
  // kbits bit fn * FM + fm records the wave's kept blocks.
  uint32_t kbits = 0;
  constexpr bool kSkipDropped = sizeof(T) == 2;
  auto compute = [&](auto ragged, auto mode, auto&& sink) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode)::value;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      auto body = [&](auto with_target) __attribute__((always_inline)) {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
          // The block's 16 (biased, capped) logits of this lane, kept in
          // registers until the block's keep decision: the largest log2
          // softmax value x = z log2(e) - LSE log2(e) over the block's 32 x 32
          // entries against -12, or a target in the block.  The lane's 16
          // values share one token column (one LSE), and rounding is
          // monotone, so the lane's largest x is that of its largest z.
          float zq[4][4];
          float zm = -INFINITY;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int rl = am.row(fm, 4 * q);
            const f32x4 bz = MODE ? bias4(sbias, rl) : f32x4{};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              float z = MODE ? acc[fm][fn][4 * q + u] + bz[u] : acc[fm][fn][4 * q + u];
              if constexpr (MODE == 2) z = softcap_f(z, softcap, kcap);
              if constexpr (decltype(ragged)::value) {
                if (v0 + rl + u < V) zm = fmaxf(zm, z);
              } else {
                zm = fmaxf(zm, z);
              }
              zq[q][u] = z;
            }
          }
          const float xm = __builtin_fmaf(zm, kLog2e, -lsel[fn]);
          // a target in the block's rows (the lower half-wave's row offset is 0)
          const bool tgt = decltype(with_target)::value && (threadIdx.x & 32) == 0 && trow[fn] >= 0 &&
                           (trow[fn] >> 5) == fm;
          // (filtering off: every block inside the problem is kept)
          const int wave = (int)(threadIdx.x >> 6);
          const bool kept = filter ? __builtin_amdgcn_ballot_w64(xm >= -12.f || tgt) != 0
                                   : v0 + wave / C::WAVES_N * C::WM + fm * 32 < V &&
                                         n0 + wave % C::WAVES_N * C::WN + fn * 32 < N;
          kbits |= (kept ? 1u : 0u) << (fn * C::FM + fm);
          // With filtering, bf16 operands: the contractions skip the MFMAs
          // of a dropped block and never read its G, which is then neither
          // formed nor stored.  Otherwise (fp32 operands, whose contractions
          // are dense, or filtering off) a block outside the kept set is
          // stored as zeros.
          if (kSkipDropped && filter && !kept) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int rl = am.row(fm, 4 * q);
            float g[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float z = zq[q][u];
              const float p = fast_exp2(__builtin_fmaf(z, kLog2e, -lsel[fn]));
              float gv;
              if constexpr (decltype(with_target)::value) {
                const float tsc = trow[fn] == fm * 32 + 8 * q + u ? st[fn] : 0.f;
                gv = __builtin_fmaf(p, sc[fn], -tsc);
              } else {
                gv = p * sc[fn];
              }
              if constexpr (MODE == 2) {
                const float y = z * rcap;
                gv *= __builtin_fmaf(-y, y, 1.f);
              }
              if constexpr (decltype(ragged)::value) gv = v0 + rl + u < V ? gv : 0.f;
              g[u] = kept ? gv : 0.f;
            }
            sink(fn, fm, q, rl, g);
          }
        }
      };
      if (__builtin_amdgcn_ballot_w64(trow[fn] >= 0 && trow[fn] < C::WM) != 0) body(std::true_type{});
      else body(std::false_type{});
    }
  };
  // The wave's kept-block bits into the block mask: byte (token block tn,
  // vocab group) holds one bit per 32-row group of the token block.  Waves
  // that share vocab rows combine through LDS (sbm, zeroed before the main
  // loop); one store per vocab group after `barrier`.
  auto publish_blocks = [&]() __attribute__((always_inline)) {
    const int wave = (int)(threadIdx.x >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        uint32_t bits = 0;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) bits |= ((kbits >> (fn * C::FM + fm)) & 1u) << (wn * C::FN + fn);
        if (bits) atomicOr(&sbm[wm * C::FM + fm], bits);
      }
      const int cnt = __builtin_popcount(kbits);
      if (cnt) atomicAdd(&hdr[kHdrBlocksKept], cnt);
    }
  };
  auto store_blocks = [&]() __attribute__((always_inline)) {
    // after a barrier that follows publish_blocks
    if ((int)threadIdx.x < kBlocksPerTile)
      bmask[(size_t)tn * nvg + (size_t)tv * kBlocksPerTile + threadIdx.x] = (uint8_t)sbm[threadIdx.x];
  };
  auto run = [&](auto&& sink) __attribute__((always_inline)) {
    auto rag = [&](auto mode) __attribute__((always_inline)) {
      if (v0 + C::BM <= V) compute(std::false_type{}, mode, sink);
      else compute(std::true_type{}, mode, sink);
    };
    // soft-capping exists for bf16 operands only (the host rejects fp32)
    if constexpr (sizeof(T) == 2) {
      if (softcap > 0.f) {
        rag(std::integral_constant<int, 2>{});
        return;
      }
    }
    if (bias) rag(std::integral_constant<int, 1>{});
    else rag(std::integral_constant<int, 0>{});
  };

  // token sums per vocabulary row (db), from this lane's share rs: across the
  // 32 lanes of a half-wave, then the waves that share the rows, through
  // LDS, in a fixed order.  Called with the LDS free.
  auto db_sums = [&](const float (&rs)[C::FM][4][4]) __attribute__((always_inline)) {
    float* red = (float*)smem;  // [WAVES_N][BM]
    const int wn = (threadIdx.x >> 6) % C::WAVES_N;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float x = rs[fm][q][u];
#pragma unroll
          for (int m = 16; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
          if ((lane & 31) == 0) red[wn * C::BM + am.row(fm, 4 * q) + u] = x;
        }
    __syncthreads();
    for (int r = threadIdx.x; r < C::BM; r += C::NT) {
      float x = 0.f;
      for (int w = 0; w < C::WAVES_N; ++w) x += red[w * C::BM + r];
      if (v0 + r < V) db_part[(size_t)tn * V + v0 + r] = x;
    }
  };
  if constexpr (sizeof(T) == 2) {
    // bf16: G only (dC reads it with transposing LDS reads; G^T is not
    // formed), staged through LDS (free after the main loop) so that it
    // leaves as rows of 16-byte stores from consecutive lanes (stored straight
    // from the accumulators, one instruction would scatter 8-byte pieces over
    // 64 rows).  A staging tile holds 256 token rows of 512 bytes; 16-byte
    // chunk j of row r sits in slot j ^ (r % 32).  A lane holds four vocab
    // rows of its token per accumulator group and the lane 32 apart the next
    // four: one v_permlane32_swap per word pairs them, so that each lane
    // writes a whole chunk (eight vocab rows; the lower half-wave for group
    // q, the upper for q + 1).  Sixteen lanes of a ds_write_b128 cycle then
    // write one chunk of 16 consecutive rows, sixteen distinct slots (the
    // 8-byte writes of half chunks had two-way conflicts on the 64-bank LDS),
    // and the row drains are conflict free.
    static_assert(C::BM == 256 && C::BN == 256 && C::LDS_DMA_BYTES >= 256 * 512, "tile staging");
    lds_u8* tile = (lds_u8*)smem;
    auto slot = [](int r, int col) -> uint32_t {
      return (uint32_t)(r * 512 + (((col >> 3) ^ (r & 31)) << 4) + ((col & 7) << 1));
    };
    const bool sums = db_part != nullptr;
    const int wrow = ((int)(threadIdx.x >> 6) / C::WAVES_N) * C::WM;  // the wave's first vocab row
    const int upper = (int)(threadIdx.x >> 5) & 1;                     // lanes 32-63
    uint32_t plo = 0, phi = 0;  // group q - 1's words, for odd q
    run([&](int fn, int fm, int q, int, const float (&g)[4]) __attribute__((always_inline)) {
      const uint32_t lo = pack_bf16(g[0], g[1]), hi = pack_bf16(g[2], g[3]);
      if ((q & 1) == 0) {
        plo = lo;
        phi = hi;
      } else {
        // lower lanes: group q - 1 whole (own rows, then the upper lane's);
        // upper lanes: group q whole (the lower lane's rows, then own)
        const auto sl = __builtin_amdgcn_permlane32_swap(plo, lo, false, false);
        const auto sh = __builtin_amdgcn_permlane32_swap(phi, hi, false, false);
        const int col = wrow + fm * 32 + 8 * (q - 1 + upper);
        *(__attribute__((address_space(3))) u32x4*)(tile + slot(am.colj(fn), col)) = u32x4{sl[0], sh[0], sl[1], sh[1]};
      }
    });
    publish_blocks();
    __syncthreads();
    store_blocks();
    // The tile leaves by 32x32 blocks (the slot's block layout: block (t, v)
    // at element (8 t + v) * 1024, [32 tokens][32 vocab]), half a block (16
    // rows of 64 bytes) per instruction: wave w drains half blocks
    // [w HPW, (w + 1) HPW); lane l takes row l / 4, chunk l % 4 of its half
    // block.  With filtering a dropped block (not staged) is not stored.
    constexpr int HPW = 128 / (C::NT / 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll 4
    for (int it = 0; it < HPW; ++it) {
      const int hb = wave * HPW + it, k = hb >> 1;  // k = 8 t + v
      const int t = k >> 3, v = k & 7;
      if (filter && !((sbm[v] >> t) & 1u)) continue;
      const int r = 16 * (hb & 1) + (lane >> 2), c = lane & 3;
      const u32x4 val =
          *(const __attribute__((address_space(3))) u32x4*)(tile + slot(32 * t + r, 32 * v + 8 * c));
      __builtin_amdgcn_raw_buffer_store_b128(
          val, rg, ((uint32_t)li * (uint32_t)(kSlotRows * kTileV) + (uint32_t)k * 1024u + (uint32_t)r * 32u +
                    (uint32_t)c * 8u) * 2u,
          0, kStoreNT);
    }
    if (sums) {
      // db: each vocab row's sum over the tile's tokens of the staged
      // (rounded) values, as the contractions see them.  Thread (chunk ch,
      // token block t) sums eight vocab rows over 32 token rows (a dropped
      // block is not staged and adds nothing), then the eight token blocks'
      // sums are added through LDS in a fixed order.
      static_assert(C::NT == 256, "db sums: one thread per (8-row chunk, token block)");
      const int ch = threadIdx.x & 31, t = threadIdx.x >> 5;
      float ps[8] = {};
      if (!filter || ((sbm[ch >> 2] >> t) & 1u)) {
#pragma unroll 4
        for (int r = 32 * t; r < 32 * t + 32; ++r) {
          const u32x4 w = *(const __attribute__((address_space(3))) u32x4*)(tile + slot(r, 8 * ch));
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            ps[2 * k] += __builtin_bit_cast(float, w[k] << 16);
            ps[2 * k + 1] += __builtin_bit_cast(float, w[k] & 0xffff0000u);
          }
        }
      }
      __syncthreads();  // the drain's LDS reads are done
      float* red = (float*)smem;  // [8 token blocks][BM]
#pragma unroll
      for (int k = 0; k < 8; ++k) red[t * C::BM + 8 * ch + k] = ps[k];
      __syncthreads();
      for (int r = threadIdx.x; r < C::BM; r += C::NT) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) x += red[w * C::BM + r];
        if (v0 + r < V) db_part[(size_t)tn * V + v0 + r] = x;
      }
    }
  } else {
    float rs[C::FM][4][4] = {};  // this lane's share of each vocab row's token sum (for db)
    run([&](int fn, int fm, int q, int rl, const float (&g)[4]) __attribute__((always_inline)) {
      const int n = n0 + am.colj(fn);
      store4(rg, ((uint32_t)n * (uint32_t)Vc + (uint32_t)(vl0 + rl)) * (uint32_t)sizeof(T), g[0], g[1], g[2], g[3],
             (const T*)nullptr);
      // G^T[v][n]: the quad's four tokens of vocab rows rl..rl+3
      store_quad_t(rgt, ((uint32_t)(vl0 + rl) * (uint32_t)gt_ld + (uint32_t)(n & ~3)) * (uint32_t)sizeof(T),
                   (uint32_t)gt_ld * (uint32_t)sizeof(T), g, (const T*)nullptr);
#pragma unroll
      for (int u = 0; u < 4; ++u) rs[fm][q][u] += g[u];
    });
    publish_blocks();
    __syncthreads();
    store_blocks();
    if (db_part) db_sums(rs);
  }
}

// Token blocks that hold valid rows (compacted slots: they come first).
__device__ __forceinline__ int valid_blocks(const int32_t* __restrict__ hdr) {
  return (hdr[kHdrNValidBwd] + kTileN - 1) / kTileN;
}

// The steps (of SPB = 4 per K block) that hold a nonzero block of the A
// tile, by their index in the full step sequence, into LDS; returns their
// count.  `nz(c)` tells whether step c of the full sequence does.
template <class F>
__device__ __forceinline__ int collect_steps(int nfull, const F& nz, uint16_t* list) {
  __shared__ int s_ns;
  if (threadIdx.x < 64) {
    int total = 0;
    for (int c0 = 0; c0 < nfull; c0 += 64) {
      const int c = c0 + (int)threadIdx.x;
      const bool k = c < nfull && nz(c);
      const uint64_t bal = __ballot(k);
      const int pre = __popcll(bal & ((1ull << threadIdx.x) - 1ull));
      if (k) list[total + pre] = (uint16_t)c;
      total += __popcll(bal);
    }
    if (threadIdx.x == 0) s_ns = total;
  }
  __syncthreads();
  return s_ns;
}

// The kept K blocks of one contraction tile, in ascending order, into LDS
// (list), with each listed block's G slot (SLOT: slots, compact storage) and
// its block-mask word (WORDS: words, filtering); returns the count.
// Candidate i is keep[kbase + i kstride] (its slot at the same index of the
// [nb][nvb_t] slot map) with mask word at bmask + mbase + i mstride.  Every
// thread loads its candidates' flag, slot and word at once, so the three
// come in one memory round trip.  count <= kMaxBlocks.
struct NoPerm {
  __device__ __forceinline__ static uint64_t apply(uint64_t w) { return w; }
};
template <int NT, bool SLOT, bool WORDS, class Perm = NoPerm>
__device__ __forceinline__ int collect_kept(const uint8_t* __restrict__ keep, size_t kbase, int kstride, int count,
                                            const int* __restrict__ slot, const uint8_t* __restrict__ bmask,
                                            size_t mbase, int mstride, uint16_t* list, uint16_t* slots,
                                            uint64_t* words) {
  constexpr int R = kMaxBlocks / NT, NW = NT / 64;
  static_assert(kMaxBlocks % NT == 0, "candidates per thread");
  __shared__ int wcnt[NW];
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bool kp[R];
  int sl[R];
  uint64_t mw[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = r * NT + tid;
    const bool in = i < count;
    kp[r] = in && keep[kbase + (size_t)i * kstride] != 0;
    if constexpr (SLOT) sl[r] = in ? slot[kbase + (size_t)i * kstride] : 0;
    if constexpr (WORDS) mw[r] = in ? *reinterpret_cast<const uint64_t*>(bmask + mbase + (size_t)i * mstride) : 0;
  }
  // (every pass ends on a barrier, and there is at least one: the caller
  // relies on one after the call)
  int base = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r > 0 && r * NT >= count) break;  // uniform
    const uint64_t bal = __ballot(kp[r]);
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    int off = base, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) off += wcnt[w];
      tot += wcnt[w];
    }
    if (kp[r]) {
      const int pos = off + __popcll(bal & ((1ull << lane) - 1ull));
      list[pos] = (uint16_t)(r * NT + tid);
      if constexpr (SLOT) slots[pos] = (uint16_t)sl[r];
      if constexpr (WORDS) words[pos] = Perm::apply(mw[r]);
    }
    __syncthreads();  // wcnt is rewritten next pass; the lists are published
    base += tot;
  }
  return __builtin_amdgcn_readfirstlane(base);  // the same in every lane
}


// ============================================================================
// 32x32 block masks of the gradient contractions (mainloop_dma MaskT).  The
// work-group stages, per entry j of its K-block list, the eight block-mask
// bytes of that K block in LDS (sm[j]); a K step is a quarter of a K block.
// ============================================================================
typedef __attribute__((address_space(3))) uint64_t lds_u64;

// Staged mask words are permuted (Perm::apply, when collect_kept stages
// them) so that bit 32 wm + 8 sub + 4 h + fm is the block of the wave's
// 32-row group fm (waves with row half wm) in K half h of step sub of the K
// block: a step's eight bits for a wave are one byte, and a step holds a
// kept block iff (w >> 8 sub) & 0x000000ff000000ff is nonzero.
constexpr uint64_t kStepBits = 0x000000ff000000ffull;

// The A-stage blocks of step f (for mainloop_dma's kSkipA) from the staged
// word's halves: stage block k = 8 h + 4 wm + fm (K half h, wave row half
// wm, group fm: the order of the block-layout DMA tiles) is bit 8 sub + 4 h +
// fm of half wm, sub = f % 4.
__device__ __forceinline__ uint32_t stage_block_bits(uint32_t lo, uint32_t hi, int f) {
  const int sh = 8 * (f & 3);
  const uint32_t a = (lo >> sh) & 0xffu, b = (hi >> sh) & 0xffu;
  return (a & 0xfu) | ((b & 0xfu) << 4) | ((a >> 4) << 8) | ((b >> 4) << 12);
}

// dE: A rows are tokens (wave rows: 32-row groups 4 wm .. 4 wm + 3 of the
// token block), K is vocabulary; the block-mask word of a K block has byte v
// for vocab group v, bit t for token group t: group fm of wave row half wm
// in K half h of step sub is bit 4 wm + fm of byte 2 sub + h.
struct DEMask {
  static constexpr bool kActive = true;
  static constexpr bool kSkipA = true;
  const lds_u64* sm;
  int shift;  // 32 wm
  __device__ __forceinline__ uint64_t raw(int f) const { return sm[f >> 2]; }
  __device__ __forceinline__ static uint32_t dma_bits(uint32_t lo, uint32_t hi, int f) {
    return stage_block_bits(lo, hi, f);
  }
  __device__ __forceinline__ static uint64_t apply(uint64_t w) {
    uint64_t o = 0;
#pragma unroll
    for (int b = 0; b < 64; ++b) {
      const int wm = b >> 5, sub = (b >> 3) & 3, h = (b >> 2) & 1, fm = b & 3;
      o |= ((w >> (8 * (2 * sub + h) + 4 * wm + fm)) & 1ull) << b;
    }
    return o;
  }
  __device__ __forceinline__ uint32_t operator()(int s) const {
    const uint32_t w = ((const __attribute__((address_space(3))) uint32_t*)sm)[2 * (s >> 2) + (shift >> 5)];
    return (w >> (8 * (s & 3))) & 0xffu;
  }
};

// dC: A rows are vocabulary (wave rows: vocab groups 4 wm .. 4 wm + 3 of the
// tile), K is tokens; the block-mask word of a token block has byte v for
// the tile's vocab group v, bit t for token group t: group fm of wave row
// half wm in K half h of step sub is bit 2 sub + h of byte 4 wm + fm.
struct DCMask {
  static constexpr bool kActive = true;
  static constexpr bool kSkipA = true;
  const lds_u64* sm;
  int shift;  // 32 wm
  __device__ __forceinline__ uint64_t raw(int f) const { return sm[f >> 2]; }
  __device__ __forceinline__ static uint32_t dma_bits(uint32_t lo, uint32_t hi, int f) {
    return stage_block_bits(lo, hi, f);
  }
  __device__ __forceinline__ static uint64_t apply(uint64_t w) {
    uint64_t o = 0;
#pragma unroll
    for (int b = 0; b < 64; ++b) {
      const int wm = b >> 5, sub = (b >> 3) & 3, h = (b >> 2) & 1, fm = b & 3;
      o |= ((w >> (8 * (4 * wm + fm) + 2 * sub + h)) & 1ull) << b;
    }
    return o;
  }
  __device__ __forceinline__ uint32_t operator()(int s) const {
    const uint32_t w = ((const __attribute__((address_space(3))) uint32_t*)sm)[2 * (s >> 2) + (shift >> 5)];
    return (w >> (8 * (s & 3))) & 0xffu;
  }
};

// ============================================================================
// db[v] = sum over token blocks (in order) of the kept tiles' column sums.
// ============================================================================
// With label smoothing, plus r1 * ssum[0] = -eps/V * sum_i scale_i.
__global__ __launch_bounds__(256) void db_reduce_kernel(const float* __restrict__ db_part,
                                                        const uint8_t* __restrict__ keep, int nb, int nvb_t, int V,
                                                        const float* __restrict__ ssum, float r1,
                                                        float* __restrict__ db) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  float s = 0.f;
  for (int b = 0; b < nb; ++b)
    if (keep[(size_t)b * nvb_t + v / kTileV]) s += db_part[(size_t)b * V + v];
  db[v] = ssum ? s + r1 * ssum[0] : s;
}

// ============================================================================
// dC rows of one vocabulary chunk (vocab tiles [chv[0], chv[1])): dC[v][d] =
// sum_n G^T[v][n] E^T[d][n] over the kept token blocks of the tile's vocab
// block.  B = E^T (K-major); A = G^T: bf16 reads the compact G (each kept
// tile in its slot, [256 tokens][256 vocab], MN-major) through transposing
// LDS reads, fp32 the K-major G^T [Vc][gt_ld].
// ============================================================================
template <class C, bool MASK>
__global__ __launch_bounds__(C::NT, 1) void dC_gemm_kernel(
    const typename C::T* __restrict__ G, const typename C::T* __restrict__ Gt, const typename C::T* __restrict__ Et,
    const uint8_t* __restrict__ keep, const int* __restrict__ slot, int cap, int Npad, int gt_ld, int D, int V,
    int nvb_t, const int* __restrict__ chv, int tiles_d, size_t g_bytes, size_t gt_bytes,
    const float* __restrict__ r1c, void* __restrict__ dC, int out_bf16, const uint8_t* __restrict__ bmask,
    int nvg) {
  using T = typename C::T;
  constexpr bool kMN = sizeof(T) == 2;
  static_assert(!MASK || (kMN && C::FM == 4), "block masks: bf16, four 32-row fragments per wave");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_DMA_BYTES];
  __shared__ uint16_t blocks[kMaxBlocks];
  __shared__ uint16_t ablk[kMN ? kMaxBlocks : 1];  // bf16: the G slot of each listed token block
  __shared__ uint64_t smask[MASK ? kMaxBlocks : 1];
  __shared__ uint16_t steps[MASK ? 4 * kMaxBlocks : 1];  // the steps with a nonzero block (masked)
  const int cvb0 = chv[0], tiles_v = chv[1] - cvb0;
  const int cv0 = cvb0 * kTileV, clen = min(tiles_v * kTileV, V - cv0);
  // Groups of GR vocab tiles (each with all its d tiles) are dealt to the
  // XCDs in turn, group g to XCD g % 8 (work-group i runs on XCD i % 8): the
  // vocab tiles with many kept token blocks (frequent targets) sit next to
  // each other, and this spreads them over the XCDs.  Inside a group the
  // order is the grouped raster (L2 reuse).  GR is the widest group (at
  // most kRasterDC) whose busiest XCD gets at most 1/32 more vocab tiles
  // than with the most even split (chunks are whole units of 8 vocab tiles
  // but the last, so that is usually GR = kRasterDC).  The chunk's width is
  // known on the device only: the grid covers 8 x GR x tiles_d x
  // ceil(groups / 8) work-groups for the widest chunk possible, and the
  // spare exit.
  auto busiest = [&](int gr) {
    // vocab tiles of XCD 0 (the busiest): groups 0, 8, 16, ..., of which
    // only the last can be partial
    const int g0 = ((tiles_v + gr - 1) / gr + 7) / 8;
    return (g0 - 1) * gr + min(gr, tiles_v - (g0 - 1) * 8 * gr);
  };
  int lmin = tiles_v;
  for (int gr = 1; gr <= kRasterDC; ++gr) lmin = min(lmin, busiest(gr));
  int GR = 1;
  for (int gr = kRasterDC; gr > 1; --gr)
    if (busiest(gr) <= lmin + lmin / 32) {
      GR = gr;
      break;
    }
  const int per = GR * tiles_d;
  const int x = (int)blockIdx.x & 7, j = (int)blockIdx.x >> 3;
  const int g = x + 8 * (j / per), r = j % per;
  const int gm = min(GR, tiles_v - g * GR);  // vocab tiles in group g
  if (gm <= 0 || r >= gm * tiles_d) return;
  const int tvl = g * GR + r % gm, td = r / gm;
  {
    const int vl0 = tvl * C::BM, d0 = td * C::BN;
    const int nb = Npad / kTileN;
    // the kept token blocks of the vocab tile with, for bf16, their G slots
    // (A's K blocks: K rows slot * 256 .., G seen as cap * 256 token rows of
    // the 256 vocab columns) and, with block masks, the tile's block-mask
    // bytes of each (byte v: vocab group v, bit t: token group t)
    const int nk = collect_kept<C::NT, kMN, MASK, DCMask>(keep, (size_t)(cvb0 + tvl), nvb_t, nb, slot, bmask,
                                                  (size_t)(cvb0 + tvl) * kBlocksPerTile, nvg, blocks, ablk,
                                                  (uint64_t*)smask);
    const Operand A =
        kMN ? make_operand(G, g_bytes, (uint32_t)kTileV, min(C::BM, clen - vl0), cap * kSlotRows)
            : make_operand(Gt + (size_t)vl0 * gt_ld, gt_bytes - (size_t)vl0 * gt_ld * sizeof(T), (uint32_t)gt_ld,
                           min(C::BM, clen - vl0), Npad);
    Operand B = make_operand(Et + (size_t)d0 * Npad, (uint64_t)(D - d0) * Npad * sizeof(T), (uint32_t)Npad,
                 min(C::BN, D - d0), Npad);
    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};
    constexpr int SPB = kTileN / C::BK;
    if constexpr (MASK) {
      // the steps (64 tokens of a token block each) with a nonzero block:
      // bits 8 v + 2 (c % 4) + h of the step's mask word
      const int ns = collect_steps(
          nk * SPB, [&](int c) { return ((smask[c >> 2] >> (8 * (c & 3))) & kStepBits) != 0; }, steps);
      const int wm = (int)(threadIdx.x >> 6) / C::WAVES_N;
      const DCMask mk{(const lds_u64*)smask, 32 * wm};
      const uint16_t* bl = nk > 0 && blocks[nk - 1] == nk - 1 ? nullptr : blocks;
      // the step list costs about 5% of the loop: taken when it leaves out
      // at least an eighth of the steps.  The step's DMA in two parts
      // (after the barrier and in the first K group): with the loads of
      // all-zero G blocks skipped, measured 1-4% faster than three.
      if (8 * ns <= 7 * nk * SPB)
        mainloop_dma<C, SPB, false, kMN, 2, DCMask, true, DmaBlockMN<C>, true, true>(acc, A, B, ns, bl, smem,
                                                                                    nullptr, mk, ablk, kSlotRows,
                                                                                    steps);
      else
        mainloop_dma<C, SPB, false, kMN, 2, DCMask, true, DmaBlockMN<C>, false, true>(acc, A, B, nk * SPB, bl, smem,
                                                                                     nullptr, mk, ablk, kSlotRows);
    } else {
      // the kept token blocks are the first nk (no filtering effect on this
      // tile; compacted slots put the blocks of ignored rows last): contiguous
      // K for B
      const uint16_t* bl = nk > 0 && blocks[nk - 1] == nk - 1 ? nullptr : blocks;
      if constexpr (kMN)
        mainloop_dma<C, SPB, false, kMN, 3, NoMask, true, DmaBlockMN<C>, false, true>(acc, A, B, nk * SPB, bl, smem,
                                                                                     nullptr, NoMask{}, ablk,
                                                                                     kSlotRows);
      else
        mainloop_dma<C, SPB, false, kMN>(acc, A, B, nk * SPB, bl, smem);
    }

    AccMap<C> am;
    const int vg0 = cv0 + vl0;
    // dC rows of the tile, float or bf16 (out_bf16)
    const size_t es = out_bf16 ? 2 : 4;
    rsrc_t ro = make_rsrc((char*)dC + (size_t)vg0 * D * es, (uint64_t)(V - vg0) * D * es);
    // the smoothing term, the same for every vocabulary row (r1c: null without)
    float add[C::FN];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int d = d0 + am.colj(fn);
      add[fn] = (r1c && d < D) ? r1c[d] : 0.f;
    }
    // Each lane quad transposes its 4x4 blocks (four rows of four columns),
    // so a lane writes four consecutive columns of one row: one 16-byte (fp32)
    // or 8-byte (bf16) store instead of four.  D is a multiple of 4: a quad's
    // columns are all inside or all outside.
    const int k = (int)threadIdx.x & 3;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int dq = d0 + (am.colj(fn) & ~3);  // the quad's first column
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t x[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) x[u] = __builtin_bit_cast(uint32_t, acc[fm][fn][4 * q + u] + add[fn]);
          quad_transpose(x);
          const int vr = am.row(fm, 4 * q) + k;
          const bool ok = dq < D && vl0 + vr < clen;
          const uint32_t e = (uint32_t)vr * (uint32_t)D + (uint32_t)dq;
          if (out_bf16) {
            const u32x2 b = {pack_bf16(__builtin_bit_cast(float, x[0]), __builtin_bit_cast(float, x[1])),
                             pack_bf16(__builtin_bit_cast(float, x[2]), __builtin_bit_cast(float, x[3]))};
            __builtin_amdgcn_raw_buffer_store_b64(b, ro, ok ? e * 2u : kOOB, 0, kStoreNT);
          } else {
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{x[0], x[1], x[2], x[3]}, ro, ok ? e * 4u : kOOB, 0,
                                                   kStoreNT);
          }
        }
      }
  }
}

// ============================================================================
// dE for one vocabulary chunk (vocab tiles [chv[0], chv[1])): dE[n][d] (+)=
// sum_v G[n][v] C[v][d] over the kept vocab blocks of the tile's token block
// in split `s` of the chunk.  A = G (K-major: bf16 the compact tiles, K block
// j in slot j's 65536 elements; fp32 [Npad][Vc]), B = C (MN-major).
// ============================================================================
template <class C, bool MASK>
__global__ __launch_bounds__(C::NT, 1) void dE_gemm_kernel(
    const typename C::T* __restrict__ G, const typename C::T* __restrict__ c,
    const uint8_t* __restrict__ keep, const int* __restrict__ slot, int cap, int N, int D, int V, int nvb_t,
    const int* __restrict__ chv, int tiles_n, int tiles_d, int splits, const int32_t* __restrict__ hdr, int Vc,
    size_t g_bytes,
    void* __restrict__ dE_out, int out_bf16,
    float* __restrict__ dE_part, int accumulate, int atomic, const int* __restrict__ rowmap,
    const float* __restrict__ scale_c, const float* __restrict__ csum, float r1, const uint8_t* __restrict__ bmask,
    int nvg) {
  using T = typename C::T;
  // bf16: LDS-DMA main loop (C fragments through transposing reads); fp32:
  // register-staged main loop (no 32-bit transposing read exists)
  constexpr bool kDma = sizeof(T) == 2;
  static_assert(!MASK || (kDma && C::FM == 4), "block masks: bf16, four 32-row fragments per wave");
  __shared__ uint64_t smask[MASK ? kMaxBlocks : 1];
  // dE as float, or (out_bf16: one pass writes it, no split or chunk adds to
  // it) as bf16
  float* dE = out_bf16 ? nullptr : (float*)dE_out;
  uint16_t* dEb = out_bf16 ? (uint16_t*)dE_out : nullptr;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDma ? C::LDS_DMA_BYTES : C::LDS_BYTES];
  __shared__ uint16_t blocks[kMaxBlocks];
  __shared__ uint16_t ablk[kDma ? kMaxBlocks : 1];  // bf16: the G slot of each listed vocab block
  __shared__ uint16_t steps[MASK ? 4 * kMaxBlocks : 1];  // the steps with a nonzero block (masked)
  const int cvb0 = chv[0], cnvb = chv[1] - cvb0;
  const int cv0 = cvb0 * kTileV, clen = min(cnvb * kTileV, V - cv0);
  // The grid holds tiles_n x tiles_d x splits work-groups.  The first
  // nbv x tiles_d x splits work on the token blocks that hold valid rows
  // (tile order remapped over exactly these, so they spread over all XCDs);
  // the next (tiles_n - nbv) x tiles_d cover the blocks of padding rows,
  // which only need zeros; the rest exit.
  const int nbv = valid_blocks(hdr);
  const int work = nbv * tiles_d * splits;
  int s, tn, td;
  if ((int)blockIdx.x < work) {
    const int tile = xcd_remap(blockIdx.x, work);
    s = tile / (nbv * tiles_d);
    grouped_tile(tile % (nbv * tiles_d), nbv, tiles_d, kRasterDE, tn, td);
  } else {
    const int p = (int)blockIdx.x - work;
    if (p >= (tiles_n - nbv) * tiles_d) return;
    // a block of padding rows: zeros into dE and every partial in use, once
    if (accumulate || atomic) return;
    tn = nbv + p / tiles_d;
    for (int dd = (int)threadIdx.x; dd < C::BN; dd += C::NT) {
      const int d = (p % tiles_d) * C::BN + dd;
      for (int ps = 0; ps < splits; ++ps) {
        float* o = ps == 0 ? dE : dE_part + (size_t)(ps - 1) * N * D;
        for (int r = 0; r < C::BM; ++r) {
          const int row = rowmap[tn * C::BM + r];
          if (row >= 0 && d < D) {
            if (o) o[(size_t)row * D + d] = 0.f;
            else dEb[(size_t)row * D + d] = 0;
          }
        }
      }
    }
    return;
  }
  const int n0 = tn * C::BM, d0 = td * C::BN;
  // token rows of the tile's compacted slots, for the epilogue (visible after
  // the barriers that end collect_kept)
  __shared__ int srow[C::BM];
  for (int i = threadIdx.x; i < C::BM; i += C::NT) srow[i] = rowmap[n0 + i];
  // this split's share of the token block's kept vocab blocks in the chunk:
  // the kept list cut into equal counts (with filtering, kept blocks gather
  // at the frequent targets, so equal vocab ranges would load one split)
  // (with, for bf16, each kept vocab block's G slot: A's K blocks, K offset
  // slot * 65536 from row n' * 256 of a slot; with block masks, the token
  // block's block-mask bytes of each: byte v vocab group v, bit t token
  // group t)
  const int nall = collect_kept<C::NT, kDma, MASK, DEMask>(keep, (size_t)tn * nvb_t + cvb0, 1, cnvb, slot, bmask,
                                                   (size_t)tn * nvg + (size_t)cvb0 * kBlocksPerTile,
                                                   kBlocksPerTile, blocks, ablk, (uint64_t*)smask);
  const int lo = (int)((int64_t)nall * s / splits), hi = (int)((int64_t)nall * (s + 1) / splits);
  const int nk = hi - lo;
  const uint16_t* bl = blocks + lo;
  const uint16_t* abl = ablk + lo;
  const uint64_t* sml = (const uint64_t*)smask + lo;

  // G rows n0.. over the chunk's vocabulary (K-major), from vocab offset ka
  // (fp32)
  auto a_op = [&](size_t ka) -> Operand {
    const size_t o = (size_t)n0 * Vc + ka;
    return make_operand(G + o, g_bytes - o * sizeof(T), (uint32_t)Vc, min(C::BM, N - n0), clen - (int)ka);
  };
  const Operand A = kDma ? make_operand(G, g_bytes, (uint32_t)kTileV, min(C::BM, N - n0), cap * kSlotRows * kTileV)
                         : a_op(0);
  Operand B = make_operand(c + (size_t)cv0 * D + d0, ((uint64_t)(V - cv0) * D - d0) * sizeof(T), (uint32_t)D,
               min(C::BN, D - d0), clen);
  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};
  constexpr int SPB = kTileV / C::BK;
  int ns = nk * SPB;  // steps that run
  if constexpr (MASK) {
    // the steps (64 vocab of one of the split's vocab blocks each) with a
    // nonzero block: the 16 bits of the two vocab-group bytes 2 (c % 4),
    // 2 (c % 4) + 1
    ns = collect_steps(nk * SPB, [&](int c) { return ((sml[c >> 2] >> (8 * (c & 3))) & kStepBits) != 0; }, steps);
  }
  auto loop = [&](const Operand& a, const Operand& b, const uint16_t* bl) {
    // the step's DMA in two parts (right after the barrier and in the first
    // K group) rather than three: measured faster for this kernel's
    // MN-major classifier tile, slower for the K-major ones
    if constexpr (MASK) {
      const int wm = (int)(threadIdx.x >> 6) / C::WAVES_N;
      const DEMask mk{(const lds_u64*)sml, 32 * wm};
      // the step list: when it leaves out at least an eighth of the steps
      if (8 * ns <= 7 * nk * SPB)
        mainloop_dma<C, SPB, true, false, 2, DEMask, true, DmaBlockK<C>, true>(acc, a, b, ns, bl, smem, nullptr, mk,
                                                                               abl, kSlotRows * kTileV, steps);
      else
        mainloop_dma<C, SPB, true, false, 2, DEMask, true, DmaBlockK<C>>(acc, a, b, nk * SPB, bl, smem, nullptr, mk,
                                                                         abl, kSlotRows * kTileV);
    } else if constexpr (kDma) {
      mainloop_dma<C, SPB, true, false, 2, NoMask, true, DmaBlockK<C>>(acc, a, b, nk * SPB, bl, smem, nullptr,
                                                                       NoMask{}, abl, kSlotRows * kTileV);
    } else {
      mainloop<C, false, true, SPB>(acc, a, b, nk * SPB, bl, (T*)smem);
    }
  };
  // the split's blocks consecutive (every block kept): contiguous K from its
  // first block (for bf16 in B only: A follows the slots)
  if (nk > 0 && (int)bl[nk - 1] - (int)bl[0] == nk - 1) {
    const size_t ka = (size_t)__builtin_amdgcn_readfirstlane((int)bl[0]) * kTileV;
    const Operand A1 = kDma ? A : a_op(ka);
    const Operand B1 = make_operand(c + ((size_t)cv0 + ka) * D + d0,
                                    ((uint64_t)(V - cv0 - (int64_t)ka) * D - d0) * sizeof(T), (uint32_t)D,
                                    min(C::BN, D - d0), clen - (int)ka);
    loop(A1, B1, nullptr);
  } else {
    loop(A, B, bl);
  }

  if (ns == 0 && (accumulate || atomic)) return;  // nothing to add
  // Rows of the tile are compacted slots n0..; slot n' is token row
  // srow[n' - n0] (ignored rows after the valid ones, -1 past N), so the first
  // write of dE also zeroes the ignored rows.  64-bit row pointers: the rows
  // of one tile may lie anywhere in dE.  Loads of old values are never
  // conditional (a masked-off element reads row 0), so each fm's loads stay
  // in flight together.
  AccMap<C> am;
  float* out = (atomic || s == 0) ? dE : dE_part + (size_t)(s - 1) * N * D;
  const bool full = n0 + C::BM <= N && d0 + C::BN <= D;  // no masked element
  int dcol[C::FN];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    const int d = d0 + am.colj(fn);
    dcol[fn] = d < D ? d : -1;
  }
  if (atomic) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = srow[am.row(fm, r)];
        float* rp = out + (size_t)(row >= 0 ? row : 0) * D;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          if (row >= 0 && dcol[fn] >= 0) unsafeAtomicAdd(rp + dcol[fn], acc[fm][fn][r]);
      }
    return;
  }
  // Accumulating into the previous chunks' sum: the old values of a row of
  // FN blocks are fetched together (one memory round trip per fm, not per
  // block), then added and stored.  The first write of dE (chunk 0, split 0)
  // adds the smoothing term r1 scale_n csum_d when csum is given.
  const bool rank1 = csum != nullptr && !accumulate && s == 0;
  float cs[C::FN];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) cs[fn] = (rank1 && dcol[fn] >= 0) ? r1 * csum[dcol[fn]] : 0.f;
  auto epilogue = [&](auto full_tile) __attribute__((always_inline)) {
    constexpr bool F = decltype(full_tile)::value;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      float* rp[16];
      bool rok[16];
      size_t rbase[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = srow[am.row(fm, r)];
        rok[r] = F || row >= 0;
        rbase[r] = (size_t)(F || row >= 0 ? row : 0) * D;
        rp[r] = out + rbase[r];
      }
      float old[C::FN][16];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int dc = F || dcol[fn] >= 0 ? dcol[fn] : 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) old[fn][r] = (accumulate && !out_bf16) ? rp[r][dc] : 0.f;
      }
      if (rank1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sr = scale_c[n0 + am.row(fm, r)];  // slots past the valid rows: 0
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn) old[fn][r] = sr * cs[fn];
        }
      }
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = acc[fm][fn][r] + old[fn][r];
          if (out_bf16) {
            const uint16_t b = __builtin_bit_cast(uint16_t, (__bf16)v);
            if constexpr (F) {
              dEb[rbase[r] + dcol[fn]] = b;
            } else {
              if (rok[r] && dcol[fn] >= 0) dEb[rbase[r] + dcol[fn]] = b;
            }
          } else if constexpr (F) {
            rp[r][dcol[fn]] = v;
          } else {
            if (rok[r] && dcol[fn] >= 0) rp[r][dcol[fn]] = v;
          }
        }
    }
  };
  if (full) epilogue(std::true_type{});
  else epilogue(std::false_type{});
}

// dE += dE_part[0] + dE_part[1] + ... in that order (deterministic).
__global__ __launch_bounds__(256) void dE_reduce_kernel(float* __restrict__ dE, const float* __restrict__ part,
                                                        size_t n4, int nparts, size_t stride4) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  f32x4 v = reinterpret_cast<f32x4*>(dE)[i];
  for (int p = 0; p < nparts; ++p) v += reinterpret_cast<const f32x4*>(part)[(size_t)p * stride4 + i];
  reinterpret_cast<f32x4*>(dE)[i] = v;
}

// bf16 dE from its fp32 accumulation: dE = bf16(acc + part[0] + part[1] + ...)
// in that order (deterministic), four elements per thread.
__global__ __launch_bounds__(256) void dE_finish_kernel(const float* __restrict__ acc,
                                                        const float* __restrict__ part, size_t n4, int nparts,
                                                        size_t stride4, uint16_t* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  f32x4 v = reinterpret_cast<const f32x4*>(acc)[i];
  for (int p = 0; p < nparts; ++p) v += reinterpret_cast<const f32x4*>(part)[(size_t)p * stride4 + i];
  const uint32_t lo = pack_bf16(v[0], v[1]), hi = pack_bf16(v[2], v[3]);
  reinterpret_cast<u32x2*>(out)[i] = u32x2{lo, hi};
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// dE[n][d] = r1 * scale[n] * csum[d]: the smoothing term, written before the
// fp32 atomics add the tiles' share.
__global__ __launch_bounds__(256) void fill_rank1_kernel(float* __restrict__ dE, const float* __restrict__ scale,
                                                         const float* __restrict__ csum, float r1, int N, int D) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)N * D) return;
  const int n = (int)(i / (size_t)D), d = (int)(i % (size_t)D);
  dE[i] = r1 * scale[n] * csum[d];
}

// ============================================================================
// Host launchers.
// ============================================================================
// Tile configuration of each contraction kernel: 256x256 work-group tiles of
// 2 x WN_x waves (one wave per SIMD with 2 x 2, two with 2 x 4).  dC and dE
// run two waves per SIMD: with most of their MFMAs (and, since the loads of
// all-zero blocks are skipped, much of their operand stream) gone on the
// filtered heads, the second wave covers the LDS latency the first waits on
// (measured: dC 2.6-3.9% faster; dE 4-10% faster with the loads skipped).
#ifndef CCE_WN_FWD
#define CCE_WN_FWD 2
#endif
#ifndef CCE_WN_GRAD
#define CCE_WN_GRAD 2
#endif
#ifndef CCE_WN_DC
#define CCE_WN_DC 4
#endif
#ifndef CCE_WN_DE
#define CCE_WN_DE 4
#endif
template <typename T> struct Cfgs;
template <> struct Cfgs<uint16_t> {
  using Fwd = Cfg<uint16_t, kTileV, kTileN, 2, CCE_WN_FWD>;
  using Grad = Cfg<uint16_t, kTileV, kTileN, 2, CCE_WN_GRAD>;
  using DC = Cfg<uint16_t, kTileV, kTileN, 2, CCE_WN_DC>;
  using DE = Cfg<uint16_t, kTileV, kTileN, 2, CCE_WN_DE>;
};
template <> struct Cfgs<float> {
  using Fwd = Cfg<float, kTileV, kTileN, 2, 2>;
  using Grad = Fwd;
  using DC = Fwd;
  using DE = Fwd;
};
static_assert(Cfgs<uint16_t>::Fwd::WM == kPartialWidth && Cfgs<float>::Fwd::WM == kPartialWidth, "partial width");
static_assert(Cfgs<uint16_t>::DC::BN == kTileN && Cfgs<uint16_t>::DE::BN == kTileN && Cfgs<float>::DE::BN == kTileN,
              "d tiles of the gradient contractions");

// out[d] = factor * sum_r w_r x[r][d] over R rows (colsum + colsum_reduce).
template <typename T>
static void launch_colsum(const T* x, const float* w, int R, int D, float factor, float* colpart, float* out,
                          hipStream_t st) {
  constexpr int VEC = Elem<T>::VEC;
  int rpb;
  const int nblk = colsum_blocks(R, rpb);  // <= kColBlocks: colpart holds [nblk][D]
  prof_before(kKColSum, st);
  hipLaunchKernelGGL(colsum_kernel<T>, dim3((D / VEC + 255) / 256, nblk), dim3(256), 0, st, x, w, R, D, rpb,
                     colpart);
  prof_after(kKColSum, st);
  prof_before(kKColReduce, st);
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((D + 63) / 64), dim3(1024), 0, st, colpart, nblk, D, factor,
                     out);
  prof_after(kKColReduce, st);
}

template <typename T>
static hipError_t launch_forward_t(const Problem& P, const Layout& L, hipStream_t st) {
  using C = typename Cfgs<T>::Fwd;
  const T* e = (const T*)P.e;
  const T* c = (const T*)P.c;
  const bool smooth = P.label_smoothing != 0.f;
  if (smooth) {
    // sum over the vocabulary of the classifier rows (and of the bias), kept
    // in the workspace for the backward's dE term
    launch_colsum<T>(c, nullptr, P.V, P.D, 1.f, L.colpart, L.csum, st);
    if (P.bias) {
      prof_before(kKVecSum, st);
      hipLaunchKernelGGL(vec_sum_kernel<T>, dim3(1), dim3(1024), 0, st, (const T*)P.bias, P.V, L.aux);
      prof_after(kKVecSum, st);
    }
  }
  const int tiles_v = (P.V + C::BM - 1) / C::BM, tiles_n = (P.N + C::BN - 1) / C::BN;
  const int total = tiles_v * tiles_n;
  prof_before(kKFwdTile, st);
  hipLaunchKernelGGL(fwd_tile_kernel<C>, dim3(total), dim3(C::NT), 0, st, c, e, (const T*)P.bias, P.N, P.D, P.V,
                     P.softcap, L.part, L.nVB, tiles_n, total);
  prof_after(kKFwdTile, st);
  prof_before(kKRows, st);
  if (smooth)
    hipLaunchKernelGGL((rows_kernel<T, true>), dim3((P.N + 3) / 4), dim3(256), 0, st, e, c, (const T*)P.bias,
                       P.targets, P.N, P.D, P.V, P.ignore_index, L.part, L.nVB, (const float*)L.csum,
                       (const float*)L.aux, P.label_smoothing, P.z_loss, P.softcap, P.lse, L.nll_out);
  else
    hipLaunchKernelGGL((rows_kernel<T, false>), dim3((P.N + 3) / 4), dim3(256), 0, st, e, c, (const T*)P.bias,
                       P.targets, P.N, P.D, P.V, P.ignore_index, L.part, L.nVB, (const float*)nullptr,
                       (const float*)nullptr, 0.f, P.z_loss, P.softcap, P.lse, L.nll_out);
  prof_after(kKRows, st);
  prof_before(kKReduce, st);
  hipLaunchKernelGGL(reduce_kernel, dim3(1), dim3(1024), 0, st, L.nll_out, P.targets, P.N, P.V, P.ignore_index,
                     P.reduction, P.loss, P.n_valid, L.hdr);
  prof_after(kKReduce, st);
  return hipGetLastError();
}

// An empty batch: the counters, the reduced loss (no term: 0 for sum, and
// for mean with its count floored at 1) and n_valid.
__global__ __launch_bounds__(64) void empty_batch_kernel(int32_t* __restrict__ hdr, float* __restrict__ loss,
                                                        int32_t* __restrict__ n_valid) {
  if (threadIdx.x < kHdrWords) hdr[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    if (loss) loss[0] = 0.f;
    if (n_valid) n_valid[0] = 0;
  }
}

__global__ __launch_bounds__(256) void zero_u32x4_kernel(u32x4* __restrict__ p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_empty(const Layout& L, float* loss, int32_t* n_valid, void* g, size_t gbytes, float* b, size_t nb,
                        hipStream_t st) {
  static_assert(kHdrWords <= 64, "one wave clears the counters");
  hipLaunchKernelGGL(empty_batch_kernel, dim3(1), dim3(64), 0, st, L.hdr, loss, n_valid);
  if (g && gbytes) {
    const size_t n = gbytes / 16;
    hipLaunchKernelGGL(zero_u32x4_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (u32x4*)g, n);
  }
  if (b && nb) hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, b, nb);
  return hipGetLastError();
}

hipError_t launch_forward(const Problem& P, const Layout& L, hipStream_t st) {
  return P.dtype == kDtypeBf16 ? launch_forward_t<uint16_t>(P, L, st) : launch_forward_t<float>(P, L, st);
}

template <typename T>
static hipError_t launch_backward_t(const Problem& P, const Layout& L, hipStream_t st) {
  using CG = typename Cfgs<T>::Grad;
  using CC = typename Cfgs<T>::DC;
  using CE = typename Cfgs<T>::DE;
  const T* e = (const T*)P.e;
  const T* c = (const T*)P.c;
  T* G = (T*)L.G;
  const bool smooth = P.label_smoothing != 0.f;
  // the smoothing term's coefficient -eps / V
  const float r1 = smooth ? (float)(-(double)P.label_smoothing / (double)P.V) : 0.f;
  prof_before(kKBwdPrep, st);
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(1), dim3(1024), 0, st, P.targets, P.N, L.Npad, P.V, P.ignore_index,
                     P.reduction, P.grad_loss, (const float*)P.lse, L.scale, L.rowmap, L.scale_c, L.lse_c, L.tgt_c,
                     L.hdr, smooth ? L.ssum : nullptr);
  prof_after(kKBwdPrep, st);
  // dE, dC and db are each optional (a null output is not formed)
  const bool want_dE = P.dE != nullptr, want_dC = P.dC != nullptr;
  // -eps/V * sum_i scale_i e_i: the smoothing share of every dC row
  if (smooth && want_dC) launch_colsum<T>(e, L.scale, P.N, P.D, r1, L.bcolpart, L.r1c, st);
  prof_before(kKFilter, st);
  hipLaunchKernelGGL(filter_kernel, dim3((L.nvb_t + 63) / 64, L.nb), dim3(1024), 0, st, P.targets, P.lse,
                     L.part, (const int*)L.rowmap, P.N, P.V, L.nVB, P.ignore_index, L.nvb_t, P.filter, L.keep,
                     L.bmask, L.nvg, L.hdr);
  prof_after(kKFilter, st);
  prof_before(kKTileList, st);
  // the chunks (compact storage: cut by kept tiles), then each chunk's list
  // (the tile lists are written after the plan: their space holds the
  // units' kept counts meanwhile)
  hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(1024), 0, st, (const uint8_t*)L.keep, L.nb, L.nvb_t, L.unit,
                     L.S, L.span_u, L.nchunks, L.ch_vb, L.tlist);
  hipLaunchKernelGGL(tile_list_kernel, dim3(L.nchunks), dim3(1024), 0, st, (const uint8_t*)L.keep, L.nvb_t,
                     L.Npad / kTileN, (const int*)L.ch_vb, L.list_stride, L.tlist, L.tcount,
                     L.compact ? L.slot : nullptr);
  prof_after(kKTileList, st);
  if (want_dC) {
    prof_before(kKTransE, st);
    hipLaunchKernelGGL(transpose_e_kernel<T>, dim3((P.D + 63) / 64, L.Npad / 64), dim3(256), 0, st, e,
                       (const int*)L.rowmap, (T*)L.Et, P.N, P.D, L.Npad);
    prof_after(kKTransE, st);
  }
  // dE: float output, or bf16 written straight by dE_gemm when a single pass
  // forms it (one vocab chunk, one split, no atomics), else accumulated in
  // fp32 (dE_acc) and rounded to bf16 at the end
  const int splits_used = P.accum == kAccumAtomic ? L.splits_atomic : L.splits;
  const bool bf_direct = P.grad_bf16 && L.nchunks == 1 && splits_used == 1 && P.accum != kAccumAtomic;
  float* dE32 = P.grad_bf16 ? (bf_direct ? nullptr : L.dE_acc) : (float*)P.dE;
  if (want_dE && P.accum == kAccumAtomic) {
    const size_t n = (size_t)P.N * P.D;
    if (smooth) {
      prof_before(kKFillRank1, st);
      hipLaunchKernelGGL(fill_rank1_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dE32, L.scale,
                         (const float*)L.csum, r1, P.N, P.D);
      prof_after(kKFillRank1, st);
    } else {
      prof_before(kKFill, st);
      hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dE32, n);
      prof_after(kKFill, st);
    }
  }
  const int tiles_n = L.Npad / kTileN;
  const int tiles_d = (P.D + kTileN - 1) / kTileN;  // d tiles of dC and dE (BN = 256)
  // block masks in the contractions: bf16 operands with filtering (fp32
  // operands form the same zero blocks of G and contract them densely)
  constexpr bool MaskOn = sizeof(T) == 2;
  const bool mask = MaskOn && P.filter != 0;
  // The chunks' vocabulary ranges are on the device (compact storage cuts
  // them by kept tiles): each grid covers the widest chunk possible and the
  // spare work-groups exit.  Dense storage (fp32): chunks of Vc columns.
  const int cvb = L.Vc / kTileV;
  const int wide = L.compact ? min(L.nvb_t, L.span_u * L.unit) : cvb;  // vocab tiles of the widest chunk
  const int gt_grid = L.compact ? L.cap : cvb * tiles_n;
  // dC: vocab-tile groups of at most kRasterDC dealt to the XCDs in turn
  // (dC_gemm_kernel): 8 x GR x tiles_d x ceil(groups / 8) <= tiles_d x
  // (tiles_v + 8 kRasterDC) work-groups for any chunk
  const int dc_grid = tiles_d * (wide + 8 * kRasterDC);
  for (int ch = 0; ch < L.nchunks; ++ch) {
    const int* chv = (const int*)L.ch_vb + ch;
    prof_before(kKGradTile, st);
    hipLaunchKernelGGL(grad_tile_kernel<CG>, dim3(gt_grid), dim3(CG::NT), 0, st, c, e, (const T*)P.bias,
                       (const int*)L.rowmap, (const int*)L.tgt_c, (const float*)L.lse_c, (const float*)L.scale_c,
                       P.label_smoothing, P.z_loss, P.softcap, (const int*)L.tlist + (size_t)ch * L.list_stride,
                       (const int*)L.tcount + ch, P.N, P.D, P.V, chv, tiles_n, L.Vc, L.gt_ld,
                       G, (T*)L.Gt, L.g_bytes, L.gt_bytes, P.dbias ? L.db_part : nullptr, L.bmask, L.nvg,
                       L.hdr, P.filter);
    prof_after(kKGradTile, st);
    if (want_dC) {
      prof_before(kKDC, st);
      // with filtering (bf16), the 32x32 block masks let dC skip zero blocks
      auto dck = mask ? dC_gemm_kernel<CC, MaskOn> : dC_gemm_kernel<CC, false>;
      hipLaunchKernelGGL(dck, dim3(dc_grid), dim3(CC::NT), 0, st, (const T*)G, (const T*)L.Gt,
                         (const T*)L.Et, L.keep, (const int*)L.slot, L.cap, L.Npad, L.gt_ld, P.D, P.V, L.nvb_t,
                         chv, tiles_d, L.g_bytes, L.gt_bytes, smooth ? (const float*)L.r1c : nullptr, P.dC,
                         P.grad_bf16, (const uint8_t*)L.bmask, L.nvg);
      prof_after(kKDC, st);
    }
    if (want_dE) {
      const int splits = splits_used;
      prof_before(kKDE, st);
      auto dek = mask ? dE_gemm_kernel<CE, MaskOn> : dE_gemm_kernel<CE, false>;
      hipLaunchKernelGGL(dek, dim3(tiles_n * tiles_d * splits), dim3(CE::NT), 0, st, G, c, L.keep,
                         (const int*)L.slot, L.cap, P.N, P.D, P.V, L.nvb_t, chv, tiles_n, tiles_d, splits,
                         (const int32_t*)L.hdr, L.Vc, L.g_bytes,
                         bf_direct ? P.dE : (void*)dE32, bf_direct ? 1 : 0, L.dE_part, ch > 0 ? 1 : 0,
                         P.accum == kAccumAtomic ? 1 : 0, (const int*)L.rowmap,
                         (const float*)L.scale_c,
                         smooth ? (const float*)L.csum : nullptr, r1, (const uint8_t*)L.bmask, L.nvg);
      prof_after(kKDE, st);
    }
  }
  if (P.dbias) {
    prof_before(kKDbReduce, st);
    hipLaunchKernelGGL(db_reduce_kernel, dim3((P.V + 255) / 256), dim3(256), 0, st, L.db_part, L.keep, L.nb,
                       L.nvb_t, P.V, smooth ? (const float*)L.ssum : nullptr, r1, P.dbias);
    prof_after(kKDbReduce, st);
  }
  const size_t n4 = (size_t)P.N * P.D / 4;  // D is a multiple of 4
  const int nparts = P.accum != kAccumAtomic ? L.splits - 1 : 0;
  if (!want_dE) return hipGetLastError();
  if (P.grad_bf16 && !bf_direct) {
    prof_before(kKDEReduce, st);
    hipLaunchKernelGGL(dE_finish_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                       (const float*)dE32, (const float*)L.dE_part, n4, nparts, n4, (uint16_t*)P.dE);
    prof_after(kKDEReduce, st);
  } else if (!P.grad_bf16 && nparts > 0) {
    prof_before(kKDEReduce, st);
    hipLaunchKernelGGL(dE_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, dE32, L.dE_part,
                       n4, nparts, n4);
    prof_after(kKDEReduce, st);
  }
  return hipGetLastError();
}

hipError_t launch_backward(const Problem& P, const Layout& L, hipStream_t st) {
  return P.dtype == kDtypeBf16 ? launch_backward_t<uint16_t>(P, L, st) : launch_backward_t<float>(P, L, st);
}

}  // namespace cce
