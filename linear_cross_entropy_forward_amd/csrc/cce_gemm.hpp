// LDS-tiled MFMA main loop shared by every contraction of the fused linear
// cross-entropy: the logit tiles S = C E^T of the forward and of the gradient
// recompute, and the two gradient contractions dE = G C and dC = G^T E.
//
// gfx950 (CDNA4) specifics:
//  * bf16 operands use v_mfma_f32_32x32x16_bf16 (8 bf16 per lane per operand,
//    fp32 accumulate); fp32 operands use v_mfma_f32_32x32x2_f32.
//  * wave64: a 32x32 output block lives in 16 accumulator registers per lane,
//    lane l owning column l%32 and rows 8*(r/4) + 4*(l/32) + r%4, r = 0..15.
//  * global traffic goes through buffer resources (raw buffer loads/stores)
//    whose range check returns zero for, or drops, every out-of-range access:
//    ragged tiles need no branches and cannot touch memory outside a tensor.
//  * tiles written to LDS by the waves carry a 16-byte row pad (a 144-byte row
//    stride puts any 16 consecutive rows, which one ds_read_b128 cycle of the
//    64-bank LDS serves, on distinct banks); tiles the DMA path writes are
//    swizzled instead (see DmaTile).
//  * operands whose contraction index is the slow (row) index in memory
//    ("MN-major", e.g. C read as C[v][d] when contracting over v) are loaded
//    as VECxVEC blocks and transposed in registers before the LDS store, so the
//    fragment reads are always K-contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace cce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Pointer into LDS (address space 3): keeps fragment reads and tile stores on
// the ds_* path instead of generic (flat) addressing.
template <typename T> using lds_ptr = __attribute__((address_space(3))) T*;
template <typename T> __device__ __forceinline__ lds_ptr<T> to_lds(T* p) { return (lds_ptr<T>)p; }

// Word 3 of a raw (unstructured) buffer descriptor on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;
// Any byte offset at or beyond a descriptor's num_records reads as zero and is
// dropped on store; this value is used to switch an access off.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  uint32_t n = bytes > 0x7fffffffull ? 0x7fffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

__device__ __forceinline__ u32x4 ld128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// Cache-policy bit of a buffer store: non-temporal (streaming).  Used for
// outputs written once and not read again soon (the gradient tiles, dC): the
// writes then leave the caches sooner, measured faster for these bursts.
constexpr int kStoreNT = 2;
__device__ __forceinline__ void st64(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

// ----------------------------------------------------------------------------
// Element types.  bf16 tensors are carried as their 16-bit patterns.
// ----------------------------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int VEC = 8;   // elements per 16-byte vector
  static constexpr int BK = 64;   // K elements staged per main-loop step
};
template <> struct Elem<float> {
  static constexpr int VEC = 4;
  static constexpr int BK = 32;
};

// A lane's share of one 32x16 (K) operand slice: 8 consecutive K elements.
template <typename T> struct Frag;
template <> struct Frag<uint16_t> { u32x4 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

__device__ __forceinline__ void lds_frag(Frag<uint16_t>& f, lds_ptr<uint16_t> p) {
  f.v = *(__attribute__((address_space(3))) u32x4*)p;
}
__device__ __forceinline__ void lds_frag(Frag<float>& f, lds_ptr<float> p) {
  f.lo = *(__attribute__((address_space(3))) f32x4*)p;
  f.hi = *(__attribute__((address_space(3))) f32x4*)(p + 4);
}
__device__ __forceinline__ void lds_st128(lds_ptr<uint16_t> p, u32x4 v) {
  *(__attribute__((address_space(3))) u32x4*)p = v;
}
__device__ __forceinline__ void lds_st128(lds_ptr<float> p, u32x4 v) {
  *(__attribute__((address_space(3))) u32x4*)p = v;
}

// acc += A(32x16) * B(16x32) for one K group of 16.
__device__ __forceinline__ void mma16(f32x16& acc, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}
// fp32: eight K=2 steps.  Lane half h holds K elements 8h..8h+7 of the group;
// step j pairs element j of both halves, so the eight steps cover the 16
// elements once each with A and B indexed identically.
__device__ __forceinline__ void mma16(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[j], b.lo[j], acc, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[j], b.hi[j], acc, 0, 0, 0);
}

// ----------------------------------------------------------------------------
// Register transposes of one VECxVEC block (rows in, columns out).
// ----------------------------------------------------------------------------
__device__ __forceinline__ void transpose_block(u32x4 (&r)[8], const uint16_t*) {
  // 8x8 of 16-bit elements.  Row i word q holds elements (2q, 2q+1) of row i.
  u32x4 o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t a = r[2 * p][q], b = r[2 * p + 1][q];
      o[2 * q][p] = (a & 0xffffu) | (b << 16);
      o[2 * q + 1][p] = (a >> 16) | (b & 0xffff0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = o[i];
}
__device__ __forceinline__ void transpose_block(u32x4 (&r)[4], const float*) {
  u32x4 o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[j][i] = r[i][j];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = o[i];
}

// ----------------------------------------------------------------------------
// Tile configuration.
// ----------------------------------------------------------------------------
template <typename T_, int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct Cfg {
  using T = T_;
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int BK = Elem<T>::BK;
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int LDK = BK + VEC;  // padded LDS row, elements
  static constexpr int KGROUPS = BK / 16;
  static constexpr int STAGE_ELEMS = (BM + BN) * LDK;
  static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * (int)sizeof(T);
  // two stages of unpadded (swizzled) rows for the LDS-DMA main loop
  static constexpr int LDS_DMA_BYTES = 2 * (BM + BN) * BK * (int)sizeof(T);
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
};

// One operand of the main loop.  K-major: element (row, k) at row*ld + k,
// rows [0, rows) valid.  MN-major: element (row, k) at k*ld + row, columns
// [0, rows) valid.  k in [0, kdim) valid.  Offsets are relative to `r`,
// which the caller has positioned at the tile's first row (K-major) or at
// k = 0 and the tile's first column (MN-major).
struct Operand {
  rsrc_t r;
  uint32_t ld;    // elements
  int rows;       // valid rows (K-major) or valid columns (MN-major) in the tile
  int kdim;       // valid K extent (relative to the same origin)
  u32x4 desc;     // the descriptor of `r` as four words, for the LDS-DMA loads
};

__device__ __forceinline__ Operand make_operand(const void* base, uint64_t bytes, uint32_t ld, int rows, int kdim) {
  const uint64_t a = (uint64_t)base;
  const uint32_t n = bytes > 0x7fffffffull ? 0x7fffffffu : (uint32_t)bytes;
  return Operand{make_rsrc(base, bytes), ld, rows, kdim,
                 u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, n, (uint32_t)kRsrcWord3}};
}

template <class C, int ROWS, bool MN>
struct Loader;

// K-major: 16-byte chunks along K, ROWS*BK/VEC chunks per tile.
template <class C, int ROWS>
struct Loader<C, ROWS, false> {
  using T = typename C::T;
  static constexpr int CPR = C::BK / C::VEC;            // chunks per row
  static constexpr int N = ROWS * CPR / C::NT;          // chunks per thread
  static_assert(ROWS * CPR % C::NT == 0, "tile not evenly split");
  u32x4 reg[N];
  __device__ __forceinline__ void load(const Operand& op, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int c = tid + i * C::NT;
      int row = c / CPR, kc = (c % CPR) * C::VEC + k0;
      bool ok = row < op.rows && kc < op.kdim;
      uint32_t off = ok ? ((uint32_t)row * op.ld + (uint32_t)kc) * (uint32_t)sizeof(T) : kOOB;
      reg[i] = ld128(op.r, off);
    }
  }
  __device__ __forceinline__ void store(lds_ptr<T> lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int c = tid + i * C::NT;
      int row = c / CPR, kc = (c % CPR) * C::VEC;
      lds_st128(lds + row * C::LDK + kc, reg[i]);
    }
  }
  // Part P of NP: chunks [P*N/NP, (P+1)*N/NP) only.
  static constexpr int part_lo(int P, int NP) { return P * N / NP; }
  template <int P, int NP>
  __device__ __forceinline__ void store_part(lds_ptr<T> lds, int tid) const {
#pragma unroll
    for (int i = part_lo(P, NP); i < part_lo(P + 1, NP); ++i) {
      int c = tid + i * C::NT;
      int row = c / CPR, kc = (c % CPR) * C::VEC;
      lds_st128(lds + row * C::LDK + kc, reg[i]);
    }
  }
  template <int P, int NP>
  __device__ __forceinline__ void load_part(const Operand& op, int k0, int tid) {
#pragma unroll
    for (int i = part_lo(P, NP); i < part_lo(P + 1, NP); ++i) {
      int c = tid + i * C::NT;
      int row = c / CPR, kc = (c % CPR) * C::VEC + k0;
      bool ok = row < op.rows && kc < op.kdim;
      uint32_t off = ok ? ((uint32_t)row * op.ld + (uint32_t)kc) * (uint32_t)sizeof(T) : kOOB;
      reg[i] = ld128(op.r, off);
    }
  }
  template <int NP> static constexpr int stores_in_part(int P) { return part_lo(P + 1, NP) - part_lo(P, NP); }
};

// MN-major: VECxVEC blocks, transposed in registers.
template <class C, int ROWS>
struct Loader<C, ROWS, true> {
  using T = typename C::T;
  static constexpr int V = C::VEC;
  static constexpr int KB = C::BK / V;                  // blocks along K
  static constexpr int UNITS = KB * (ROWS / V);
  static constexpr int N = UNITS / C::NT;               // blocks per thread
  static_assert(UNITS % C::NT == 0, "tile not evenly split");
  u32x4 reg[N][V];
  __device__ __forceinline__ void load(const Operand& op, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int u = tid + i * C::NT;
      int kb = u % KB, mb = u / KB;
      int col = mb * V;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        int k = k0 + kb * V + j;
        bool ok = k < op.kdim && col < op.rows;
        uint32_t off = ok ? ((uint32_t)k * op.ld + (uint32_t)col) * (uint32_t)sizeof(T) : kOOB;
        reg[i][j] = ld128(op.r, off);
      }
    }
  }
  __device__ __forceinline__ void store(lds_ptr<T> lds, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int u = tid + i * C::NT;
      int kb = u % KB, mb = u / KB;
      transpose_block(reg[i], (const T*)nullptr);
#pragma unroll
      for (int j = 0; j < V; ++j) lds_st128(lds + (mb * V + j) * C::LDK + kb * V, reg[i][j]);
    }
  }
  // Part P of NP: part 0 transposes every block; part P stores columns
  // [P*V/NP, (P+1)*V/NP) of each block, and load_part reloads the same rows
  // (their registers are free once those columns are stored).
  static constexpr int part_lo(int P, int NP) { return P * V / NP; }
  template <int P, int NP>
  __device__ __forceinline__ void store_part(lds_ptr<T> lds, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int u = tid + i * C::NT;
      int kb = u % KB, mb = u / KB;
      if (P == 0) transpose_block(reg[i], (const T*)nullptr);
#pragma unroll
      for (int j = part_lo(P, NP); j < part_lo(P + 1, NP); ++j)
        lds_st128(lds + (mb * V + j) * C::LDK + kb * V, reg[i][j]);
    }
  }
  template <int P, int NP>
  __device__ __forceinline__ void load_part(const Operand& op, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int u = tid + i * C::NT;
      int kb = u % KB, mb = u / KB;
      int col = mb * V;
#pragma unroll
      for (int j = part_lo(P, NP); j < part_lo(P + 1, NP); ++j) {
        int k = k0 + kb * V + j;
        bool ok = k < op.kdim && col < op.rows;
        uint32_t off = ok ? ((uint32_t)k * op.ld + (uint32_t)col) * (uint32_t)sizeof(T) : kOOB;
        reg[i][j] = ld128(op.r, off);
      }
    }
  }
  template <int NP> static constexpr int stores_in_part(int P) { return N * (part_lo(P + 1, NP) - part_lo(P, NP)); }
};

// Scheduling pattern for one K group: MM MFMAs, each followed by up to PER of
// the group's other instructions in the order NR LDS reads, NW LDS writes,
// NL global loads (sched_group_barrier masks 0x008 MFMA, 0x100 DS read,
// 0x200 DS write, 0x020 VMEM read).
template <int T, int NR, int NW, int NL>
__device__ __forceinline__ void pattern_extra() {
  if constexpr (T < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  else if constexpr (T < NR + NW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
  else if constexpr (T < NR + NW + NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
}
template <int M, int PER, int NR, int NW, int NL>
__device__ __forceinline__ void pattern_slot() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  [&]<int... Q>(std::integer_sequence<int, Q...>) {
    (pattern_extra<M * PER + Q, NR, NW, NL>(), ...);
  }(std::make_integer_sequence<int, PER>{});
}
template <int MM, int NR, int NW, int NL>
__device__ __forceinline__ void issue_pattern() {
  constexpr int extra = NR + NW + NL;
  constexpr int per = (extra + MM - 1) / MM;
  [&]<int... M>(std::integer_sequence<int, M...>) {
    (pattern_slot<M, per, NR, NW, NL>(), ...);
  }(std::make_integer_sequence<int, MM>{});
}

// Main loop: acc[fm][fn] += sum over the listed K steps of A_tile * B_tile^T.
// `nsteps` K steps of BK each; step s covers K offset kofs(s).  With
// `blocks` == nullptr the steps are contiguous from 0; otherwise step s lies in
// K block blocks[s / SPB] (of SPB*BK elements) at sub-step s % SPB.
//
// Pipeline: two register sets alternate as global prefetch buffers, so the
// loads of step s+3 are issued in the middle of step s, right after the data
// of step s+1 has been written to the idle LDS stage: every load has about
// two steps of MFMA work to land.  Within a step the MFMAs of K group g run
// while the fragments of group g+1 are read from LDS.  One barrier per step,
// placed before the last K group: by then every wave has issued its last
// fragment reads of the current stage and its stores to the next one, so the
// last group's MFMAs cover the reads of the next step's first fragments and
// no step starts on an LDS round trip.
// Steps past the end (the count is padded to even) address K = kdim and read
// zeros, so the loop body has no branches.
template <class C, bool A_MN, bool B_MN, int SPB>
__device__ __forceinline__ void mainloop(f32x16 (&acc)[C::FM][C::FN], const Operand& A,
                                         const Operand& B, int nsteps, const uint16_t* blocks,
                                         typename C::T* smem) {
  using T = typename C::T;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  // stage st: A tile at st*STAGE_ELEMS, B tile right after it
  const lds_ptr<T> base = to_lds(smem);
  constexpr int BOFF = C::BM * C::LDK;
  constexpr int KG = C::KGROUPS;
  static_assert(KG % 2 == 0, "fragment buffers alternate per K group");
  if (nsteps <= 0) return;
  const int kend = A.kdim > B.kdim ? A.kdim : B.kdim;

  auto kofs = [&](int s) -> int {
    if (s >= nsteps) return kend;
    return blocks ? (int)blocks[s / SPB] * (SPB * C::BK) + (s % SPB) * C::BK : s * C::BK;
  };

  Loader<C, C::BM, A_MN> la0, la1;
  Loader<C, C::BN, B_MN> lb0, lb1;
  la0.load(A, kofs(0), tid);
  lb0.load(B, kofs(0), tid);
  la1.load(A, kofs(1), tid);
  lb1.load(B, kofs(1), tid);
  la0.store(base, tid);
  lb0.store(base + BOFF, tid);
  la0.load(A, kofs(2), tid);
  lb0.load(B, kofs(2), tid);
  __syncthreads();

  // Fragment read offsets within a stage.
  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  const int a_base = (wm * C::WM + frow) * C::LDK + fk;
  const int b_base = BOFF + (wn * C::WN + frow) * C::LDK + fk;

  Frag<T> fa[2][C::FM], fb[2][C::FN];
  // MFMA instructions per K group and LDS reads per fragment for the issue
  // pattern below
  constexpr int MMAS = C::FM * C::FN * (sizeof(T) == 2 ? 1 : 8);
  constexpr int LDS_READS_PER_FRAG = sizeof(T) == 2 ? 1 : 2;
  auto read_frags = [&](int buf, lds_ptr<T> st, int g) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) lds_frag(fa[buf][i], st + a_base + i * 32 * C::LDK + g * 16);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) lds_frag(fb[buf][j], st + b_base + j * 32 * C::LDK + g * 16);
  };
  read_frags(0, base, 0);

  // One step computing from stage `st`.  The prefetch set (lsa, lsb) holds
  // step s+1; during the first KG-1 groups it is written to stage `nx` part by
  // part, and each part's registers are reloaded with step s+3 right after.
  // The stores and loads are spread between the MFMAs instead of issued in one
  // burst: a burst fills the LDS write queue and stalls the only wave on the
  // SIMD, idling the matrix core.
  constexpr int NP = KG > 1 ? KG - 1 : 1;
  auto step = [&](int s, lds_ptr<T> st, lds_ptr<T> nx, auto& lsa, auto& lsb) {
    const int k3 = kofs(s + 3);
    auto group = [&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g + 1 < KG) {
        read_frags((g + 1) & 1, st, g + 1);
      } else {
        __syncthreads();
        read_frags(0, nx, 0);
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) mma16(acc[i][j], fa[g & 1][i], fb[g & 1][j]);
      if constexpr (g < NP) {
        lsa.template store_part<g, NP>(nx, tid);
        lsb.template store_part<g, NP>(nx + BOFF, tid);
        lsa.template load_part<g, NP>(A, k3, tid);
        lsb.template load_part<g, NP>(B, k3, tid);
      }
      // issue order within the group: MFMAs interleaved with the next group's
      // fragment reads, then with this part's LDS stores and global loads
      constexpr int nr = (C::FM + C::FN) * LDS_READS_PER_FRAG;
      constexpr int nw = g < NP ? std::remove_reference_t<decltype(lsa)>::template stores_in_part<NP>(g) +
                                      std::remove_reference_t<decltype(lsb)>::template stores_in_part<NP>(g)
                                : 0;
      issue_pattern<MMAS, nr, nw, nw>();
      __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... G>(std::integer_sequence<int, G...>) {
      (group(std::integral_constant<int, G>{}), ...);
    }(std::make_integer_sequence<int, KG>{});
  };

  const lds_ptr<T> st0 = base, st1 = base + C::STAGE_ELEMS;
  for (int s = 0; s < nsteps; s += 2) {
    step(s, st0, st1, la1, lb1);       // set 1 holds step s+1
    step(s + 1, st1, st0, la0, lb0);   // set 0 holds step s+2
  }
  __syncthreads();  // the last group's reads are done before the caller may reuse LDS
}

// ============================================================================
// LDS-DMA main loop for two K-major operands.
//
// gfx950 can write a buffer load straight into LDS (16 bytes per lane, lane l
// landing at M0 + 16 l).  Feeding both tiles this way removes the LDS stores
// and their staging registers from the waves: with one wave per SIMD every
// ds_write_b128 issued between MFMAs costs the matrix core about two dozen
// cycles, while a buffer load costs next to nothing.
//
// Tile layout: BK elements = 128 bytes per row, no padding.  The 16-byte chunk
// c of row r is stored in slot c ^ swz(r), swz(r) = (r % 8) ^ (r / 8 % 2).  A
// fragment read serves 16 lanes (one chunk of 16 consecutive rows, 256 bytes)
// per cycle of the 64-bank LDS; two rows 128 bytes apart fall on the two bank
// halves, so the 16 pieces are conflict free when the even rows take eight
// distinct slots and so do the odd rows, which swz gives (it also keeps any 8
// consecutive rows in distinct slots).  The plain (r % 8) swizzle repeats
// every 8 rows and measured two-way conflicts on every read.  A contiguous
// 1 KB DMA write could not produce a padded layout; this one needs none.  One
// DMA instruction fills 8 rows; lane l writes slot l % 8 of row r = 8 i + l / 8
// and therefore fetches logical chunk (l % 8) ^ swz(r) of that row.
// ============================================================================

// One 16-byte-per-lane buffer load into LDS at lds_addr + 16 * lane.  Written
// as assembly: the instruction returns nothing to registers, and the
// compiler's own wait insertion, which cannot tell the LDS stages apart, would
// otherwise drain every DMA before each fragment read.  The main loop waits
// for these loads itself (wait_vmcnt) before the barrier that publishes them.
__device__ __forceinline__ void dma16(const u32x4& desc, uint32_t voff, uint32_t lds_addr) {
  // one wait state between the M0 write and the LDS-DMA instruction reading it
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(desc)
               : "memory", "m0");
}
// The same, for loads issued under a wave-uniform branch (the block-layout
// tiles, whose loads of all-zero blocks are skipped): readfirstlane keeps
// lds_addr in a scalar register, where the compiler would otherwise carry
// it in a vector one across the branch.
__device__ __forceinline__ void dma16_branch(const u32x4& desc, uint32_t voff, uint32_t lds_addr) {
  dma16(desc, voff, __builtin_amdgcn_readfirstlane(lds_addr));
}

// s_waitcnt vmcnt(n), other counters unconstrained (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ void lds_frag_at(Frag<uint16_t>& f, const lds_u8* st, uint32_t lo, uint32_t) {
  f.v = *(const __attribute__((address_space(3))) u32x4*)(st + lo);
}
__device__ __forceinline__ void lds_frag_at(Frag<float>& f, const lds_u8* st, uint32_t lo, uint32_t hi) {
  f.lo = *(const __attribute__((address_space(3))) f32x4*)(st + lo);
  f.hi = *(const __attribute__((address_space(3))) f32x4*)(st + hi);
}

// A DMA-fed tile provides: BYTES (one stage), PER (DMA instructions per wave
// per step), init(op) and issue(i, op, k0, tile) for the loads, and
// frag_init(rc0) / read(f, st, g, j) for fragment j (the 32 rows or columns
// starting at rc0 + 32 j) of K group g.

// K-major operand: ROWS rows of BK elements (128 bytes).  KFULL: every step
// inside the K extent is whole (kdim a multiple of BK, step offsets multiples
// of BK), so only a step past the end needs zeros, a scalar decision.
template <class C, int ROWS, bool KFULL = false>
struct DmaTile {
  using T = typename C::T;
  static constexpr int ROWB = C::BK * (int)sizeof(T);
  static_assert(ROWB == 128, "DMA-fed rows are 128 bytes");
  static constexpr int BYTES = ROWS * ROWB;
  static constexpr int NW = C::NT / 64;
  static constexpr int PER = BYTES / 1024 / NW;  // DMA instructions per wave per step
  static_assert(BYTES % (1024 * NW) == 0, "tile not evenly split");
  static_assert(PER % 2 == 0, "instruction parity gives the row's swizzle");
  static constexpr int KG = C::KGROUPS;
  // slot of logical chunk c in row r: c ^ swz(r)
  __device__ static constexpr int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
  // byte offset of the lane's row, kOOB past the valid rows (KFULL: plus the
  // lane's chunk)
  uint32_t roff[PER];
  uint32_t kc[2];      // K offset (elements) of the lane's chunk within a step, by instruction parity
  uint32_t mwave;      // LDS byte offset of the wave's first rows in a stage
  uint32_t flo[KG], fhi[KG];  // fragment chunk offsets by K group (fp32: two chunks)
  // With `rowmap`, tile row r is row rowmap[r] of the operand (-1: none).
  __device__ __forceinline__ void init(const Operand& op, const int* __restrict__ rowmap = nullptr) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    mwave = (uint32_t)(wave * PER) * 1024u;
    // instruction i fills rows 8 (wave PER + i) .. +7: row % 16 / 8 is the
    // parity of i (PER is even)
#pragma unroll
    for (int p = 0; p < 2; ++p) kc[p] = (uint32_t)(((lane & 7) ^ swz(8 * p + (lane >> 3))) * C::VEC);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int row = 8 * (wave * PER + i) + (lane >> 3);
      const int src = row < op.rows ? (rowmap ? rowmap[row] : row) : -1;
      roff[i] = src >= 0 ? (uint32_t)src * op.ld * (uint32_t)sizeof(T) + (KFULL ? kc[i & 1] * (uint32_t)sizeof(T) : 0u)
                         : kOOB;
    }
  }
  // DMA instruction i of this wave for the step at K offset k0 into the tile
  // whose LDS byte address is `tile` (wave-uniform).  KFULL: a step past the
  // end adds kOOB, which puts every valid row's offset at or past 2^31,
  // beyond any buffer (a kOOB row then wraps to an offset inside the buffer:
  // it feeds only outputs past the tile, and only in such a step, where the
  // other operand is zero).
  __device__ __forceinline__ void issue(int i, const Operand& op, int k0, uint32_t tile) const {
    if constexpr (KFULL) {
      const uint32_t sk = (uint32_t)k0 < (uint32_t)op.kdim ? (uint32_t)k0 * (uint32_t)sizeof(T) : kOOB;
      dma16(op.desc, roff[i] + sk, tile + mwave + (uint32_t)i * 1024u);
    } else {
      const uint32_t kk = (uint32_t)k0 + kc[i & 1];
      const uint32_t off = (roff[i] == kOOB || kk >= (uint32_t)op.kdim) ? kOOB : roff[i] + kk * (uint32_t)sizeof(T);
      dma16(op.desc, off, tile + mwave + (uint32_t)i * 1024u);
    }
  }
  // Lane l of a fragment reads row rc0 + 32 j + l % 32 (rc0 a multiple of 8),
  // K elements 8 (l / 32) .. +7 of the group.
  __device__ __forceinline__ void frag_init(int rc0) {
    const int lane = threadIdx.x & 63;
    const int row = rc0 + (lane & 31);
    const int sw = swz(row);
    constexpr int CPG = 16 / C::VEC;  // chunks per K group of 16
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      const int c = CPG * g + (CPG / 2) * (lane >> 5);
      flo[g] = (uint32_t)(row * ROWB + ((c ^ sw) << 4));
      fhi[g] = (uint32_t)(row * ROWB + (((c + 1) ^ sw) << 4));
    }
  }
  __device__ __forceinline__ void read(Frag<T>& f, const lds_u8* st, int g, int j) const {
    lds_frag_at(f, st, flo[g] + j * 32 * ROWB, fhi[g] + j * 32 * ROWB);
  }
};

// MN-major bf16 operand (element (col, k) at k*ld + col): BK rows, one per K
// index, of COLS columns (512 bytes), loaded as they lie in memory.  Chunk c
// (columns 8c..8c+7) of K row k sits in slot c ^ swz(k), swz(k) = 2 (k % 4) ^
// 8 (k % 2).  Fragments come
// from the transposing read ds_read_b64_tr_b16: within each group of 16
// lanes, output lane i element e is element i % 4 of the 8 bytes addressed by
// source lane i / 4 + 4 e.  Source lane s addresses K row k0 + s / 4, columns
// c0 + 4 (s % 4) .. +3, so output lane i receives column c0 + i at K rows
// k0..k0+3; two such reads give a lane its 8 K elements.  The sixteen 8-byte
// pieces of one group cover four rows and two chunks, and the 32 pieces that
// share a cycle of the 64-bank LDS (two groups: four rows, four chunks) cover
// sixteen slots that are distinct modulo 16 (256 bytes) under the swizzle: no
// bank conflicts.
template <class C, int COLS, int NF>
struct DmaTileMN {
  using T = typename C::T;
  static_assert(sizeof(T) == 2, "transposing fragment reads are for 16-bit operands");
  static constexpr int ROWB = COLS * (int)sizeof(T);
  static_assert(ROWB == 512, "DMA-fed K rows are 512 bytes");
  static constexpr int RPI = 1024 / ROWB;  // K rows per DMA instruction
  static constexpr int BYTES = C::BK * ROWB;
  static constexpr int NW = C::NT / 64;
  static constexpr int PER = BYTES / 1024 / NW;
  static_assert(BYTES % (1024 * NW) == 0 && PER % 2 == 0, "tile not evenly split");
  static constexpr int FN = NF;  // fragments per wave
  __device__ static constexpr int swz(int k) { return 2 * (k & 3) ^ 8 * (k & 1); }
  // by instruction parity: the byte offset of the lane's chunk in its K row
  // (K row RPI * (the wave's first instruction) + lane / 32), kOOB past the
  // columns
  uint32_t vrow[2];
  uint32_t mwave;  // LDS byte offset of the wave's first instruction's rows in a stage
  uint32_t foff[FN];
  __device__ __forceinline__ void init(const Operand& op) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int rsub = lane / 32, slot = lane & 31;
    mwave = (uint32_t)(wave * PER) * 1024u;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = slot ^ swz(RPI * p + rsub);
      vrow[p] = c * 8 < op.rows ? (uint32_t)(RPI * wave * PER + rsub) * op.ld * (uint32_t)sizeof(T) + (uint32_t)c * 16u
                                : kOOB;
    }
  }
  // K rows k0 + RPI (wave PER + i) + lane / 32.  In a step inside the K
  // extent the scalar part is below 2^31, so a lane past the columns (lane
  // part kOOB) lands at or past 2^31, beyond any buffer (zeros).  A step past
  // the extent (k0 >= kdim) takes kOOB as its scalar part, which puts every
  // lane with a valid column past the buffer as well; a lane past the
  // columns then wraps to an offset inside the buffer, but it feeds only
  // output columns past the tile, and only in a step whose other operand is
  // zero.  A step that straddles kdim occurs only at the end of the
  // operand's rows, where its buffer ends.
  __device__ __forceinline__ void issue(int i, const Operand& op, int k0, uint32_t tile) const {
    const uint32_t rb = op.ld * (uint32_t)sizeof(T);
    const uint32_t sk = (uint32_t)k0 < (uint32_t)op.kdim ? (uint32_t)k0 * rb : kOOB;
    dma16(op.desc, vrow[i & 1] + (sk + (uint32_t)(RPI * i) * rb), tile + mwave + (uint32_t)i * 1024u);
  }
  __device__ __forceinline__ void frag_init(int rc0) {
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, sl = lane & 15;
    const int krow = 8 * (grp >> 1) + (sl >> 2);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = rc0 + 32 * j + 16 * (grp & 1) + 4 * (sl & 3);
      foff[j] = (uint32_t)(krow * ROWB + (((col >> 3) ^ swz(krow)) << 4) + ((col & 7) << 1));
    }
  }
  __device__ __forceinline__ void read(Frag<T>& f, const lds_u8* st, int g, int j) const {
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + foff[j] + 16 * g * ROWB));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + foff[j] + (16 * g + 4) * ROWB));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    f.v = u32x4{ua[0], ua[1], ub[0], ub[1]};
  }
};

// ----------------------------------------------------------------------------
// The gradient tiles stored by 32x32 blocks (compact storage, bf16): slot j
// of G holds a 256 x 256 tile as 64 blocks, block (t, v) (token group t,
// vocab group v) at element j * 65536 + (8 t + v) * 1024, each [32 tokens]
// [32 vocab] row-major (rows of 64 bytes).  A K step of 64 reads 16 blocks,
// each block 2 KB of the stage, by two DMA instructions of 16 rows (1 KB).
// The step's slot and position come from the A K offset of the main loop
// (SEPA): ka = slot * STRIDE + q * 64, q the step's quarter of the tile.
// Past the last step ka is the slot count, whose offsets lie outside G: the
// loads read zeros.  (Not issuing the loads of zero blocks, by a branch or
// with EXEC off, measured 5-8% slower for dC and dE at the Llama-3.1-8B
// head, where 36% of the blocks are kept; whole K steps without a kept block
// are left out of the step list instead.)
// ----------------------------------------------------------------------------
// dE's A = G (rows: tokens, K: vocab).  Stage block k = 8 h + t: token group
// t, vocab group 2 q + h.  In LDS the 16-byte chunk c of block row r sits in
// slot c ^ ((r >> 2) & 3): the 16 rows one ds_read_b128 cycle serves then
// cover 16 distinct slots modulo 256 bytes (conflict free).
template <class C>
struct DmaBlockK {
  static_assert(sizeof(typename C::T) == 2 && C::BK == 64 && C::BM == 256, "bf16 256-row tiles, 64-deep steps");
  using T = typename C::T;
  static constexpr int BYTES = 16 * 2048;
  static constexpr int NW = C::NT / 64;
  static constexpr int PER = 32 / NW;  // DMA instructions per wave per step
  static constexpr int KG = C::KGROUPS;
  // Half block d of a step (d = 2 k + half, stage block k = 8 h + t: token
  // group t, vocab group 2 q + h) lies at slot * 131072 + q * 4096 + part(d)
  // in G (block t * 8 + 2 q + h of the slot).  part() is additive over the
  // wave's first half block and the instruction index (their bit fields do
  // not overlap), so an instruction's offset is a per-wave lane constant plus
  // one scalar.
  __device__ static constexpr uint32_t part(int d) {
    return (uint32_t)((((d >> 1) & 7) * 8 + (d >> 4)) * 2048 + (d & 1) * 1024);
  }
  static constexpr bool additive() {
    for (int w = 0; w < NW; ++w)
      for (int i = 0; i < PER; ++i)
        if (part(w * PER + i) != part(w * PER) + part(i)) return false;
    return true;
  }
  static_assert(additive(), "half-block offsets split into wave and instruction parts");
  uint32_t vlane;      // the lane's 16 bytes within its half block, plus the wave's part
  uint32_t mwave;      // LDS byte offset of the wave's first half block in a stage
  uint32_t fbase[KG];  // fragment 0's LDS offset by K group
  __device__ __forceinline__ void init(const Operand&) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // lane l writes LDS chunk l % 4 of half-block row l / 4: logical chunk
    // (l % 4) ^ ((l >> 4) & 3) of that row
    const int r = lane >> 2, c = (lane & 3) ^ ((lane >> 4) & 3);
    vlane = (uint32_t)((r * 32 + c * 8) * 2) + part(wave * PER);
    mwave = (uint32_t)(wave * PER) * 1024u;
  }
  // ka = slot * 65536 + 64 q (q: the step within the slot's vocab tile);
  // past the last step ka = kend, slot >= cap: every offset lies past the
  // buffer (zeros)
  __device__ __forceinline__ void issue(int i, const Operand& op, int ka, uint32_t tile) const {
    const uint32_t sbase = ((uint32_t)ka >> 16) * 131072u + (((uint32_t)ka >> 6) & 3u) * 4096u;
    dma16_branch(op.desc, vlane + (sbase + part(i)), tile + mwave + (uint32_t)i * 1024u);
  }
  // rows rc0 + 32 j + lane % 32: token group rc0 / 32 + j; K group g: vocab
  // group half g / 2, chunk 2 (g % 2) + lane / 32
  __device__ __forceinline__ void frag_init(int rc0) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, sw = (r >> 2) & 3;
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      const int c = 2 * (g & 1) + (lane >> 5);
      fbase[g] = (uint32_t)(((g >> 1) * 8 + (rc0 >> 5)) * 2048 + r * 64 + ((c ^ sw) << 4));
    }
  }
  __device__ __forceinline__ void read(Frag<T>& f, const lds_u8* st, int g, int j) const {
    f.v = *(const __attribute__((address_space(3))) u32x4*)(st + fbase[g] + j * 2048);
  }
};

// dC's A = G^T (rows: vocab, K: tokens), read through transposing LDS reads.
// Stage block k = 8 h + v: vocab group v, token group 2 q + h, stored as in
// memory (rows of 64 bytes): the 32 lanes of one ds_read_b64_tr_b16 cycle
// read 4 whole consecutive rows, 256 contiguous bytes (conflict free).
template <class C>
struct DmaBlockMN {
  static_assert(sizeof(typename C::T) == 2 && C::BK == 64 && C::BM == 256, "bf16 256-column tiles, 64-deep steps");
  using T = typename C::T;
  static constexpr int BYTES = 16 * 2048;
  static constexpr int NW = C::NT / 64;
  static constexpr int PER = 32 / NW;
  static constexpr int KG = C::KGROUPS;
  uint32_t fbase[KG];
  uint32_t vlane;  // the lane's 16 bytes plus the wave's first half block
  uint32_t mwave;  // LDS byte offset of the wave's first half block in a stage
  __device__ __forceinline__ void init(const Operand&) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    mwave = (uint32_t)(wave * PER) * 1024u;
    vlane = (uint32_t)lane * 16u + mwave;
  }
  // Half block d of a step (stage block k = d / 2 = 8 h + v: vocab group v,
  // token group 2 q + h) is block 16 q + k of the slot: the step's 32 KB are
  // contiguous, at slot * 131072 + q * 32768, half block d at d * 1024.
  // ka = slot * 256 + 64 q; past the last step slot >= cap: every offset lies
  // past the buffer (zeros).
  __device__ __forceinline__ void issue(int i, const Operand& op, int ka, uint32_t tile) const {
    const uint32_t sbase = ((uint32_t)ka >> 8) * 131072u + (((uint32_t)ka >> 6) & 3u) * 32768u;
    dma16_branch(op.desc, vlane + (sbase + (uint32_t)i * 1024u), tile + mwave + (uint32_t)i * 1024u);
  }  // columns rc0 + 32 j ..: vocab group rc0 / 32 + j.  Within each group of
  // 16 lanes, source lane s addresses K row 8 (lane / 32) + s / 4 of the K
  // group's 16 (plus 4 for the second read) and columns 16 ((lane / 16) % 2)
  // + 4 (s % 4) .. +3 of the block: output lane i then holds column 16
  // ((lane / 16) % 2) + i at those K rows, as in DmaTileMN.
  __device__ __forceinline__ void frag_init(int rc0) {
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, sl = lane & 15;
    const int krow = 8 * (grp >> 1) + (sl >> 2);
    const int col = 16 * (grp & 1) + 4 * (sl & 3);
#pragma unroll
    for (int g = 0; g < KG; ++g)
      fbase[g] = (uint32_t)(((g >> 1) * 8 + (rc0 >> 5)) * 2048 + (16 * (g & 1) + krow) * 64 + col * 2);
  }
  __device__ __forceinline__ void read(Frag<T>& f, const lds_u8* st, int g, int j) const {
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + fbase[g] + j * 2048));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + fbase[g] + j * 2048 + 4 * 64));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    f.v = u32x4{ua[0], ua[1], ub[0], ub[1]};
  }
};

// acc[fm][fn] += sum over the K steps of A_tile * B_tile^T, as mainloop()
// (same step/offset conventions), both operands DMA-fed: K-major (DmaTile),
// or with A_MN / B_MN MN-major (DmaTileMN, 16-bit only).  The A and B
// fragments of the MFMA share one lane layout (lane l: row or column l % 32,
// K elements 8 (l / 32) .. +7), so either tile kind serves either operand.
//
// Two LDS stages.  Within a step the MFMAs of K group g run while the
// fragments of group g+1 are read.  Before the last group each wave waits for
// its DMA loads of the next step and joins one barrier: after it the next
// stage is complete and the current one is free.  A stage is therefore free
// for one step between its last read and the first read of its next contents;
// its DMA loads (which the memory pipeline delivers at about 64 bytes per
// clock per CU, so a step's 64 KB needs about half a step) are issued in
// NPARTS parts over that window: part 0 right after the barrier, in the last
// group, and part p in group p-1 of the following step, each spread about two
// instructions per MFMA over the first half of its group so the issue never
// stalls the matrix core.
// Steps past the end (the count is padded to even) read zeros.
// MFMA block mask of a K step (see mainloop_dma): all blocks on.
struct NoMask {
  static constexpr bool kActive = false;
  __device__ __forceinline__ uint32_t operator()(int) const { return 0xffffffffu; }
};
// MaskT::kSkipA (a block-layout A tile): mask.raw(f) is an LDS read of the
// 64-bit word behind step f's bits and MaskT::dma_bits(lo, hi, f), from its
// two (wave-uniform) halves, the step's sixteen A-stage blocks, bit k for
// stage block k (half blocks 2 k, 2 k + 1).
template <class M, class = void>
struct SkipA : std::false_type {};
template <class M>
struct SkipA<M, std::void_t<decltype(M::kSkipA)>> : std::bool_constant<M::kSkipA> {};

//
// With `ablocks` (SEPA), the A operand takes its own K blocks: step s reads A
// at K offset ablocks[s / SPB] * astride + (s % SPB) * BK (the gradient
// tiles stored one per slot), B as above.
//
// With ATile (a DmaBlockK / DmaBlockMN), A is read from the block layout of
// the compact gradient tiles.
//
// With `steps`, only the listed steps run: steps[s] is the index, in the
// full sequence above, of the s-th step of the loop (ascending; nsteps
// listed), so K offsets, block lists and masks follow it (the steps whose
// blocks are all zero are left out).
template <class C, int SPB, bool B_MN = false, bool A_MN = false, int NPARTS = (C::KGROUPS > 2 ? 3 : 1),
          class MaskT = NoMask, bool SEPA = false, class ATile = void, bool STEPS = false, bool BKFULL = false>
__device__ __forceinline__ void mainloop_dma(f32x16 (&acc)[C::FM][C::FN], const Operand& A, const Operand& B,
                                             int nsteps, const uint16_t* blocks, void* smem,
                                             const int* __restrict__ brow = nullptr, const MaskT& mask = MaskT{},
                                             const uint16_t* ablocks = nullptr, int astride = 0,
                                             const uint16_t* steps = nullptr) {
  using T = typename C::T;
  using TA = std::conditional_t<!std::is_void_v<ATile>, ATile,
                                std::conditional_t<A_MN, DmaTileMN<C, C::BM, C::FM>, DmaTile<C, C::BM>>>;

  using TB = std::conditional_t<B_MN, DmaTileMN<C, C::BN, C::FN>, DmaTile<C, C::BN, BKFULL>>;
  constexpr int KG = C::KGROUPS;
  static_assert(KG % 2 == 0, "fragment buffers alternate per K group");
  static_assert(NPARTS >= 1 && NPARTS < KG, "the last DMA part must precede the wait");
  constexpr int STAGE = TA::BYTES + TB::BYTES;
  static_assert(2 * STAGE == C::LDS_DMA_BYTES, "stage size");
  if (nsteps <= 0) return;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int kend = A.kdim > B.kdim ? A.kdim : B.kdim;
  // Index of step s in the full sequence (clamped to the last step), and
  // K offsets of step s from it; steps past the end read zeros (offset kend).
  // The loop reads step s + 3's index one step ahead of its offsets, so no
  // LDS read waits on another.
  auto full = [&](int s) -> int {
    if constexpr (STEPS) return (int)steps[s < nsteps ? s : nsteps - 1];
    else return s;
  };
  // block-list index of full step f, kept inside the list
  const int last_blk = STEPS ? 0 : (nsteps - 1) / SPB;
  auto blk = [&](int f) -> int {
    if constexpr (STEPS) return f / SPB;
    else return f / SPB < last_blk ? f / SPB : last_blk;
  };
  auto kofs_f = [&](int s, int f) -> int {
    const int k = blocks ? (int)blocks[blk(f)] * (SPB * C::BK) + (f % SPB) * C::BK : f * C::BK;
    return s < nsteps ? k : kend;
  };
  // A's K offset: the same, or from its own block list
  auto kofs_a_f = [&](int s, int f) -> int {
    if constexpr (SEPA) return s < nsteps ? (int)ablocks[blk(f)] * astride + (f % SPB) * C::BK : kend;
    else return kofs_f(s, f);
  };
  auto kofs = [&](int s) -> int { return kofs_f(s, full(s)); };
  auto kofs_a = [&](int s) -> int { return kofs_a_f(s, full(s)); };
  const lds_u8* base = (const lds_u8*)smem;
  const uint32_t base_addr = (uint32_t)(uintptr_t)base;

  constexpr int NDMA = TA::PER + TB::PER;  // DMA instructions per wave per step
  TA ta;
  TB tb;
  ta.init(A);
  // B rows through `brow` (K-major B only): the gathered token rows
  if constexpr (B_MN) tb.init(B);
  else tb.init(B, brow);
  // With kSkipA, the A loads of a stage block whose bit is clear (an all-zero
  // 32x32 block of the gradient, whose MFMAs the mask skips) are not issued
  // at all: no request, no LDS write; the stage keeps stale bytes there,
  // which no MFMA reads.  Steps past the end load every block (zeros).  The
  // wave issues half blocks wave * PER .. + PER - 1, i.e. stage blocks from
  // wave * PER / 2 on: wb = the step's bits shifted by that.
  constexpr bool kSkipA = SkipA<MaskT>::value;
  static_assert(!kSkipA || TA::PER % 2 == 0, "whole blocks per wave");
  const int wsh = kSkipA ? __builtin_amdgcn_readfirstlane(wave) * (TA::PER / 2) : 0;
  // The A blocks to load for step s (full index f), from the mask word
  // `raw` (read from LDS into vector registers): made wave-uniform, then
  // decoded; every block for a step past the end
  auto uniform_bits = [&](int s, int f, uint64_t raw) -> uint32_t {
    if constexpr (kSkipA) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)raw);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(raw >> 32));
      return s < nsteps ? MaskT::dma_bits(lo, hi, __builtin_amdgcn_readfirstlane(f)) : 0xffffffffu;
    } else {
      return 0xffffffffu;
    }
  };
  // the mask word of full step f (without a step list, an index past the
  // end reads the last word, whose bits are then not used)
  auto raw_at = [&](int f) -> uint64_t {
    if constexpr (kSkipA) return mask.raw(f < nsteps || STEPS ? f : nsteps - 1);
    else return 0;
  };
  // ka: A's K offset, kb: B's (the same without SEPA); wb: the A blocks to load
  auto dma = [&](int d, int ka, int kb, uint32_t st, uint32_t wb) {
    if (d < TA::PER) {
      if (!kSkipA || ((wb >> (d >> 1)) & 1u)) ta.issue(d, A, ka, st);
    } else {
      tb.issue(d - TA::PER, B, kb, st + TA::BYTES);
    }
  };
  // prologue: step 0 whole, part 0 of step 1 (its other parts follow in step 0)
  constexpr int P0 = NDMA / NPARTS;
  const uint32_t wb0 = uniform_bits(0, full(0), raw_at(full(0))) >> wsh;
  uint32_t db1 = uniform_bits(1, full(1), raw_at(full(1)));
#pragma unroll
  for (int d = 0; d < NDMA; ++d) dma(d, kofs_a(0), kofs(0), base_addr, wb0);
#pragma unroll
  for (int d = 0; d < P0; ++d) dma(d, kofs_a(1), kofs(1), base_addr + STAGE, db1 >> wsh);
  // step 0 has landed (with kSkipA the number of step 1's loads in flight
  // varies, so all are awaited)
  if constexpr (kSkipA) wait_vmcnt<0>();
  else wait_vmcnt<P0>();
  __syncthreads();

  ta.frag_init(wm * C::WM);
  tb.frag_init(wn * C::WN);
  Frag<T> fa[2][C::FM], fb[2][C::FN];
  auto read_one = [&](int buf, const lds_u8* st, int g, int q) {
    if (q < C::FM) ta.read(fa[buf][q], st, g, q);
    else tb.read(fb[buf][q - C::FM], st + TA::BYTES, g, q - C::FM);
  };
#pragma unroll
  for (int q = 0; q < C::FM + C::FN; ++q) read_one(0, base, 0, q);
  // With a block mask (MaskT::kActive), mask(s) gives step s's bit
  // h * FM + fm: the A rows of fragment fm times the K half h (K groups 2h,
  // 2h + 1) hold nonzero values.  The MFMAs of a zero block are skipped (they
  // would add exact zeros).  The bits of step s + 1 are read at the top of
  // step s (LDS, after the first barrier has published them).
  uint32_t mcur =
      MaskT::kActive ? (uint32_t)__builtin_amdgcn_readfirstlane((int)mask(STEPS ? full(0) : 0)) : 0xffffffffu;

  constexpr int NFR = C::FM + C::FN;
  constexpr int BLOCKS = C::FM * C::FN;

  // k1 = kofs(s + 1) comes from the previous step; kofs(s + 2), first needed
  // after the barrier, is read (from the LDS block list when there is one) at
  // the top of the step, ahead of the step's fragment reads, so the waits for
  // those cover it and the loop never waits on that read alone.
  // (With SEPA, A's offsets ka1 / ka2 likewise.)
  int kan = SEPA ? __builtin_amdgcn_readfirstlane(kofs_a(1)) : 0;
  // (with a step list) full indices of steps s + 1 and s + 2, carried from
  // step to step
  int fn1 = STEPS ? __builtin_amdgcn_readfirstlane(full(1)) : 0;
  int fn2 = STEPS ? __builtin_amdgcn_readfirstlane(full(2)) : 0;
  auto step = [&](int s, const lds_u8* st, const lds_u8* nx, uint32_t st_addr, uint32_t nx_addr, int k1) -> int {
    // wave-uniform: kept in a scalar register
    const int f1 = STEPS ? fn1 : (s + 1 < nsteps ? s + 1 : nsteps - 1), f2 = STEPS ? fn2 : s + 2;
    const int ka1 = SEPA ? kan : k1;
    // The LDS reads behind the step's later scalars (step s + 3's index, the
    // K offsets of step s + 2, the mask of step s + 1) are issued in the first
    // group, after its fragment wait, and made wave-uniform in the last
    // group, which first needs them: their latency passes under the MFMAs
    // instead of stalling the step.  (The raw list entries only: the
    // arithmetic on them is scalar, after.)
    int f3v = 0, bv = 0, av = 0;
    uint32_t mv = 0;
    int f3 = 0, k2 = 0, ka2 = 0;
    uint32_t mnext = 0xffffffffu;
    uint64_t dv = 0;  // the raw word behind step s + 2's A blocks
    uint32_t db2 = 0xffffffffu;
    auto group = [&](auto gc) {
      constexpr int g = decltype(gc)::value;
      constexpr bool last = g + 1 == KG;
      if constexpr (last) {
        if constexpr (STEPS) f3 = __builtin_amdgcn_readfirstlane(f3v);
        const bool in = s + 2 < nsteps;
        const int sub = (f2 % SPB) * C::BK;
        k2 = !in ? kend : blocks ? __builtin_amdgcn_readfirstlane(bv) * (SPB * C::BK) + sub : f2 * C::BK;
        if constexpr (SEPA) ka2 = in ? __builtin_amdgcn_readfirstlane(av) * astride + sub : kend;
        else ka2 = k2;
        if constexpr (MaskT::kActive) mnext = (uint32_t)__builtin_amdgcn_readfirstlane((int)mv);
        if constexpr (kSkipA) db2 = uniform_bits(s + 2, f2, dv);
        wait_vmcnt<0>();
        __syncthreads();
      }
      // DMA share of this group: part 0 of step s+2 into this stage after the
      // barrier, or part g+1 of step s+1 into the next stage
      constexpr int dp = last ? 0 : g + 1;
      constexpr bool has_dma = last || g + 1 < NPARTS;
      constexpr int dlo = has_dma ? dp * NDMA / NPARTS : 0;
      constexpr int dn = has_dma ? (dp + 1) * NDMA / NPARTS - dlo : 0;
      // With a block mask: the group's fragments (read during the previous
      // group) are awaited once here, so that the MFMAs of each A fragment
      // sit under one scalar branch with no waits of their own.
      if constexpr (MaskT::kActive) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      if constexpr (g == 0) {
        if constexpr (STEPS) f3v = full(s + 3);
        bv = blocks ? (int)blocks[blk(f2)] : 0;
        if constexpr (SEPA) av = (int)ablocks[blk(f2)];
        if constexpr (MaskT::kActive) mv = mask(f1);
        if constexpr (kSkipA) dv = raw_at(f2);
      }
      [&]<int... Q>(std::integer_sequence<int, Q...>) {
        (
            [&] {
              constexpr int b = Q;
              if constexpr (MaskT::kActive) {
                if constexpr (b % C::FN == 0) {
                  if ((mcur >> ((g >> 1) * C::FM + b / C::FN)) & 1u) {
#pragma unroll
                    for (int fn = 0; fn < C::FN; ++fn)
                      mma16(acc[b / C::FN][fn], fa[g & 1][b / C::FN], fb[g & 1][fn]);
                  }
                }
              } else {
                mma16(acc[b / C::FN][b % C::FN], fa[g & 1][b / C::FN], fb[g & 1][b % C::FN]);
              }
              constexpr int r0 = b * NFR / BLOCKS, r1 = (b + 1) * NFR / BLOCKS;
#pragma unroll
              for (int q = r0; q < r1; ++q) {
                if constexpr (last) read_one(0, nx, 0, q);
                else read_one((g + 1) & 1, st, g + 1, q);
              }
              // the part's DMA over the group's first half of MFMAs (about
              // two per MFMA there): the loads start earlier than spread over
              // the whole group (measured 1% faster), while more bunched
              // issue (first quarter) stalls the matrix core (2% slower)
              constexpr int HALF = BLOCKS / 2;
              constexpr int d0 = b * dn / HALF < dn ? b * dn / HALF : dn;
              constexpr int d1 = (b + 1) * dn / HALF < dn ? (b + 1) * dn / HALF : dn;
#pragma unroll
              for (int d = d0; d < d1; ++d) {
                if constexpr (last) dma(dlo + d, ka2, k2, st_addr, db2 >> wsh);
                else dma(dlo + d, ka1, k1, nx_addr, db1 >> wsh);
              }
              __builtin_amdgcn_sched_barrier(0);
            }(),
            ...);
      }(std::make_integer_sequence<int, BLOCKS>{});
    };
    [&]<int... G>(std::integer_sequence<int, G...>) {
      (group(std::integral_constant<int, G>{}), ...);
    }(std::make_integer_sequence<int, KG>{});
    mcur = mnext;
    db1 = db2;
    if constexpr (SEPA) kan = ka2;
    if constexpr (STEPS) {
      fn1 = f2;
      fn2 = f3;
    }
    return k2;
  };

  const lds_u8* st0 = base;
  const lds_u8* st1 = base + STAGE;
  int kn = __builtin_amdgcn_readfirstlane(kofs(1));
  for (int s = 0; s < nsteps; s += 2) {
    kn = step(s, st0, st1, base_addr, base_addr + STAGE, kn);
    kn = step(s + 1, st1, st0, base_addr + STAGE, base_addr, kn);
  }
  wait_vmcnt<0>();  // the trailing loads (zeros past the end) have landed
  __syncthreads();
}

// Output coordinates of accumulator element r of block (fm, fn) for this lane,
// relative to the work-group tile origin.
template <class C>
struct AccMap {
  int row0, col;  // row of r = row0 + fm*32 + 8*(r/4) + (r%4); col + fn*32
  __device__ __forceinline__ AccMap() {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    row0 = wm * C::WM + 4 * (lane >> 5);
    col = wn * C::WN + (lane & 31);
  }
  __device__ __forceinline__ int row(int fm, int r) const { return row0 + fm * 32 + 8 * (r >> 2) + (r & 3); }
  __device__ __forceinline__ int colj(int fn) const { return col + fn * 32; }
};

}  // namespace cce
