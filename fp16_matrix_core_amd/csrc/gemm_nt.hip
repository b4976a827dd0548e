// gemm_nt.hip -- Out = A @ B.T, fp16 operands, fp32 accumulation, on gfx950.
//
// The operation is the one "Warp Matrix Instructions" and "Blackwell Tensor
// Cores" compute (Out = A @ B.T, K accumulated slice by slice into a fresh
// fp32 accumulator).  The data path is the same in spirit -- operand tiles
// staged in shared memory, moved into per-lane register fragments, multiplied
// by wavefront-collective matrix instructions -- laid out for CDNA4:
//
//   global -> LDS   direct loads (buffer_load_dwordx4 ... lds): each lane
//                   moves one 16-byte chunk (8 fp16 of one row) straight into
//                   LDS; a wavefront fills 1 KiB of whole rows per load.
//   LDS layout      a K slice of a row is BK = 32 or 64 fp16, i.e. 64 or 128
//                   bytes = 4 or 8 chunks, placed by the XOR swizzles of
//                   layout.hpp (conflict-free for the direct loads and for
//                   the fragment reads below).  With BK = 64 the 8 lanes of a
//                   row fetch one whole 128-byte line, which halves the L2
//                   requests of BK = 32 (two half-line requests per line).
//   LDS -> VGPR     one ds_read_b128 per lane per operand fragment: the 8
//                   consecutive-K fp16 that v_mfma_f32_32x32x16_f16 takes
//                   from each lane.  Both operands are K-contiguous (NT), so
//                   no transpose is needed.
//   MFMA            A's fragment is the instruction's first operand, B's
//                   the second, so in each accumulator register the 32
//                   lanes of a half-wavefront hold 32 consecutive columns of
//                   one output row: a dword store per register writes two
//                   whole 128-byte row segments.
//   K loop          a ring of LDS stages; each slice's loads are issued
//                   STAGES-1 slices ahead, spread between MFMAs, and the
//                   fragments of the next K step are read while the current
//                   one multiplies; one workgroup barrier per slice.
//   scheduler       XCD-contiguous ranges of tile ids, grouped so that the
//                   tiles an XCD runs together share A and B panels in L2.
//   edges           rows past M or N are clamped on load (their results are
//                   never stored); K past the end is zero-filled; the
//                   epilogue masks columns past N and rows past M.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "kernels.hpp"
#include "layout.hpp"

namespace fp16mc {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Operand element types.  Both move through the kernels as raw 16-bit
// patterns; only the matrix instruction that consumes them differs.
struct InF16 {
  typedef f16x8 V8;
  static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
struct InBF16 {
  typedef bf16x8 V8;
  static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// One output element: the fp32 sum, plus the element's previous value when
// accumulating, stored as fp32 or rounded to nearest-even fp16 / bf16.
template <class OutT, bool ACC>
__device__ __forceinline__ void store_out(OutT* p, float v) {
  if constexpr (ACC) v += static_cast<float>(*p);
  *p = static_cast<OutT>(v);
}

// BM x BN output tile per workgroup, WM x WN wavefronts, each owning a
// (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles.  K advances in slices
// of BK (32 or 64) held in a ring of STAGES LDS stages; WAVES_PER_SIMD
// workgroups' worth of wavefronts share each SIMD (the register budget
// follows from it).
template <int BM_, int BN_, int WM_, int WN_, int GROUP_M_, int STAGES_, int WAVES_PER_SIMD_, int BK_ = 32>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, GROUP_M = GROUP_M_;
  static constexpr int BK = BK_;
  using Swz = LdsSwizzle<2 * BK_>;
  static constexpr int STAGES = STAGES_;
  static constexpr int WAVES_PER_SIMD = WAVES_PER_SIMD_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int SI = WTM / 32, SJ = WTN / 32;
  static constexpr int A_STAGE = BM * Swz::kRowBytes;
  static constexpr int B_STAGE = BN * Swz::kRowBytes;
  static constexpr int ROWS_PER_WAVE = 1024 / Swz::kRowBytes;     // one 1 KiB direct load
  static constexpr int ROWS_PER_PASS = (NT / 64) * ROWS_PER_WAVE;
  static constexpr int A_LOADS = BM / ROWS_PER_PASS;
  static constexpr int B_LOADS = BN / ROWS_PER_PASS;
  static constexpr int LDS_BYTES = STAGES * (A_STAGE + B_STAGE);
  static_assert(BK == 32 || BK == 64, "an LDS row holds one 32- or 64-wide K slice");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "rows must split evenly");
  static_assert(STAGES >= 2 && STAGES <= 4, "two to four LDS stages");
  static constexpr int WGS_PER_CU = WAVES_PER_SIMD * 256 / NT > 0 ? WAVES_PER_SIMD * 256 / NT : 1;
  static_assert(LDS_BYTES * WGS_PER_CU <= 160 * 1024, "gfx950 LDS is 160 KiB per CU");
};

using CfgWave32 = Cfg<32, 32, 1, 1, 1, 4, 1>;
// 128x64 tiles: 64-wide slices in three 24 KiB stages (two workgroups per CU
// by LDS); measured 28% faster at 2048^3 than 32-wide slices in four stages.
using CfgWg128x64 = Cfg<128, 64, 4, 1, 8, 3, 1, 64>;
// 256x256 tiles: 64-wide slices in two 64 KiB stages (three do not fit in
// 160 KiB); measured 6-7% faster at 8192^3 than 32-wide slices in four stages.
using CfgWg256 = Cfg<256, 256, 2, 2, 4, 2, 1, 64>;

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// Elements [k, k+8) of a row, zero past K.  `row` points at element 0.
// Only the last, partial K slice of a problem takes this path.
__device__ __forceinline__ u32x4 load_chunk_masked(const unsigned short* row, int64_t k, int64_t K) {
  const unsigned short* r16 = row;
  unsigned int w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (k + e < K) w[e >> 1] |= static_cast<unsigned int>(r16[k + e]) << (16 * (e & 1));
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds):
// lane l's bytes land at lds_span + 16 l; `lds_span` and `soff` are uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, unsigned char* lds_span, unsigned voff,
                                      unsigned soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_span, 16, voff, soff, 0, 0);
}

// Buffer descriptor over [base, base + bytes).  Both values are workgroup-
// uniform; passing them through readfirstlane lets the compiler keep the
// descriptor in SGPRs instead of re-checking uniformity at every load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// Scheduling hints: keep `n` instructions of one kind together at this point.
#define SCHED_MFMA(n) __builtin_amdgcn_sched_group_barrier(0x008, (n), 0)
#define SCHED_VMEM_READ(n) __builtin_amdgcn_sched_group_barrier(0x020, (n), 0)
#define SCHED_DS_READ(n) __builtin_amdgcn_sched_group_barrier(0x100, (n), 0)
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Compile-time loop: f(std::integral_constant<int, i>) for i in [0, N).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// How many of `total` instructions go after the n-th of k MFMAs for an even spread.
constexpr int spread(int n, int total, int k) { return (n + 1) * total / k - n * total / k; }

// s_waitcnt immediate for "vmcnt(n)" with the other counters left alone (gfx9 encoding).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <class C, class In, class OutT, bool ACC>
__global__ void __launch_bounds__(C::NT, C::WAVES_PER_SIMD)
gemm_nt_kernel(const unsigned short* __restrict__ A, const unsigned short* __restrict__ B, OutT* __restrict__ Out,
               int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldo,
               int64_t sA, int64_t sB, int64_t sO, int64_t tiles_m, int64_t tiles_n, int64_t total) {
  // One array per (operand, stage): the compiler then knows that the
  // asynchronous LDS writes into one stage never alias reads of another.
  constexpr int kS = C::STAGES;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_a0[C::A_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_a1[C::A_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_a2[kS > 2 ? C::A_STAGE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_a3[kS > 3 ? C::A_STAGE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_b0[C::B_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_b1[C::B_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_b2[kS > 2 ? C::B_STAGE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_b3[kS > 3 ? C::B_STAGE : 16];
  auto stage_a = [&](auto st) -> unsigned char* {
    constexpr int S = decltype(st)::value % kS;
    return S == 0 ? lds_a0 : S == 1 ? lds_a1 : S == 2 ? lds_a2 : lds_a3;
  };
  auto stage_b = [&](auto st) -> unsigned char* {
    constexpr int S = decltype(st)::value % kS;
    return S == 0 ? lds_b0 : S == 1 ? lds_b1 : S == 2 ? lds_b2 : lds_b3;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WN;
  const int wn = wave % C::WN;

  // ---- tile scheduler -------------------------------------------------------
  const uint32_t lin = sched::xcd_remap(blockIdx.x, static_cast<uint32_t>(total));
  const uint32_t per_problem = static_cast<uint32_t>(tiles_m * tiles_n);
  const uint32_t b = lin / per_problem;
  const sched::Tile tile = sched::grouped_tile(lin - b * per_problem, static_cast<uint32_t>(tiles_m),
                                               static_cast<uint32_t>(tiles_n), C::GROUP_M);
  const int64_t i0 = static_cast<int64_t>(tile.m) * C::BM;
  const int64_t j0 = static_cast<int64_t>(tile.n) * C::BN;
  A += b * sA;
  B += b * sB;
  Out += b * sO;

  // ---- global -> LDS assignment ------------------------------------------------
  // Pass p of wavefront w fills LDS rows [p*ROWS_PER_PASS + 16w, +16): lane l
  // lands at byte 16 l of that 1 KiB span, i.e. row +l/4, physical chunk l%4,
  // so it fetches the logical chunk that the swizzle places there.  Rows past
  // the matrix edge re-read its last row (their results are never stored).
  // Addresses are byte offsets inside a buffer that starts at the tile's first
  // row: a per-lane VGPR offset plus a uniform K offset.
  constexpr int RW = C::ROWS_PER_WAVE;
  const int prow = lane / C::Swz::kChunks;
  const int pchunk = lane % C::Swz::kChunks;
  const int64_t a_rows = (M - i0) < C::BM ? (M - i0) : C::BM;
  const int64_t b_rows = (N - j0) < C::BN ? (N - j0) : C::BN;
  const unsigned short* a_tile = A + i0 * lda;
  const unsigned short* b_tile = B + j0 * ldb;
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(a_tile, static_cast<unsigned>(2 * ((a_rows - 1) * lda + K)));
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(b_tile, static_cast<unsigned>(2 * ((b_rows - 1) * ldb + K)));
  unsigned a_off[C::A_LOADS];
  unsigned b_off[C::B_LOADS];
#pragma unroll
  for (int p = 0; p < C::A_LOADS; ++p) {
    const int r = p * C::ROWS_PER_PASS + RW * wave + prow;
    const int64_t rr = r < a_rows ? r : a_rows - 1;
    a_off[p] = static_cast<unsigned>(2 * (rr * lda + 8 * C::Swz::logical_chunk(r, pchunk)));
  }
#pragma unroll
  for (int p = 0; p < C::B_LOADS; ++p) {
    const int r = p * C::ROWS_PER_PASS + RW * wave + prow;
    const int64_t rr = r < b_rows ? r : b_rows - 1;
    b_off[p] = static_cast<unsigned>(2 * (rr * ldb + 8 * C::Swz::logical_chunk(r, pchunk)));
  }
  auto span = [&](int p) { return (p * C::ROWS_PER_PASS + RW * wave) * C::Swz::kRowBytes; };
  constexpr int kLoads = C::A_LOADS + C::B_LOADS;   // direct loads per slice per wavefront
  // Load number q of a full slice (A passes first, then B passes).
  auto dma = [&](unsigned char* as, unsigned char* bs, int q, unsigned koff) {
    if (q < C::A_LOADS) dma16(a_rsrc, as + span(q), a_off[q], koff);
    else dma16(b_rsrc, bs + span(q - C::A_LOADS), b_off[q - C::A_LOADS], koff);
  };
  auto dma_all = [&](unsigned char* as, unsigned char* bs, unsigned koff) {
#pragma unroll
    for (int q = 0; q < kLoads; ++q) dma(as, bs, q, koff);
  };
  // Last, partial K slice: through registers with per-element masks.
  auto load_tail = [&](unsigned char* as, unsigned char* bs, int64_t k0) {
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) {
      const int lc = C::Swz::logical_chunk(p * C::ROWS_PER_PASS + RW * wave + prow, pchunk);
      const unsigned short* row = a_tile + a_off[p] / 2 - 8 * lc;
      *reinterpret_cast<u32x4*>(as + span(p) + 16 * lane) = load_chunk_masked(row, k0 + 8 * lc, K);
    }
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) {
      const int lc = C::Swz::logical_chunk(p * C::ROWS_PER_PASS + RW * wave + prow, pchunk);
      const unsigned short* row = b_tile + b_off[p] / 2 - 8 * lc;
      *reinterpret_cast<u32x4*>(bs + span(p) + 16 * lane) = load_chunk_masked(row, k0 + 8 * lc, K);
    }
  };

  // ---- fragment reads + MFMA ------------------------------------------------
  f32x16 acc[C::SI][C::SJ];
#pragma unroll
  for (int si = 0; si < C::SI; ++si)
#pragma unroll
    for (int sj = 0; sj < C::SJ; ++sj) acc[si][sj] = f32x16{};

  const int frow = mfma32::operand_row(lane);      // row inside a 32-row MFMA tile
  const int khalf = lane >> 5;                     // which 8-wide K group of a 16-K step
  const int key = C::Swz::key(frow);          // equal to key(row) for every fragment row
  const int a_row0 = (wm * C::WTM + frow) * C::Swz::kRowBytes;
  const int b_row0 = (wn * C::WTN + frow) * C::Swz::kRowBytes;
  constexpr int KK = C::BK / mfma32::kK;           // 16-wide K steps per slice (2 or 4)
  constexpr int NMF = C::SI * C::SJ;               // MFMAs per K step
  constexpr int kFr = C::SI + C::SJ;               // fragment reads per K step
  static_assert(KK % 2 == 0, "fragments alternate between two register sets");

  struct Frags {
    typename In::V8 a[C::SI];
    typename In::V8 b[C::SJ];
  };
  auto read_frags = [&](const unsigned char* as, const unsigned char* bs, int kk, Frags& f) {
    const int pc = ((2 * kk + khalf) ^ key) << 4;
#pragma unroll
    for (int si = 0; si < C::SI; ++si)
      f.a[si] = *reinterpret_cast<const typename In::V8*>(as + a_row0 + si * 32 * C::Swz::kRowBytes + pc);
#pragma unroll
    for (int sj = 0; sj < C::SJ; ++sj)
      f.b[sj] = *reinterpret_cast<const typename In::V8*>(bs + b_row0 + sj * 32 * C::Swz::kRowBytes + pc);
  };
  auto mfma = [&](const Frags& f, int n) {
    const int si = n / C::SJ, sj = n % C::SJ;
    acc[si][sj] = In::mfma32(f.a[si], f.b[sj], acc[si][sj]);
  };
  auto mfma_all = [&](const Frags& f) {
#pragma unroll
    for (int n = 0; n < NMF; ++n) mfma(f, n);
  };
  // Wait until at most `n` direct loads of this thread are in flight and its
  // LDS reads/writes are done, then make everyone's writes visible.
  // (A plain s_barrier: a fenced __syncthreads would also wait for the loads
  // that are meant to stay in flight.)
  auto publish_keep = [&](auto n) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(decltype(n)::value) & ~(15 << 8));  // lgkmcnt(0) as well
    asm volatile("s_barrier" ::: "memory");
  };

  // ---- K loop --------------------------------------------------------------------
  // Full slice s lives in stage s % S of an S-stage ring.  Slices s+1 ..
  // s+S-2 are already in flight when phase s begins; phase s issues slice
  // s+S-1 into the stage of slice s-1, whose reads all completed before the
  // barrier that opened the phase.  In phase s a wavefront
  //   1. reads the fragments of K step (s, 0);
  //   2. issues the MFMAs of step (s-1, KK-1), read before the barrier;
  //   3. for kk = 1 .. KK-1 issues the MFMAs of step (s, kk-1) with the
  //      fragment reads of step (s, kk) spread between them;
  //   4. waits until slice s+1 has landed (only the S-2 later slices may
  //      still be in flight) and its own fragment reads are done; barrier.
  // Slice s+S-1's loads are spread over the MFMAs of the first two steps of
  // 2 and 3, so that they leave early in the phase.  The MFMA pipe restarts
  // after each barrier on registers that are already loaded.
  constexpr int kAhead = kS - 1;                   // prefetch distance in slices
  const int64_t nfull = K / C::BK;
  Frags f0, f1;
  auto koff_of = [&](int64_t slice) {
    // slices past the end reload the last one into an idle stage: no branch, never read
    return static_cast<unsigned>(2 * C::BK * (slice < nfull ? slice : nfull - 1));
  };
  std::integral_constant<int, (kAhead - 1) * kLoads> keep_later;
  constexpr int kLoadSteps = 2;                    // MFMA steps the slice loads are spread over
  auto phase = [&](auto st, int64_t s, auto pending) {
    constexpr int S = decltype(st)::value;
    constexpr bool kPending = decltype(pending)::value;
    unsigned char* as = stage_a(st);
    unsigned char* bs = stage_b(st);
    unsigned char* an = stage_a(std::integral_constant<int, S + kAhead>{});
    unsigned char* bn = stage_b(std::integral_constant<int, S + kAhead>{});
    const unsigned koff = koff_of(s + kAhead);
    read_frags(as, bs, 0, f0);
    if constexpr (kPending) mfma_all(f1);
    dma_all(an, bn, koff);
    static_for<KK - 1>([&](auto t) {
      constexpr int kk = decltype(t)::value + 1;
      if constexpr (kk % 2 == 1) {
        read_frags(as, bs, kk, f1);
        mfma_all(f0);
      } else {
        read_frags(as, bs, kk, f0);
        mfma_all(f1);
      }
    });
    // Issue order for the scheduler: each step's fragment reads spread between
    // the previous step's MFMAs, the slice loads between the first two steps'.
    SCHED_DS_READ(kFr);
    constexpr int v0 = spread(0, kLoads, kLoadSteps);
    if constexpr (kPending) {
      static_for<NMF>([&](auto n) {
        constexpr int v = spread(decltype(n)::value, v0, NMF);
        SCHED_MFMA(1);
        if constexpr (v > 0) SCHED_VMEM_READ(v);
      });
    } else {
      SCHED_VMEM_READ(v0);
    }
    static_for<KK - 1>([&](auto t) {
      constexpr int g = decltype(t)::value + 1;
      constexpr int vg = g < kLoadSteps ? spread(g, kLoads, kLoadSteps) : 0;
      static_for<NMF>([&](auto n) {
        constexpr int d = spread(decltype(n)::value, kFr, NMF);
        constexpr int v = spread(decltype(n)::value, vg, NMF);
        SCHED_MFMA(1);
        if constexpr (d > 0) SCHED_DS_READ(d);
        if constexpr (v > 0) SCHED_VMEM_READ(v);
      });
    });
    publish_keep(keep_later);
  };
  std::integral_constant<bool, true> with_pending;
  std::integral_constant<bool, false> first;
  if (nfull > 0 && nfull <= kAhead) {
    // Short K: every full slice fits in the ring at once -- load them all,
    // one barrier, multiply.
    static_for<kAhead>([&](auto i) {
      if (decltype(i)::value < nfull) dma_all(stage_a(i), stage_b(i), koff_of(decltype(i)::value));
    });
    publish_keep(std::integral_constant<int, 0>{});
    static_for<kAhead>([&](auto i) {
      if (decltype(i)::value < nfull) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          read_frags(stage_a(i), stage_b(i), kk, f0);
          mfma_all(f0);
        }
      }
    });
  } else if (nfull > 0) {
    static_for<kAhead>([&](auto i) { dma_all(stage_a(i), stage_b(i), koff_of(decltype(i)::value)); });
    publish_keep(keep_later);
    phase(std::integral_constant<int, 0>{}, 0, first);
    int64_t s = 1;
    for (; s + kS <= nfull; s += kS) {
      static_for<kS>([&](auto i) {
        phase(std::integral_constant<int, (decltype(i)::value + 1) % kS>{}, s + decltype(i)::value, with_pending);
      });
    }
    static_for<kS - 1>([&](auto i) {
      if (s < nfull) {
        phase(std::integral_constant<int, (decltype(i)::value + 1) % kS>{}, s, with_pending);
        ++s;
      }
    });
    mfma_all(f1);  // step (nfull-1, KK-1)
    // drain the idle reloads before any stage is reused or the workgroup ends
    publish_keep(std::integral_constant<int, 0>{});
  }
  // The partial slice, if any, goes through registers into stage nfull % S
  // (unused by the short path, idle after the pipelined one).
  if (K % C::BK != 0) {
    const int st = static_cast<int>(nfull % kS);
    unsigned char* as = lds_a0;
    unsigned char* bs = lds_b0;
    static_for<kS>([&](auto i) {
      if (st == decltype(i)::value) {
        as = stage_a(i);
        bs = stage_b(i);
      }
    });
    load_tail(as, bs, nfull * C::BK);
    publish_keep(std::integral_constant<int, 0>{});
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      read_frags(as, bs, kk, f0);
      mfma_all(f0);
    }
  }

  // ---- epilogue: element v of lane l in tile (si, sj) is Out[i][j] with
  // i = i0 + wm*WTM + 32 si + 8(v/4) + 4(l/32) + v%4, j = j0 + wn*WTN + 32 sj + l%32:
  // one dword store per v writes two whole 128-byte row segments.  When
  // accumulating, a row block's previous values are all loaded before any of
  // its stores (ldo is a run-time value, so the compiler cannot prove that a
  // store does not alias a later load and would otherwise wait on each load).
#pragma unroll
  for (int si = 0; si < C::SI; ++si) {
    float prev[C::SJ][16];
    if constexpr (ACC) {
#pragma unroll
      for (int sj = 0; sj < C::SJ; ++sj) {
        const int64_t j = j0 + wn * C::WTN + sj * 32 + mfma32::acc_col(lane, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t i = i0 + wm * C::WTM + si * 32 + mfma32::acc_row(lane, v);
          prev[sj][v] = (i < M && j < N) ? static_cast<float>(Out[i * ldo + j]) : 0.0f;
        }
      }
    }
#pragma unroll
    for (int sj = 0; sj < C::SJ; ++sj) {
      const int64_t j = j0 + wn * C::WTN + sj * 32 + mfma32::acc_col(lane, 0);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + wm * C::WTM + si * 32 + mfma32::acc_row(lane, v);
        const float val = ACC ? acc[si][sj][v] + prev[sj][v] : acc[si][sj][v];
        if (i < M && j < N) Out[i * ldo + j] = static_cast<OutT>(val);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny products (N <= 16): Out (M x N) = A (M x K) @ B (N x K)^T.
// The work is a stream over A (each element used once), so A bypasses LDS:
// every lane loads four 16-byte chunks of one row per 128-wide K block (the
// four lanes of a row cover its 256 bytes), and B -- padded with zero
// columns to 16 -- is loaded in the same K order, which is all the MFMA
// needs (any K order gives the same sum as long as both operands agree).
// v_mfma_f32_16x16x32_f16: lane l supplies row/column l%16 and 8 fp16 of K;
// here lane (r = l%16, q = l/16) of MFMA step j uses K elements
// kb + 32j + 8q .. +8 of its row, so each load instruction covers 64
// contiguous bytes of 16 rows (a quarter-line per lane scattered over 256
// bytes measured 29% slower).  The last, partial block uses K elements
// kb + 32q + 8j instead (any order works while A and B agree).  Eight
// wavefronts split K; their partial 64 x 16 results are summed through LDS.
// ---------------------------------------------------------------------------
constexpr int kSkRows = 64;        // output rows per workgroup (4 MFMA row tiles)
constexpr int kSkWaves = 8;        // wavefronts splitting K
constexpr int kSkBlock = 128;      // K per block per wavefront

// Four 16-byte chunks of a row at elements k + 32 j (all inside K).  With
// k = kb + 8q the four lanes of a row read 64 contiguous bytes per load.
__device__ __forceinline__ void sk_load(const unsigned short* row, int64_t k, u32x4 (&v)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const u32x4*>(row + k + 32 * j);
}
// The same with zeros past K (the last, partial block only).
__device__ __forceinline__ void sk_load_masked(const unsigned short* row, int64_t k, int64_t K, u32x4 (&v)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = load_chunk_masked(row, k + 8 * j, K);
}

template <class In, class OutT, bool ACC>
__global__ void __launch_bounds__(kSkWaves * 64, 1)
gemm_nt_skinny_kernel(const unsigned short* __restrict__ A, const unsigned short* __restrict__ B,
                      OutT* __restrict__ Out,
                      int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldo,
                      int64_t sA, int64_t sB, int64_t sO, int64_t tiles_m) {
  __shared__ float red[kSkWaves][kSkRows][16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t b = blockIdx.x / static_cast<uint32_t>(tiles_m);
  const int64_t i0 = static_cast<int64_t>(blockIdx.x - b * static_cast<uint32_t>(tiles_m)) * kSkRows;
  A += b * sA;
  B += b * sB;
  Out += b * sO;

  const int r = mfma16::operand_row(lane);   // row in a 16-row tile / column of B
  const int q = lane >> 4;                   // 32-element quarter of the block
  const unsigned short* arow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t i = i0 + 16 * t + r;
    arow[t] = A + (i < M ? i : M - 1) * lda;
  }
  // lanes past N read row N-1 (in bounds) and zero it: no divergent branch
  const bool has_b = r < N;
  const unsigned short* brow = B + (has_b ? r : N - 1) * ldb;
  const unsigned bmask = has_b ? 0xFFFFFFFFu : 0u;

  // Full 128-wide K blocks are split evenly over the wavefronts; the last,
  // partial block (if any) goes to the last wavefront with masked loads.
  const int64_t nfull = K / kSkBlock;
  const int64_t per = (nfull + kSkWaves - 1) / kSkWaves;
  const int64_t blk0 = wave * per < nfull ? wave * per : nfull;
  const int64_t blk1 = (blk0 + per < nfull) ? blk0 + per : nfull;

  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{};
  u32x4 va[2][4][4];
  u32x4 vb[2][4];
  auto load = [&](int buf, int64_t blk) {
    const int64_t k = blk * kSkBlock + 8 * q;
#pragma unroll
    for (int t = 0; t < 4; ++t) sk_load(arow[t], k, va[buf][t]);
    sk_load(brow, k, vb[buf]);
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const typename In::V8 bj = __builtin_bit_cast(typename In::V8, vb[buf][j] & bmask);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = In::mfma16(__builtin_bit_cast(typename In::V8, va[buf][t][j]), bj, acc[t]);
    }
  };
  if (blk0 < blk1) {
    load(0, blk0);
    int64_t blk = blk0;
    for (; blk + 2 < blk1; blk += 2) {  // blocks blk+1 and blk+2 exist: no branch in the body
      load(1, blk + 1);
      mma(0);
      load(0, blk + 2);
      mma(1);
    }
    if (blk + 1 < blk1) {
      load(1, blk + 1);
      mma(0);
      mma(1);
    } else {
      mma(0);
    }
  }
  if (K % kSkBlock != 0 && wave == kSkWaves - 1) {
    const int64_t k = nfull * kSkBlock + 32 * q;
#pragma unroll
    for (int t = 0; t < 4; ++t) sk_load_masked(arow[t], k, K, va[0][t]);
    sk_load_masked(brow, k, K, vb[0]);
    mma(0);
  }

  // partial sums -> LDS: element v of lane l in row tile t is (row 16t + 4(l/16) + v, column l%16)
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][16 * t + mfma16::acc_row(lane, v)][mfma16::acc_col(lane, v)] = acc[t][v];
  __syncthreads();
  for (int e = threadIdx.x; e < kSkRows * 16; e += kSkWaves * 64) {
    const int row = e / 16, col = e % 16;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) sum += red[w][row][col];
    const int64_t i = i0 + row;
    if (i < M && col < N) store_out<OutT, ACC>(Out + i * ldo + col, sum);
  }
}

template <class C>
int64_t tiles_of(int64_t M, int64_t N, int64_t batch, int64_t* tm, int64_t* tn) {
  *tm = (M + C::BM - 1) / C::BM;
  *tn = (N + C::BN - 1) / C::BN;
  return *tm * *tn * batch;
}

template <class C, class In, class OutT, bool ACC>
hipError_t launch(const GemmProblem& p, hipStream_t stream) {
  int64_t tm, tn;
  const int64_t total = tiles_of<C>(p.M, p.N, p.batch, &tm, &tn);
  const unsigned short* A = static_cast<const unsigned short*>(p.A);
  const unsigned short* B = static_cast<const unsigned short*>(p.B);
  OutT* Out = static_cast<OutT*>(p.Out);
  int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb, ldo = p.ldo;
  int64_t sA = p.sA, sB = p.sB, sO = p.sO;
  void* args[] = {&A, &B, &Out, &M, &N, &K, &lda, &ldb, &ldo, &sA, &sB, &sO, &tm, &tn,
                  const_cast<int64_t*>(&total)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_nt_kernel<C, In, OutT, ACC>),
                         dim3(static_cast<unsigned>(total)), dim3(C::NT), args, 0, stream);
}

template <class In, class OutT, bool ACC>
hipError_t launch_skinny(const GemmProblem& p, hipStream_t stream) {
  const unsigned short* A = static_cast<const unsigned short*>(p.A);
  const unsigned short* B = static_cast<const unsigned short*>(p.B);
  OutT* Out = static_cast<OutT*>(p.Out);
  int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb, ldo = p.ldo;
  int64_t sA = p.sA, sB = p.sB, sO = p.sO;
  int64_t tiles_m = (M + kSkRows - 1) / kSkRows;
  void* args[] = {&A, &B, &Out, &M, &N, &K, &lda, &ldb, &ldo, &sA, &sB, &sO, &tiles_m};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_nt_skinny_kernel<In, OutT, ACC>),
                         dim3(static_cast<unsigned>(tiles_m * p.batch)), dim3(kSkWaves * 64), args, 0, stream);
}

template <class T>
struct Tag {
  typedef T type;
};

// Calls f(Tag<In>, Tag<OutT>, integral_constant<bool, ACC>) for the problem's types.
template <class F>
hipError_t with_types(const GemmProblem& p, F&& f) {
  std::integral_constant<bool, true> acc;
  std::integral_constant<bool, false> fresh;
  if (p.ab_type == Dtype::kBF16) {
    if (p.out_type == Dtype::kF32) return p.accumulate ? f(Tag<InBF16>{}, Tag<float>{}, acc) : f(Tag<InBF16>{}, Tag<float>{}, fresh);
    return p.accumulate ? f(Tag<InBF16>{}, Tag<__bf16>{}, acc) : f(Tag<InBF16>{}, Tag<__bf16>{}, fresh);
  }
  if (p.out_type == Dtype::kF32) return p.accumulate ? f(Tag<InF16>{}, Tag<float>{}, acc) : f(Tag<InF16>{}, Tag<float>{}, fresh);
  return p.accumulate ? f(Tag<InF16>{}, Tag<_Float16>{}, acc) : f(Tag<InF16>{}, Tag<_Float16>{}, fresh);
}

template <class C>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  return with_types(p, [&](auto in, auto out, auto acc) {
    return launch<C, typename decltype(in)::type, typename decltype(out)::type, decltype(acc)::value>(p, stream);
  });
}

hipError_t launch_skinny_typed(const GemmProblem& p, hipStream_t stream) {
  return with_types(p, [&](auto in, auto out, auto acc) {
    return launch_skinny<typename decltype(in)::type, typename decltype(out)::type, decltype(acc)::value>(p, stream);
  });
}

}  // namespace

GemmPlan choose_gemm_plan(int64_t M, int64_t N, int64_t /*K*/, int64_t batch) {
  if (M <= 0 || N <= 0 || batch <= 0) return GemmPlan::kNone;
  if (M <= 32 && N <= 32) return GemmPlan::kWave32;
  if (N <= 16) return GemmPlan::kSkinny;
  // 256x256 tiles only where they are mostly full and there are enough of
  // them to occupy at least half of the 256 CUs.
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256) * batch;
  if (M >= 256 && N >= 256 && big_tiles >= 128) return GemmPlan::kWg256;
  return GemmPlan::kWg128x64;
}

const char* gemm_plan_name(GemmPlan plan) {
  switch (plan) {
    case GemmPlan::kWave32: return "wave32x32_mfma32x32x16";
    case GemmPlan::kWg128x64: return "wg128x64_w4_mfma32x32x16";
    case GemmPlan::kWg256: return "wg256x256_w4_mfma32x32x16";
    case GemmPlan::kSkinny: return "skinny64xN16_w8_mfma16x16x32";
    default: return nullptr;
  }
}

int64_t gemm_plan_grid(GemmPlan plan, int64_t M, int64_t N, int64_t batch) {
  int64_t tm, tn;
  switch (plan) {
    case GemmPlan::kWave32: return tiles_of<CfgWave32>(M, N, batch, &tm, &tn);
    case GemmPlan::kWg128x64: return tiles_of<CfgWg128x64>(M, N, batch, &tm, &tn);
    case GemmPlan::kWg256: return tiles_of<CfgWg256>(M, N, batch, &tm, &tn);
    case GemmPlan::kSkinny: return (M + kSkRows - 1) / kSkRows * batch;
    default: return 0;
  }
}

template <class C>
bool fits_offsets(int64_t K, int64_t lda, int64_t ldb) {
  const int64_t limit = int64_t(1) << 32;
  return 2 * ((C::BM - 1) * lda + K) < limit && 2 * ((C::BN - 1) * ldb + K) < limit;
}

bool gemm_plan_fits_offsets(GemmPlan plan, int64_t K, int64_t lda, int64_t ldb) {
  switch (plan) {
    case GemmPlan::kWave32: return fits_offsets<CfgWave32>(K, lda, ldb);
    case GemmPlan::kWg128x64: return fits_offsets<CfgWg128x64>(K, lda, ldb);
    case GemmPlan::kWg256: return fits_offsets<CfgWg256>(K, lda, ldb);
    default: return true;
  }
}

hipError_t launch_gemm(GemmPlan plan, const GemmProblem& p, hipStream_t stream) {
  switch (plan) {
    case GemmPlan::kWave32: return launch_cfg<CfgWave32>(p, stream);
    case GemmPlan::kWg128x64: return launch_cfg<CfgWg128x64>(p, stream);
    case GemmPlan::kWg256: return launch_cfg<CfgWg256>(p, stream);
    case GemmPlan::kSkinny: return launch_skinny_typed(p, stream);
    default: return hipSuccess;
  }
}

}  // namespace fp16mc
