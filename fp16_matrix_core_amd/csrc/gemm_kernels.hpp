// gemm_kernels.hpp -- Out = A @ B.T on gfx950: the kernel templates.
// Each storage order of the operands is instantiated in a source file of its
// own (gemm_nt.hip, gemm_nn.hip, gemm_tt.hip, gemm_tn.hip) so that they
// compile in parallel; gemm_plan.hip holds the host-side plan logic.
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
//                   consecutive-K fp16 that v_mfma_f32_16x16x32_f16 (or
//                   v_mfma_f32_32x32x16_f16) takes from each lane, for a
//                   K-contiguous operand; an operand stored MN-contiguous is
//                   staged as it lies and read with two ds_read_b64_tr_b16.
//   MFMA            A's fragment is the instruction's first operand, B's
//                   the second, so in each accumulator register consecutive
//                   lanes hold consecutive columns of one output row (32 for
//                   32x32 tiles, 16 for 16x16 ones).
//   K loop          a ring of LDS stages; each slice's loads are issued
//                   STAGES-1 slices ahead, spread between MFMAs, and the
//                   fragments of the next K step are read while the current
//                   one multiplies; one workgroup barrier per slice.
//   scheduler       XCD-contiguous ranges of tile ids, grouped so that the
//                   tiles an XCD runs together share A and B panels in L2
//                   (streamed operands: dispatch order, K staggered).
//   edges           rows past M or N are clamped on load (their results are
//                   never stored); K past the end is zero-filled; Out is
//                   accessed through a buffer that ends at the tile's last
//                   valid element, with columns past N given an offset
//                   outside it, so every tile stores through one path.

#pragma once

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
// The accumulator type picks the instruction shape: 32x32x16 or 16x16x32.
struct InF16 {
  typedef f16x8 V8;
  static __device__ __forceinline__ f32x16 mma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // The same instruction with the accumulator tied to one AGPR quad.  The
  // compiler inserts no wait states around inline assembly, so the hazards
  // are the caller's: mma_tied_nop adds the two wait states that a VALU write
  // of the accumulator (its zero initialisation) needs before an MFMA reads
  // it; mma_fresh starts an accumulator from an inline-constant zero C
  // operand instead, reading no register; after the last MFMA, see
  // tied_mma_fence.
  static __device__ __forceinline__ f32x4 mma_tied(V8 a, V8 b, f32x4 c) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
  }
  static __device__ __forceinline__ f32x4 mma_tied_nop(V8 a, V8 b, f32x4 c) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
  }
  static __device__ __forceinline__ f32x4 mma_fresh(V8 a, V8 b) {
    f32x4 c;
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
    return c;
  }
};
struct InBF16 {
  typedef bf16x8 V8;
  static __device__ __forceinline__ f32x16 mma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma_tied(V8 a, V8 b, f32x4 c) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
  }
  static __device__ __forceinline__ f32x4 mma_tied_nop(V8 a, V8 b, f32x4 c) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
  }
  static __device__ __forceinline__ f32x4 mma_fresh(V8 a, V8 b) {
    f32x4 c;
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
    return c;
  }
};

// Lane maps of the two instruction shapes as the kernel uses them: the
// operand row and 8-wide K group of a lane (a K step of kK values is
// kGroups groups), its accumulator cells, and for transposed tiles the K
// row and M offset of the 8 bytes it names in a ds_read_b64_tr_b16.
template <int MI>
struct Mma;
template <>
struct Mma<32> {
  static constexpr int kM = mfma32::kM, kK = mfma32::kK, kAcc = mfma32::kAcc, kGroups = 2;
  typedef f32x16 Acc;
  static __device__ __forceinline__ int row(int lane) { return mfma32::operand_row(lane); }
  static __device__ __forceinline__ int kgroup(int lane) { return lane >> 5; }
  static __device__ __forceinline__ int acc_row(int lane, int v) { return mfma32::acc_row(lane, v); }
  static __device__ __forceinline__ int acc_col(int lane) { return mfma32::acc_col(lane, 0); }
  static __device__ __forceinline__ int tr_k(int lane) { return 8 * (lane >> 5) + ((lane >> 2) & 3); }
  static __device__ __forceinline__ int tr_m(int lane) { return 16 * ((lane >> 4) & 1) + 4 * (lane & 3); }
};
template <>
struct Mma<16> {
  static constexpr int kM = mfma16::kM, kK = mfma16::kK, kAcc = mfma16::kAcc, kGroups = 4;
  typedef f32x4 Acc;
  static __device__ __forceinline__ int row(int lane) { return mfma16::operand_row(lane); }
  static __device__ __forceinline__ int kgroup(int lane) { return lane >> 4; }
  static __device__ __forceinline__ int acc_row(int lane, int v) { return mfma16::acc_row(lane, v); }
  static __device__ __forceinline__ int acc_col(int lane) { return mfma16::acc_col(lane, 0); }
  static __device__ __forceinline__ int tr_k(int lane) { return 8 * (lane >> 4) + ((lane >> 2) & 3); }
  static __device__ __forceinline__ int tr_m(int lane) { return 4 * (lane & 3); }
};

// BM x BN output tile per workgroup, WM x WN wavefronts, each owning a
// (BM/WM) x (BN/WN) sub-tile made of MI x MI MFMA tiles (MI = 32: 32x32x16,
// MI = 16: 16x16x32).  K advances in slices of BK (32 or 64) held in a ring
// of STAGES LDS stages; WAVES_PER_SIMD workgroups' worth of wavefronts share
// each SIMD (the register budget follows from it).
template <int BM_, int BN_, int WM_, int WN_, int GROUP_M_, int STAGES_, int WAVES_PER_SIMD_, int BK_ = 32,
          int STREAM_ = 0, int MI_ = 32>
struct Cfg {
  // STREAM bit 0 / bit 1: A's / B's tiles are read by one workgroup only, so
  // their direct loads are non-temporal (no reuse to keep them cached for).
  // Bit 2: the output is written with non-temporal stores.
  static constexpr int STREAM = STREAM_;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, GROUP_M = GROUP_M_;
  static constexpr int BK = BK_;
  static constexpr int MI = MI_;
  using Mm = Mma<MI_>;
  using Swz = LdsSwizzle<2 * BK_, MI_>;
  static constexpr int STAGES = STAGES_;
  static constexpr int WAVES_PER_SIMD = WAVES_PER_SIMD_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int SI = WTM / MI, SJ = WTN / MI;
  static constexpr int A_STAGE = BM * Swz::kRowBytes;
  static constexpr int B_STAGE = BN * Swz::kRowBytes;
  static constexpr int ROWS_PER_WAVE = 1024 / Swz::kRowBytes;     // one 1 KiB direct load
  static constexpr int ROWS_PER_PASS = (NT / 64) * ROWS_PER_WAVE;
  static constexpr int A_LOADS = BM / ROWS_PER_PASS;
  static constexpr int B_LOADS = BN / ROWS_PER_PASS;
  static constexpr int LDS_BYTES = STAGES * (A_STAGE + B_STAGE);
  static_assert(BK == 32 || BK == 64, "an LDS row holds one 32- or 64-wide K slice");
  static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile must be whole MFMA tiles");
  static_assert(BK % (2 * Mm::kK) == 0, "a slice holds an even number of K steps");
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "rows must split evenly");
  static_assert(STAGES >= 2 && STAGES <= 4, "two to four LDS stages");
  static constexpr int WGS_PER_CU = WAVES_PER_SIMD * 256 / NT > 0 ? WAVES_PER_SIMD * 256 / NT : 1;
  static_assert(LDS_BYTES * WGS_PER_CU <= 160 * 1024, "gfx950 LDS is 160 KiB per CU");
};

using CfgWave32 = Cfg<32, 32, 1, 1, 1, 4, 1>;
// 64x64 tiles, four wavefronts of 32x32 (64-wide slices in four 16 KiB
// stages), for products with at most 256 such tiles -- at most one per CU --
// that the larger tiles would spread over a fraction of the CUs.  Against
// 128x64 tiles: 1024^2 x 4096 22 -> 15 us, 1024^2 x 8192 38 -> 24 us,
// 512^2 x 16384 69 -> 42 us, 2048 x 512 x 4096 21 -> 15 us; with more tiles
// the 128x64 ones win again (1280^2 x 4096 24.5 against 22 us).  One
// wavefront per 32x32 tile with 64-wide slices was within 5% of these on
// long-K shapes and up to 16% slower on others.
using CfgWg64 = Cfg<64, 64, 2, 2, 8, 4, 1, 64, 0, 16>;
using CfgWg64Mn = Cfg<64, 64, 2, 2, 8, 4, 1, 64>;
// 128x64 tiles: 64-wide slices in three 24 KiB stages (two workgroups per CU
// by LDS); measured 28% faster at 2048^3 than 32-wide slices in four stages.
// K-contiguous operands use 16x16x32 instructions, MN-contiguous ones
// 32x32x16 (the "Mn" twin; the larger tiles below use 16x16x32 for both).
using CfgWg128x64 = Cfg<128, 64, 4, 1, 8, 3, 1, 64, 0, 16>;
using CfgWg128x64Mn = Cfg<128, 64, 4, 1, 8, 3, 1, 64>;
// 256x256 tiles: 64-wide slices in two 64 KiB stages (three do not fit in
// 160 KiB); measured 6-7% faster at 8192^3 than 32-wide slices in four stages.
// Each tile ends with its 256 KiB of output written by one CU, which its
// write path takes about 15 us to drain (about 8% of a tile at 8192^3, in
// every wave of tiles); non-temporal stores and buffer stores without
// per-element bounds checks shorten it.
// 16x16x32 instructions: with random operands the chip is power-bound, and
// the 16x16 form sustains about 17% more MFMA throughput than the 32x32 one
// (it moves half the accumulator per flop); 8192^3 is 5-8% faster with it.
// With the fragment reads interleaved the smaller tiles gain from it too
// (256x128 and 128x128 5-10%, 128x64 2-3%; only single-slice K = 64 loses,
// 7%). With an operand stored MN-contiguous the compiler's MFMA builtin made
// NN and TN spill and TT run 13% slower (accumulators shuffled between
// AGPRs); those kernels issue the MFMA with tied accumulators instead (see
// kTied in the kernel): 8192^3 NN 842 -> 789 us, TT 839 -> 791 us, TN 842
// -> 800 us against 32x32x16; without a wait state before every MFMA
// (interleaved on one box) NN 800 -> 758, TT 799 -> 756, TN 808 -> 760 us,
// against NT 744 us.
using CfgWg256 = Cfg<256, 256, 2, 2, 4, 2, 1, 64, 4, 16>;
// Tall 64x32 tiles for N <= 32: the product streams A (read by one
// workgroup each, non-temporal) against a B that every workgroup shares.
// 16384x8x16384: 93 us against 118 us for a dedicated register-streaming
// kernel with 16x16x32 MFMAs (full-line direct loads and the streaming hint
// make the difference), 80 us with the staggered K sweep of the K loop.
using CfgTall = Cfg<64, 32, 2, 1, 1, 4, 1, 64, 1>;
// The 128x64 tiles with operands and output streamed, for problems that are
// one tile each (batches of small products; each workgroup reads and writes
// its own data once): two 24 KiB stages, so more workgroups share a CU.
// 4096 x 128x64x64: 47 -> 43 us.
using CfgWg128x64Stream = Cfg<128, 64, 4, 1, 8, 2, 2, 64, 7>;
// Intermediate tiles for problems too small to fill the 256 CUs with
// 256x256 tiles: 256x128 (three 48 KiB stages) and 128x128 (two 32 KiB
// stages, two workgroups per CU).
// With an MN-contiguous operand these two and the 256x256 tiles keep their
// 16x16x32 configuration (accumulators tied to their AGPRs, see the
// kernel): against 32x32x16, 8192x1024x8192 NN 117.7 -> 113.1 us, TN 118.9
// -> 117.4 us, 6144^2x2048 NN 158.2 -> 153.7 us, TN 157.9 -> 152.5 us.  The
// 128x64 and 64x64 tiles keep 32x32x16 for them (16x16x32 measured 1-2%
// slower there: 2048^3 TN 26.2 -> 26.8 us, 1024^2x4096 17.2 -> 17.5 us).
using CfgWg256x128 = Cfg<256, 128, 2, 2, 4, 3, 1, 64, 0, 16>;
using CfgWg128x128 = Cfg<128, 128, 2, 2, 8, 2, 2, 64, 0, 16>;
// Wide 32x64 tiles for M <= 32: the mirror of the tall tiles, B streamed.
using CfgWide = Cfg<32, 64, 1, 2, 1, 4, 1, 64, 2>;

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// Elements [k, k+8) of a row, zero past K.  `row` points at element 0 and
// k is a multiple of 8, so a chunk wholly inside the row is one aligned
// 16-byte load (rows are 16-byte aligned); only the chunk that straddles K
// goes element by element.  Only the last, partial K slice of a problem
// takes this path.
__device__ __forceinline__ u32x4 load_chunk_masked(const unsigned short* row, int64_t k, int64_t K) {
  if (k + 8 <= K) return *reinterpret_cast<const u32x4*>(row + k);
  unsigned int w[4] = {0u, 0u, 0u, 0u};
  if (k < K) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (k + e < K) w[e >> 1] |= static_cast<unsigned int>(row[k + e]) << (16 * (e & 1));
    }
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds):
// lane l's bytes land at lds_span + 16 l; `lds_span` and `soff` are uniform.
// NT = true sets the non-temporal hint.
template <bool NT = false>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, unsigned char* lds_span, unsigned voff,
                                      unsigned soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_span, 16, voff, soff, 0, NT ? 2 : 0);
}

// 8 consecutive-K values of one M for an MFMA operand from a transposed
// (MN-contiguous) LDS tile: two ds_read_b64_tr_b16, K rows k..k+3 at `lo` and
// k+4..k+7 at `hi` (addresses as set up by the kernel).
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
template <class V8>
__device__ __forceinline__ V8 tr_read8(const unsigned char* lo, const unsigned char* hi) {
  typedef __attribute__((address_space(3))) short4v lds_short4v;
  const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(lo));
  const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(hi));
  return __builtin_bit_cast(V8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
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

// The K loop's lambdas hold the accumulators and fragments by reference:
// they must be inlined for those arrays to live in registers.
#define FP16MC_INLINE __attribute__((always_inline))

// v_permlane16_swap_b32 x, y: 16-lane rows 1 and 3 of x trade places with
// rows 0 and 2 of y (measured on gfx950).  Inline assembly: the compiler's
// builtin for it merged the swaps of different elements of one accumulator
// vector into one.  The s_nop covers the VALU write of x and y just before.
__device__ __forceinline__ void permlane16_swap(float& x, float& y) {
  asm volatile("s_nop 4\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
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

template <class C, class In, class OutT, bool ACC, bool A_MN, bool B_MN>
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
  // Tiles that share operand panels take XCD-contiguous id ranges (their L2
  // reuse); with a streamed operand nothing worth keeping is shared, and the
  // dispatch order itself keeps the concurrently running tiles on adjacent
  // memory (the ranges put the 8 XCDs' streams a power-of-two stride apart:
  // 4096 x 128x64x64 43 -> 41 us, 32x16384x8192 43 -> 40 us).
  const uint32_t lin =
      (C::STREAM & 3) != 0 ? blockIdx.x : sched::xcd_remap(blockIdx.x, static_cast<uint32_t>(total));
  const uint32_t per_problem = static_cast<uint32_t>(tiles_m * tiles_n);
  const uint32_t b = __builtin_amdgcn_readfirstlane(lin / per_problem);
  const sched::Tile tile = sched::grouped_tile(lin - b * per_problem, static_cast<uint32_t>(tiles_m),
                                               static_cast<uint32_t>(tiles_n), C::GROUP_M);
  // Integer division runs on the vector unit: name the (uniform) results as
  // scalars so that the tile origin does not hold vector registers.
  const int64_t i0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(tile.m)) * C::BM;
  const int64_t j0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(tile.n)) * C::BN;
  A += b * sA;
  B += b * sB;
  Out += b * sO;

  // ---- global -> LDS assignment ------------------------------------------------
  // Direct load p of wavefront w fills the 1 KiB LDS span [(p*NW + w) KiB,
  // +1 KiB) of a stage; lane l lands at byte 16 l of it.
  //   K-contiguous operand (A[i*lda + k]): the span holds RW whole tile rows of
  //     BK values; lane l fetches the logical chunk that the row swizzle puts
  //     at its physical slot.  Rows past the matrix edge re-read its last row
  //     (their results are never stored).  Byte offsets are relative to a
  //     buffer at the tile's first row: a per-lane offset plus a uniform K
  //     offset; the last, partial K slice goes through registers with masks.
  //   MN-contiguous operand (A[k*lda + i]): the span holds 1024/(2W) K rows of
  //     the tile's W values, placed by the transposed-tile swizzle.  The buffer
  //     is rebuilt for every slice at the slice's first K row and ends at the
  //     last element of row K-1, so K rows past the end read as zeros (the
  //     partial slice needs no special path).  Columns past M read whatever
  //     memory holds there; they only feed output rows that are never stored.
  constexpr int NW = C::NT / 64;                   // wavefronts per workgroup
  constexpr int RW = C::ROWS_PER_WAVE;
  auto span = [&](int p) { return (p * NW + wave) * 1024; };
  const int64_t a_ext = (M - i0) < C::BM ? (M - i0) : C::BM;   // valid tile rows (K-contiguous)
  const int64_t b_ext = (N - j0) < C::BN ? (N - j0) : C::BN;
  const unsigned short* a_tile = A_MN ? A + i0 : A + i0 * lda;
  const unsigned short* b_tile = B_MN ? B + j0 : B + j0 * ldb;
  unsigned a_off[C::A_LOADS];
  unsigned b_off[C::B_LOADS];
  // Per-lane byte offsets of the direct loads of one operand.
  auto setup_offsets = [&](auto mn, auto w, int64_t ext, int64_t ld, unsigned* off, auto loads) {
    constexpr int kLoadsOp = decltype(loads)::value;
    if constexpr (!decltype(mn)::value) {
      const int prow = lane / C::Swz::kChunks;
      const int pchunk = lane % C::Swz::kChunks;
#pragma unroll
      for (int p = 0; p < kLoadsOp; ++p) {
        const int r = p * C::ROWS_PER_PASS + RW * wave + prow;
        const int64_t rr = r < ext ? r : ext - 1;
        off[p] = static_cast<unsigned>(2 * (rr * ld + 8 * C::Swz::logical_chunk(r, pchunk)));
      }
    } else {
      using TZ = TrSwizzle<2 * decltype(w)::value, C::MI>;
      constexpr int RK = 1024 / TZ::kRowBytes;     // K rows per 1 KiB span
      const int kr = lane / TZ::kChunks;
      const int pc = lane % TZ::kChunks;
#pragma unroll
      for (int p = 0; p < kLoadsOp; ++p) {
        const int k = (p * NW + wave) * RK + kr;
        off[p] = static_cast<unsigned>(2 * (k * ld + 8 * TZ::logical_chunk(k, pc)));
      }
    }
  };
  setup_offsets(std::integral_constant<bool, A_MN>{}, std::integral_constant<int, C::BM>{}, a_ext, lda, a_off,
                std::integral_constant<int, C::A_LOADS>{});
  setup_offsets(std::integral_constant<bool, B_MN>{}, std::integral_constant<int, C::BN>{}, b_ext, ldb, b_off,
                std::integral_constant<int, C::B_LOADS>{});
  // K-contiguous operands: one buffer over the tile's rows for the whole loop.
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(a_tile, static_cast<unsigned>(2 * ((a_ext - 1) * lda + K)));
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(b_tile, static_cast<unsigned>(2 * ((b_ext - 1) * ldb + K)));
  // MN-contiguous operands: the buffer of slice `slice` (rows [slice*BK, K)).
  // The range check works per dword, so the last row's extent is rounded up
  // to the 16-byte block that holds its last element (same page, never a
  // fault; the extra values only feed outputs past M or N); rows past the
  // slice's end still start beyond the range, because ld is a multiple of 8.
  auto slice_rsrc = [&](const unsigned short* tile, int64_t ld, int64_t cols, int64_t slice) {
    const int64_t k0 = slice * C::BK;
    const int64_t rows = (K - k0) < C::BK ? (K - k0) : C::BK;
    const int64_t last = (2 * cols + 15) & ~int64_t(15);
    return make_rsrc(tile + k0 * ld, static_cast<unsigned>(2 * (rows - 1) * ld + last));
  };
  constexpr int kLoads = C::A_LOADS + C::B_LOADS;   // direct loads per slice per wavefront
  constexpr bool kNtA = (C::STREAM & 1) != 0, kNtB = (C::STREAM & 2) != 0;
  // All direct loads of slice `slice` (A's, then B's).
  auto dma_all = [&](unsigned char* as, unsigned char* bs, int64_t slice) FP16MC_INLINE {
    const unsigned koff = static_cast<unsigned>(2 * C::BK * slice);
    if constexpr (!A_MN) {
#pragma unroll
      for (int q = 0; q < C::A_LOADS; ++q) dma16<kNtA>(a_rsrc, as + span(q), a_off[q], koff);
    } else {
      const __amdgpu_buffer_rsrc_t r = slice_rsrc(a_tile, lda, M - i0, slice);
#pragma unroll
      for (int q = 0; q < C::A_LOADS; ++q) dma16<kNtA>(r, as + span(q), a_off[q], 0);
    }
    if constexpr (!B_MN) {
#pragma unroll
      for (int q = 0; q < C::B_LOADS; ++q) dma16<kNtB>(b_rsrc, bs + span(q), b_off[q], koff);
    } else {
      const __amdgpu_buffer_rsrc_t r = slice_rsrc(b_tile, ldb, N - j0, slice);
#pragma unroll
      for (int q = 0; q < C::B_LOADS; ++q) dma16<kNtB>(r, bs + span(q), b_off[q], 0);
    }
  };
  // Direct load q (A's first, then B's) of slice `slice`.
  auto dma_one = [&](unsigned char* as, unsigned char* bs, int64_t slice, auto qc) FP16MC_INLINE {
    constexpr int q = decltype(qc)::value;
    const unsigned koff = static_cast<unsigned>(2 * C::BK * slice);
    if constexpr (q < C::A_LOADS) {
      if constexpr (!A_MN) dma16<kNtA>(a_rsrc, as + span(q), a_off[q], koff);
      else dma16<kNtA>(slice_rsrc(a_tile, lda, M - i0, slice), as + span(q), a_off[q], 0);
    } else {
      constexpr int qb = q - C::A_LOADS;
      if constexpr (!B_MN) dma16<kNtB>(b_rsrc, bs + span(qb), b_off[qb], koff);
      else dma16<kNtB>(slice_rsrc(b_tile, ldb, N - j0, slice), bs + span(qb), b_off[qb], 0);
    }
  };
  // Last, partial K slice (index nfull): K-contiguous operands through
  // registers with per-element masks, MN-contiguous ones by direct loads.
  auto load_tail = [&](unsigned char* as, unsigned char* bs, int64_t slice) FP16MC_INLINE {
    const int64_t k0 = slice * C::BK;
    if constexpr (!A_MN) {
#pragma unroll
      for (int p = 0; p < C::A_LOADS; ++p) {
        const int lc = C::Swz::logical_chunk(p * C::ROWS_PER_PASS + RW * wave + lane / C::Swz::kChunks,
                                             lane % C::Swz::kChunks);
        const unsigned short* row = a_tile + a_off[p] / 2 - 8 * lc;
        *reinterpret_cast<u32x4*>(as + span(p) + 16 * lane) = load_chunk_masked(row, k0 + 8 * lc, K);
      }
    } else {
      const __amdgpu_buffer_rsrc_t r = slice_rsrc(a_tile, lda, M - i0, slice);
#pragma unroll
      for (int p = 0; p < C::A_LOADS; ++p) dma16<kNtA>(r, as + span(p), a_off[p], 0);
    }
    if constexpr (!B_MN) {
#pragma unroll
      for (int p = 0; p < C::B_LOADS; ++p) {
        const int lc = C::Swz::logical_chunk(p * C::ROWS_PER_PASS + RW * wave + lane / C::Swz::kChunks,
                                             lane % C::Swz::kChunks);
        const unsigned short* row = b_tile + b_off[p] / 2 - 8 * lc;
        *reinterpret_cast<u32x4*>(bs + span(p) + 16 * lane) = load_chunk_masked(row, k0 + 8 * lc, K);
      }
    } else {
      const __amdgpu_buffer_rsrc_t r = slice_rsrc(b_tile, ldb, N - j0, slice);
#pragma unroll
      for (int p = 0; p < C::B_LOADS; ++p) dma16<kNtB>(r, bs + span(p), b_off[p], 0);
    }
  };

  // ---- fragment reads + MFMA ------------------------------------------------
  using Mm = typename C::Mm;
  typename Mm::Acc acc[C::SI][C::SJ];
#pragma unroll
  for (int si = 0; si < C::SI; ++si)
#pragma unroll
    for (int sj = 0; sj < C::SJ; ++sj) acc[si][sj] = typename Mm::Acc{};

  const int frow = Mm::row(lane);                  // row inside an MFMA tile
  const int kgrp = Mm::kgroup(lane);               // which 8-wide K group of a K step
  const int key = C::Swz::key(frow);          // equal to key(row) for every fragment row
  const int a_row0 = (wm * C::WTM + frow) * C::Swz::kRowBytes;
  const int b_row0 = (wn * C::WTN + frow) * C::Swz::kRowBytes;
  constexpr int KK = C::BK / Mm::kK;               // K steps per slice (2 or 4)
  constexpr int NMF = C::SI * C::SJ;               // MFMAs per K step
  // LDS reads per K step: one ds_read_b128 per K-contiguous fragment, two
  // ds_read_b64_tr_b16 per MN-contiguous one.
  constexpr int kFr = C::SI * (A_MN ? 2 : 1) + C::SJ * (B_MN ? 2 : 1);
  static_assert(KK % 2 == 0, "fragments alternate between two register sets");

  struct Frags {
    typename In::V8 a[C::SI];
    typename In::V8 b[C::SJ];
  };
  // MN-contiguous tiles: lane l = 16g + 4r + q names K row Mm::tr_k(l) (+4
  // for the second half of its 8 K values, +kK per K step) at M offset
  // Mm::tr_m(l) of each MFMA tile; the swizzle key is a per-lane constant.
  int a_tr[C::SI];
  int b_tr[C::SJ];
  if constexpr (A_MN) {
    using TZ = TrSwizzle<2 * C::BM, C::MI>;
#pragma unroll
    for (int si = 0; si < C::SI; ++si)
      a_tr[si] = TZ::offset_bytes(Mm::tr_k(lane), wm * C::WTM + Mm::kM * si + Mm::tr_m(lane));
  }
  if constexpr (B_MN) {
    using TZ = TrSwizzle<2 * C::BN, C::MI>;
#pragma unroll
    for (int sj = 0; sj < C::SJ; ++sj)
      b_tr[sj] = TZ::offset_bytes(Mm::tr_k(lane), wn * C::WTN + Mm::kM * sj + Mm::tr_m(lane));
  }
  // Fragment x of K step kk: A's fragment si = x for x < SI, else B's sj = x - SI.
  auto read_one = [&](const unsigned char* as, const unsigned char* bs, int kk, Frags& f, auto xc) FP16MC_INLINE {
    constexpr int x = decltype(xc)::value;
    static_assert(x >= 0 && x < C::SI + C::SJ, "fragment index");
    const int pc = ((Mm::kGroups * kk + kgrp) ^ key) << 4;
    if constexpr (x < C::SI) {
      constexpr int si = x;
      if constexpr (!A_MN) {
        f.a[si] = *reinterpret_cast<const typename In::V8*>(as + a_row0 + si * Mm::kM * C::Swz::kRowBytes + pc);
      } else {
        const unsigned char* p = as + a_tr[si] + Mm::kK * kk * (2 * C::BM);
        f.a[si] = tr_read8<typename In::V8>(p, p + 4 * (2 * C::BM));
      }
    } else {
      constexpr int sj = x - C::SI;
      if constexpr (!B_MN) {
        f.b[sj] = *reinterpret_cast<const typename In::V8*>(bs + b_row0 + sj * Mm::kM * C::Swz::kRowBytes + pc);
      } else {
        const unsigned char* p = bs + b_tr[sj] + Mm::kK * kk * (2 * C::BN);
        f.b[sj] = tr_read8<typename In::V8>(p, p + 4 * (2 * C::BN));
      }
    }
  };
  auto read_frags = [&](const unsigned char* as, const unsigned char* bs, int kk, Frags& f) FP16MC_INLINE {
    static_for<C::SI + C::SJ>([&](auto x) { read_one(as, bs, kk, f, x); });
  };
  // Fresh 16-bit outputs of the four-wavefront 16x16x32 tiles leave through LDS
  // (epilogue below).  Their MFMAs take B's fragment first, which transposes
  // each 16x16 accumulator: lane l then holds row l%16 and the four
  // consecutive columns 4(l/16) .. 4(l/16)+3, i.e. 8 bytes of one output row
  // once rounded.  Each element is the same sum of the same products.
  constexpr bool kLdsOut = sizeof(OutT) == 2 && !ACC && C::MI == 16 && C::NT == 256;
  // With an MN-contiguous operand the 16x16x32 kernels hold two more sets of
  // per-fragment LDS offsets, and the register allocator, free to give an
  // MFMA's result other registers than its accumulator input, then shuffled
  // the 256 accumulators between AGPRs (some 400 moves per K-loop iteration,
  // or spills).  Those kernels issue the MFMA as inline assembly with the
  // accumulator tied to its AGPRs, which leaves the result-read hazard to
  // tied_mma_fence below.
  constexpr bool kTied = C::MI == 16 && (A_MN || B_MN);
  // How a tied MFMA meets its accumulator (ignored by the builtin form):
  // kAfterMfma -- last written by an MFMA, at least a K step earlier;
  // kFresh -- not yet written: start from zero (the first K step of the
  // pipelined path); kAfterInit -- just zeroed by the compiler (short K and
  // the partial slice), two wait states first.
  enum { kAfterMfma, kFresh, kAfterInit };
  auto mfma = [&](const Frags& f, int n, auto how) FP16MC_INLINE {
    constexpr int kHow = decltype(how)::value;
    const int si = n / C::SJ, sj = n % C::SJ;
    const auto& x = kLdsOut ? f.b[sj] : f.a[si];
    const auto& y = kLdsOut ? f.a[si] : f.b[sj];
    if constexpr (!kTied) acc[si][sj] = In::mma(x, y, acc[si][sj]);
    else if constexpr (kHow == kFresh) acc[si][sj] = In::mma_fresh(x, y);
    else if constexpr (kHow == kAfterInit) acc[si][sj] = In::mma_tied_nop(x, y, acc[si][sj]);
    else acc[si][sj] = In::mma_tied(x, y, acc[si][sj]);
  };
  std::integral_constant<int, kAfterMfma> after_mfma;
  std::integral_constant<int, kAfterInit> after_init;
  // The compiler inserts no wait states around an MFMA written as inline
  // assembly.  Before the first ones: the zeroes the compiler writes into
  // the accumulators must have landed before an MFMA reads them as its C
  // operand (without the wait, elements of the accumulators that the first
  // MFMAs read came out wrong, varying from run to run); the pipelined path
  // reads none (kFresh).  Between MFMAs nothing is needed: an accumulator's
  // next MFMA comes a whole K step later, and a wait state before every MFMA
  // made the 8192^3 product 4% slower.  After the last one (tied_mma_fence):
  // before anything other than the next MFMA reads an accumulator, wait
  // longer than the instruction's result latency (32 wait states, against
  // at most 19 in the CDNA3 ISA's dependency table), then pass every
  // accumulator through an empty statement ordered after the wait, so that
  // no read of them can be scheduled above it.
  auto tied_mma_fence = [&]() FP16MC_INLINE {
    if constexpr (kTied) {
      asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
      for (int si = 0; si < C::SI; ++si)
#pragma unroll
        for (int sj = 0; sj < C::SJ; ++sj) asm volatile("" : "+a"(acc[si][sj]));
    }
  };
  auto mfma_all = [&](const Frags& f, auto how) FP16MC_INLINE {
    static_for<NMF>([&](auto n) { mfma(f, decltype(n)::value, how); });
  };
  // Wait until at most `n` direct loads of this thread are in flight and its
  // LDS reads/writes are done, then make everyone's writes visible.
  // (A plain s_barrier: a fenced __syncthreads would also wait for the loads
  // that are meant to stay in flight.)
  auto publish_keep = [&](auto n) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(decltype(n)::value) & ~(15 << 8));  // lgkmcnt(0) as well
    asm volatile("s_barrier" ::: "memory");
  };

  // ---- Out tile addressing (epilogue) ---------------------------------------------
  // Every access to Out is a buffer access relative to the tile's origin,
  // with the whole offset (lane, column block and row) in the per-lane
  // offset register, which the buffer's range check covers.  The buffer ends
  // at the last valid element of the tile's last valid row, so rows past M
  // read as zero and their stores are dropped; lanes whose column is past N
  // take an offset beyond any buffer for that column block.  (The host keeps
  // BM * ldo * sizeof(OutT) below 2^31, so no offset wraps, and every tile
  // takes this one path.)
  constexpr int kSz = sizeof(OutT);
  constexpr int kAux = (C::STREAM & 4) != 0 ? 2 : 0;    // non-temporal stores
  constexpr unsigned kOff = 0x80000000u;               // beyond every tile's buffer
  const int64_t o_rows = (M - i0) < C::BM ? (M - i0) : C::BM;
  const int o_cols = static_cast<int>((N - j0) < C::BN ? (N - j0) : C::BN);
  const __amdgpu_buffer_rsrc_t orsrc =
      make_rsrc(Out + i0 * ldo + j0, static_cast<unsigned>(((o_rows - 1) * ldo + o_cols) * kSz));
  const int ldo_b = static_cast<int>(ldo) * kSz;       // bytes per row of Out
  // Per-lane offsets of column blocks 0 .. NC-1 of width CW, for a lane at
  // tile row `row` and column `col` of block 0.
  auto col_offsets = [&](unsigned* off, int nc, int cw, int row, int col) FP16MC_INLINE {
#pragma unroll
    for (int c = 0; c < nc; ++c)
      off[c] = col + c * cw < o_cols ? static_cast<unsigned>(row * ldo_b + (col + c * cw) * kSz) : kOff;
  };
  // Register layout of the stores.  16x16 tiles with an even SJ: the
  // registers of each pair of horizontally adjacent tiles (sj = 2p, 2p+1)
  // are regrouped with v_permlane16_swap (16-lane rows 1 and 3 of the first
  // operand trade places with rows 0 and 2 of the second), so that in
  // register t, element v, lane l holds Out[i][j] with
  // i = i0 + wm*WTM + 16 si + 4t + v + 8(l/32), j = j0 + wn*WTN + 32p + l%32:
  // each store covers two whole 32-column row pieces (128 bytes of fp32)
  // instead of four 16-column ones.  Otherwise element v of lane l in tile
  // (si, sj) is Out[i][j] with i = i0 + wm*WTM + MI si + acc_row(l, v),
  // j = j0 + wn*WTN + MI sj + acc_col(l) (two whole 128-byte row segments per
  // store with 32x32 tiles).  Below, (c, t, v) names element v of register t
  // of column block c (a tile pair p, or a tile sj with t = 0).
  constexpr bool kSwap = C::MI == 16 && C::SJ % 2 == 0;
  constexpr int kNC = kSwap ? C::SJ / 2 : C::SJ;   // column blocks
  constexpr int kNT = kSwap ? 2 : 1;               // registers per column block
  constexpr int kNV = kSwap ? 4 : Mm::kAcc;        // elements per register
  constexpr int kCW = kSwap ? 32 : Mm::kM;         // columns per block
  typedef float OutBlock[kNC][kNT][kNV];           // one row block's values
  auto elem_row = [&](int t, int v) { return kSwap ? mfma16::swapped_row(0, t, v) : Mm::acc_row(0, v); };
  auto so = [&](int si, int t, int v) { return (si * Mm::kM + elem_row(t, v)) * ldo_b; };
  auto acc_to_block = [&](int si, OutBlock& val) FP16MC_INLINE {
#pragma unroll
    for (int c = 0; c < kNC; ++c)
#pragma unroll
      for (int v = 0; v < kNV; ++v) {
        if constexpr (kSwap) {
          val[c][0][v] = acc[si][2 * c][v];
          val[c][1][v] = acc[si][2 * c + 1][v];
          permlane16_swap(val[c][0][v], val[c][1][v]);
        } else {
          val[c][0][v] = acc[si][c][v];
        }
      }
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
  // A streamed operand (each tile's rows read by that workgroup alone) is
  // swept from a per-workgroup starting slice, wrapping around: its rows lie
  // a power-of-two stride apart, and with every workgroup at the same K
  // offset their reads crowd the same memory channels (a 512 MiB row stream
  // ran at 5.9-6.0 TB/s in lockstep and 6.8-6.9 TB/s with staggered starts;
  // 16384x8x16384 93 -> 80 us).  Tiles that share operand panels keep the
  // common order, which their L2 reuse depends on (staggering the 8 XCDs'
  // starts gained under 1% at 8192^3; a one-tile-wide 128x64 grid gained
  // 1%).  The order of the sum changes, not its terms.
  constexpr bool kRotate = (C::STREAM & 3) != 0;
  const int64_t rot = kRotate && nfull > 1
                          ? __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(blockIdx.x * 37u % static_cast<uint32_t>(nfull)))
                          : 0;
  auto slice_of = [&](int64_t slice) {
    // slices past the end reload the last one into an idle stage: no branch, never read
    const int64_t s = (slice < nfull ? slice : nfull - 1) + rot;
    return s < nfull ? s : s - nfull;
  };
  std::integral_constant<int, (kAhead - 1) * kLoads> keep_later;
  static_assert((kAhead - 1) * kLoads <= 63, "loads kept in flight must fit the 6-bit vmcnt");
  constexpr int kLoadSteps = 2;                    // MFMA steps the slice loads are spread over
  // With 16x16 tiles a fragment set is 64 VGPRs, and the scheduler's own
  // interleaving (or group hints) keeps a third set live and shuffles the
  // accumulators.  Those phases are issued in a fixed order instead, fenced
  // in small groups: each step's MFMAs (the first step's are the carried
  // ones) with the next step's fragment reads after every kRdEvery-th, so
  // that the last read has a quarter of the step to land, and the slice
  // loads after every kLdEvery-th of the first step (offset by kLdFirst).
  // Reads issued back to back instead stall issue: 16 of them ahead of the
  // carried MFMAs made that step a third slower.
  constexpr bool kPinned = C::MI == 16;
  constexpr int kLdEvery = NMF / kLoads > 0 ? NMF / kLoads : 1;
  constexpr int kLdFirst = kLdEvery > 1 ? 1 : 0;
  constexpr int kFrags = C::SI + C::SJ;            // fragments per K step (read_one calls)
  constexpr int kRdEvery = NMF / kFrags > 1 ? NMF / kFrags * 3 / 4 : 1;
  static_assert(!kPinned || (kLdEvery * (kLoads - 1) < KK * NMF && kRdEvery * (kFrags - 1) < NMF),
                "every load and read finds an MFMA to follow");
  auto phase = [&](auto st, int64_t s, auto pending) FP16MC_INLINE {
    constexpr int S = decltype(st)::value;
    constexpr bool kPending = decltype(pending)::value;
    unsigned char* as = stage_a(st);
    unsigned char* bs = stage_b(st);
    unsigned char* an = stage_a(std::integral_constant<int, S + kAhead>{});
    unsigned char* bn = stage_b(std::integral_constant<int, S + kAhead>{});
    const int64_t next = slice_of(s + kAhead);
    if constexpr (kPinned) {
      if constexpr (kPending) {
        static_for<NMF>([&](auto n) {
          constexpr int i = decltype(n)::value;
          mfma(f1, i, after_mfma);
          if constexpr (i % kRdEvery == 0 && i / kRdEvery < kFrags)
            read_one(as, bs, 0, f0, std::integral_constant<int, i / kRdEvery>{});
          if constexpr (i % kLdEvery == kLdFirst && i / kLdEvery < kLoads)
            dma_one(an, bn, next, std::integral_constant<int, i / kLdEvery>{});
          sched_fence();
        });
      } else {
        read_frags(as, bs, 0, f0);
        dma_all(an, bn, next);
        sched_fence();
      }
      static_for<KK - 1>([&](auto t) {
        constexpr int kk = decltype(t)::value + 1;
        Frags& cur = kk % 2 == 1 ? f0 : f1;
        Frags& nxt = kk % 2 == 1 ? f1 : f0;
        static_for<NMF>([&](auto n) {
          constexpr int i = decltype(n)::value;
          constexpr int g = kk * NMF + i;          // MFMA index in the phase
          mfma(cur, i, std::integral_constant<int, (!kPending && kk == 1) ? kFresh : kAfterMfma>{});
          if constexpr (kPending && g % kLdEvery == kLdFirst && g / kLdEvery < kLoads)
            dma_one(an, bn, next, std::integral_constant<int, g / kLdEvery>{});
          if constexpr (i % kRdEvery == 0 && i / kRdEvery < kFrags)
            read_one(as, bs, kk, nxt, std::integral_constant<int, i / kRdEvery>{});
          sched_fence();
        });
      });
      publish_keep(keep_later);
      return;
    }
    read_frags(as, bs, 0, f0);
    if constexpr (kPending) mfma_all(f1, after_mfma);
    dma_all(an, bn, next);
    static_for<KK - 1>([&](auto t) {
      constexpr int kk = decltype(t)::value + 1;
      if constexpr (kk % 2 == 1) {
        read_frags(as, bs, kk, f1);
        mfma_all(f0, after_mfma);
      } else {
        read_frags(as, bs, kk, f0);
        mfma_all(f1, after_mfma);
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
      if (decltype(i)::value < nfull) dma_all(stage_a(i), stage_b(i), decltype(i)::value);
    });
    publish_keep(std::integral_constant<int, 0>{});
    static_for<kAhead>([&](auto i) {
      if (decltype(i)::value < nfull) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          read_frags(stage_a(i), stage_b(i), kk, f0);
          mfma_all(f0, after_init);
        }
      }
    });
  } else if (nfull > 0) {
    static_for<kAhead>([&](auto i) { dma_all(stage_a(i), stage_b(i), slice_of(decltype(i)::value)); });
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
    mfma_all(f1, after_mfma);  // step (nfull-1, KK-1)
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
    load_tail(as, bs, nfull);
    publish_keep(std::integral_constant<int, 0>{});
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      read_frags(as, bs, kk, f0);
      mfma_all(f0, after_init);
    }
  }

  // ---- 16-bit epilogue through LDS (the store direction of the fragment
  // copy: register fragments -> shared memory -> whole rows).  Wavefront w
  // owns one K-loop stage array as its staging region (stage a0, a1, b0, b1
  // for w = 0..3), free once every wavefront is past its last fragment read.
  // Each lane rounds its four values per tile and writes them as 8 bytes at
  // their place in a row-major (WTM x WTN) image of the wave tile (rows
  // swizzled by OutSwizzle, so that the 16 lanes writing 16 different rows
  // hit 16 different bank groups); the wavefront then reads the image back
  // as 16-byte row pieces, one row of the wave tile per WTN/8 lanes, and
  // stores them with 16-byte stores: every store instruction writes whole
  // row pieces of WTN values, against 2-byte stores of one element per lane.
  // A row piece that straddles N is stored element by element, so the ldo
  // padding is never written; rows past M fall outside the output buffer's
  // range.  (Accumulating 16-bit outputs keep the register epilogue below:
  // adding the previous values read from the image in the accumulator's
  // layout made the register allocator split the accumulators and spill.)
  tied_mma_fence();
  if constexpr (kLdsOut) {
    using OS = OutSwizzle<2 * C::WTN>;
    constexpr int kRowsPerAccess = 1024 / OS::kRowBytes;      // rows of the image per 1 KiB wavefront access
    constexpr int kAccesses = C::WTM / kRowsPerAccess;        // 16-byte accesses per lane over the wave tile
    static_assert(C::WM * C::WN == 4, "one staging region per wavefront: stages a0, a1, b0, b1");
    static_assert(C::WTM * OS::kRowBytes <= C::A_STAGE && C::WTM * OS::kRowBytes <= C::B_STAGE,
                  "a wave tile's 16-bit image fits one stage array");
    static_assert(C::WTM % kRowsPerAccess == 0, "whole 1 KiB accesses");
    unsigned char* region = wave == 0 ? lds_a0 : wave == 1 ? lds_a1 : wave == 2 ? lds_b0 : lds_b1;
    const int row0 = wm * C::WTM, col0 = wn * C::WTN;           // wave tile inside the workgroup tile
    const int ldo_b2 = static_cast<int>(ldo) * 2;               // bytes per row of Out
    // LDS byte offset of a lane's four values of tile (si, sj) in the image
    auto acc_off = [&](int si, int sj) {
      const int r = si * 16 + (lane & 15);
      const int col = sj * 16 + 4 * (lane >> 4);
      return OS::offset_bytes(r, col >> 3) + 2 * (col & 7);
    };
    // every wavefront is past its last read of the stages
    publish_keep(std::integral_constant<int, 0>{});
#pragma unroll
    for (int si = 0; si < C::SI; ++si)
#pragma unroll
      for (int sj = 0; sj < C::SJ; ++sj) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[si][sj][e];
        unsigned int* w = reinterpret_cast<unsigned int*>(region + acc_off(si, sj));
        unsigned int h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(unsigned short, static_cast<OutT>(v[e]));
        w[0] = h[0] | (h[1] << 16);
        w[1] = h[2] | (h[3] << 16);
        sched_fence();   // one tile at a time: no hoisted reads holding registers
      }
#pragma unroll
    for (int p = 0; p < kAccesses; ++p) {
      const int r = p * kRowsPerAccess + lane / OS::kChunks;
      const int c = lane % OS::kChunks;                       // logical chunk of row r
      const u32x4 val = *reinterpret_cast<const u32x4*>(region + OS::offset_bytes(r, c));
      const int col = col0 + 8 * c;                            // first column, inside the workgroup tile
      const unsigned off = static_cast<unsigned>((row0 + r) * ldo_b2 + col * 2);
      if (col + 8 <= o_cols) {
        __builtin_amdgcn_raw_buffer_store_b128(val, orsrc, off, 0, kAux);
      } else if (col < o_cols) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < o_cols)
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(val[e >> 1] >> (16 * (e & 1))), orsrc,
                                                  off + 2 * e, 0, kAux);
      }
    }
    return;
  }

  // ---- epilogue: each row block's values in the (c, t, v) layout, plus the
  // block's previous values when accumulating, stored as fp32 or rounded to
  // nearest-even fp16 / bf16.  The previous values are loaded kPre row
  // blocks ahead of their use: loads and stores share one in-order
  // completion counter, so waiting for a block's loads also waits for every
  // store issued before them, and a deeper prefetch lets the stores of the
  // last blocks stay in flight meanwhile (the registers of the blocks already
  // stored hold the prefetched values).  Measured at 8192^3 (16x16 tiles,
  // 32 values per block): three blocks ahead 4% faster than one for fp32,
  // two as good as three for 16 bits.  The depth is set in values, so that
  // the 64-value blocks of 32x32 tiles stay one block ahead (deeper, their
  // 256x256 kernels spill).
  unsigned vs[kNC];
  col_offsets(vs, kNC, kCW, wm * C::WTM + (kSwap ? mfma16::swapped_row(lane, 0, 0) : Mm::acc_row(lane, 0)),
              wn * C::WTN + (kSwap ? mfma16::swapped_col(lane) : Mm::acc_col(lane)));
  constexpr int kBlockVals = kNC * kNT * kNV;        // loads per row block
  constexpr int kPreVals = kSz == 4 ? 96 : 64;       // values in flight
  constexpr int kPre = kPreVals / kBlockVals < 1 ? 1 : (kPreVals / kBlockVals > C::SI ? C::SI : kPreVals / kBlockVals);
  OutBlock prev[kPre];
  auto load_block = [&](int si, OutBlock& pv) FP16MC_INLINE {
#pragma unroll
    for (int c = 0; c < kNC; ++c)
#pragma unroll
      for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int v = 0; v < kNV; ++v) {
          if constexpr (kSz == 4)
            pv[c][t][v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(orsrc, vs[c] + so(si, t, v), 0, 0));
          else
            pv[c][t][v] = static_cast<float>(
                __builtin_bit_cast(OutT, __builtin_amdgcn_raw_buffer_load_b16(orsrc, vs[c] + so(si, t, v), 0, 0)));
        }
  };
  if constexpr (ACC) {
#pragma unroll
    for (int si = 0; si < kPre; ++si) load_block(si, prev[si]);
  }
#pragma unroll
  for (int si = 0; si < C::SI; ++si) {
    OutBlock val;
    acc_to_block(si, val);
    if constexpr (ACC) {
#pragma unroll
      for (int c = 0; c < kNC; ++c)
#pragma unroll
        for (int t = 0; t < kNT; ++t)
#pragma unroll
          for (int v = 0; v < kNV; ++v) val[c][t][v] += prev[si % kPre][c][t][v];
      if (si + kPre < C::SI) load_block(si + kPre, prev[si % kPre]);
    }
#pragma unroll
    for (int c = 0; c < kNC; ++c)
#pragma unroll
      for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int v = 0; v < kNV; ++v) {
          if constexpr (kSz == 4)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, val[c][t][v]), orsrc,
                                                  vs[c] + so(si, t, v), 0, kAux);
          else
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, static_cast<OutT>(val[c][t][v])),
                                                  orsrc, vs[c] + so(si, t, v), 0, kAux);
        }
  }
}

template <class C>
int64_t tiles_of(int64_t M, int64_t N, int64_t batch, int64_t* tm, int64_t* tn) {
  *tm = (M + C::BM - 1) / C::BM;
  *tn = (N + C::BN - 1) / C::BN;
  return *tm * *tn * batch;
}

template <class C, class In, class OutT, bool ACC, bool A_MN, bool B_MN>
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
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_nt_kernel<C, In, OutT, ACC, A_MN, B_MN>),
                         dim3(static_cast<unsigned>(total)), dim3(C::NT), args, 0, stream);
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

template <class C, bool A_MN, bool B_MN>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  return with_types(p, [&](auto in, auto out, auto acc) {
    return launch<C, typename decltype(in)::type, typename decltype(out)::type, decltype(acc)::value, A_MN, B_MN>(
        p, stream);
  });
}

template <class C>
int64_t plan_tiles(int64_t M, int64_t N, int64_t batch) {
  int64_t tm, tn;
  return tiles_of<C>(M, N, batch, &tm, &tn);
}

// The 16x16 configuration for K-contiguous operands, its 32x32 twin otherwise.
template <class C16, class C32, bool A_MN, bool B_MN>
hipError_t launch_by_order(const GemmProblem& p, hipStream_t stream) {
  if constexpr (A_MN || B_MN) return launch_cfg<C32, A_MN, B_MN>(p, stream);
  else return launch_cfg<C16, A_MN, B_MN>(p, stream);
}

// Launch of one plan for one storage order of the operands.
template <bool A_MN, bool B_MN>
hipError_t launch_layout(GemmPlan plan, const GemmProblem& p, hipStream_t stream) {
  switch (plan) {
    case GemmPlan::kWave32: return launch_cfg<CfgWave32, A_MN, B_MN>(p, stream);
    case GemmPlan::kWg128x64: return launch_by_order<CfgWg128x64, CfgWg128x64Mn, A_MN, B_MN>(p, stream);
    case GemmPlan::kWg256: return launch_cfg<CfgWg256, A_MN, B_MN>(p, stream);
    case GemmPlan::kTall: return launch_cfg<CfgTall, A_MN, B_MN>(p, stream);
    case GemmPlan::kWg128x64Stream: return launch_cfg<CfgWg128x64Stream, A_MN, B_MN>(p, stream);
    case GemmPlan::kWg256x128: return launch_cfg<CfgWg256x128, A_MN, B_MN>(p, stream);
    case GemmPlan::kWg128x128: return launch_cfg<CfgWg128x128, A_MN, B_MN>(p, stream);
    case GemmPlan::kWide: return launch_cfg<CfgWide, A_MN, B_MN>(p, stream);
    case GemmPlan::kWg64: return launch_by_order<CfgWg64, CfgWg64Mn, A_MN, B_MN>(p, stream);
    default: return hipSuccess;
  }
}

}  // namespace
}  // namespace fp16mc
