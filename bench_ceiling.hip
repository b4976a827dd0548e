// bench_ceiling.hip -- two ceilings that bench.py reports beside the product's
// figures (measurement only; not part of libfp16mc.so):
//
//   ceiling_mfma  what the matrix pipe sustains on its own: each wavefront
//                 loads one set of operand fragments and then issues nothing
//                 but independent MFMAs on them, into the same 256 fp32
//                 accumulators per lane that the 256x256 product tile uses
//                 (8x8 tiles of 16x16x32, or 4x4 tiles of 32x32x16).  No LDS
//                 and no memory traffic inside the loop.  Fed with the
//                 product's own operand values it shows how far the operand
//                 data alone pulls the clock down (the chip is power-limited
//                 with random operands); fed with zeros, the issue-rate peak.
//   ceiling_copy  a plain 16-byte copy with non-temporal loads and stores,
//                 in four access shapes: what the memory system gives a
//                 pure streaming kernel of the same size as a fragment copy
//                 (the best shape differs from box to box by a few percent).
//   ceiling_stream  a read/write stream with the batched product's mix per
//                 workgroup (its operands read, its output written once).
//
// One workgroup of four wavefronts per CU for the MFMA loop (a 256-register
// accumulator leaves room for one wavefront per SIMD).

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int MI>
struct Shape;
template <>
struct Shape<16> {
  static constexpr int T = 8;   // 8x8 tiles of 16x16 = a 128x128 wave tile
  typedef f32x4 Acc;
  static __device__ __forceinline__ Acc mma(f16x8 a, f16x8 b, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Shape<32> {
  static constexpr int T = 4;   // 4x4 tiles of 32x32 = a 128x128 wave tile
  typedef f32x16 Acc;
  static __device__ __forceinline__ Acc mma(f16x8 a, f16x8 b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Wavefront w reads fragments 2T*w .. 2T*w + 2T-1 (16 bytes per lane each):
// T for the first operand, T for the second.
template <int MI>
__global__ void __launch_bounds__(256, 1) mfma_loop(const f16x8* __restrict__ ops, float* __restrict__ sink,
                                                    int iters) {
  using S = Shape<MI>;
  constexpr int T = S::T;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  f16x8 a[T], b[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    a[t] = ops[(static_cast<int64_t>(w) * 2 * T + t) * 64 + lane];
    b[t] = ops[(static_cast<int64_t>(w) * 2 * T + T + t) * 64 + lane];
  }
  typename S::Acc acc[T][T];
#pragma unroll
  for (int i = 0; i < T; ++i)
#pragma unroll
    for (int j = 0; j < T; ++j) acc[i][j] = typename S::Acc{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < T; ++i)
#pragma unroll
      for (int j = 0; j < T; ++j) acc[i][j] = S::mma(a[i], b[j], acc[i][j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < T; ++i)
#pragma unroll
    for (int j = 0; j < T; ++j)
#pragma unroll
      for (int v = 0; v < static_cast<int>(sizeof(typename S::Acc) / 4); ++v) s += acc[i][j][v];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

// Each thread copies D chunks of 16 bytes, T chunks apart (T threads per
// workgroup, T*D chunks per workgroup); n16 is a multiple of 4096.
template <int D, int T>
__global__ void __launch_bounds__(T) copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * T * D + threadIdx.x;
  u32x4 v[D];
#pragma unroll
  for (int k = 0; k < D; ++k) v[k] = __builtin_nontemporal_load(src + base + T * k);
#pragma unroll
  for (int k = 0; k < D; ++k) __builtin_nontemporal_store(v[k], dst + base + T * k);
}

// Units of work that each read rd16 16-byte chunks of their source span and
// write wr16 chunks of their destination span (both non-temporal), the same
// read/write mix per unit as a batched product whose problems each read A and
// B and write their output once.  Workgroups take units grid-stride.  With
// OVERLAP false a unit's written values derive from its own reads (the
// product's dependence: its writes wait for its reads); with OVERLAP true
// they carry the workgroup's previous unit's values, so that a unit's reads
// and writes can be in flight together.  Either way no load is dropped.
template <bool OVERLAP>
__global__ void __launch_bounds__(256) stream_mix(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                  int rd16, int wr16, int64_t units) {
  u32x4 prev = {0u, 0u, 0u, 0u};
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const u32x4* s = src + u * rd16;
    u32x4* d = dst + u * wr16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int i = threadIdx.x; i < rd16; i += 256) acc ^= __builtin_nontemporal_load(s + i);
    const u32x4 w = OVERLAP ? prev : acc;
    for (int i = threadIdx.x; i < wr16; i += 256) __builtin_nontemporal_store(w + static_cast<unsigned>(i), d + i);
    prev = acc;
  }
  if (OVERLAP && prev[0] == 0x9E3779B9u && prev[1] == 0x7F4A7C15u) dst[threadIdx.x] = prev;  // keep the last reads live
}

}  // namespace

extern "C" {

// Operand buffer of ops_bytes: 16 KiB per wavefront with 16x16 tiles, 8 KiB
// with 32x32 (grid * 4 wavefronts); sink: grid * 256 floats.  Returns 0, -1
// for bad arguments (nothing launched) or a HIP error.
int ceiling_mfma(const void* ops, int64_t ops_bytes, float* sink, int mi, int iters, int grid, void* stream) {
  if (grid <= 0 || iters <= 0 || (mi != 16 && mi != 32)) return -1;
  if (ops_bytes < static_cast<int64_t>(grid) * 4 * (mi == 16 ? 16384 : 8192)) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mi == 16)
    hipLaunchKernelGGL(mfma_loop<16>, dim3(grid), dim3(256), 0, s, static_cast<const f16x8*>(ops), sink, iters);
  else
    hipLaunchKernelGGL(mfma_loop<32>, dim3(grid), dim3(256), 0, s, static_cast<const f16x8*>(ops), sink, iters);
  return static_cast<int>(hipGetLastError());
}

// Copies `bytes` (a multiple of 64 KiB) from src to dst, both 16-byte aligned,
// with one of four access shapes (chunks per thread x threads per workgroup:
// 0: 1 x 512, 1: 2 x 256, 2: 4 x 256, 3: 1 x 256); -1 for bad arguments.
int ceiling_copy(const void* src, void* dst, int64_t bytes, int shape, void* stream) {
  if (bytes <= 0 || bytes % 65536 != 0 || shape < 0 || shape > 3) return -1;
  const int64_t n16 = bytes / 16;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (shape) {
    case 0: hipLaunchKernelGGL((copy16<1, 512>), dim3(static_cast<unsigned>(n16 / 512)), dim3(512), 0, st, s, d, n16); break;
    case 1: hipLaunchKernelGGL((copy16<2, 256>), dim3(static_cast<unsigned>(n16 / 512)), dim3(256), 0, st, s, d, n16); break;
    case 2: hipLaunchKernelGGL((copy16<4, 256>), dim3(static_cast<unsigned>(n16 / 1024)), dim3(256), 0, st, s, d, n16); break;
    default: hipLaunchKernelGGL((copy16<1, 256>), dim3(static_cast<unsigned>(n16 / 256)), dim3(256), 0, st, s, d, n16); break;
  }
  return static_cast<int>(hipGetLastError());
}

// `units` units, each reading rd_bytes from src + u*rd_bytes and writing
// wr_bytes to dst + u*wr_bytes (both multiples of 16), taken by `grid`
// workgroups (0: one per unit), overlapped or not (see stream_mix); -1 for
// bad arguments.
int ceiling_stream(const void* src, void* dst, int units, int rd_bytes, int wr_bytes, int grid, int overlap,
                   void* stream) {
  if (units <= 0 || rd_bytes <= 0 || wr_bytes <= 0 || rd_bytes % 16 != 0 || wr_bytes % 16 != 0 || grid < 0 ||
      wr_bytes < 256 * 16 * (overlap != 0))
    return -1;
  const dim3 g(static_cast<unsigned>(grid == 0 || grid > units ? units : grid));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  if (overlap)
    hipLaunchKernelGGL(stream_mix<true>, g, dim3(256), 0, st, s, d, rd_bytes / 16, wr_bytes / 16, static_cast<int64_t>(units));
  else
    hipLaunchKernelGGL(stream_mix<false>, g, dim3(256), 0, st, s, d, rd_bytes / 16, wr_bytes / 16, static_cast<int64_t>(units));
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
