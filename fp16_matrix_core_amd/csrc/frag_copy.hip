// frag_copy.hip -- the 8x8 b16 matrix load/store between shared memory and
// the per-lane register fragment ("copy -> ldstmatrix": demonstration program,
// Algorithm steps 2-4, "How inputs change the algorithm"), on gfx950.
//
// CDNA4 has no single warp-collective instruction that performs this
// shuffle, so each lane reads (or writes) exactly the LDS words its fragment
// owns:
//   row-major image     the two b16 of a word are adjacent and 4-byte
//                       aligned: one ds_read_b32 / ds_write_b32 per word;
//   column-major image  the two b16 of a word sit one column (8 elements)
//                       apart: a ds_read_u16 pair / ds_write_b16 pair.
// One 64-lane wavefront carries two 32-lane fragments (lanes [0,32) and
// [32,64)), i.e. two consecutive groups.
//
// Each workgroup walks blocks of 8 KiB of groups.  Both sides of a block
// are contiguous 8 KiB spans in HBM: the image, and the fragments stored
// lane-major (group, lane, num words).  The kernel is HBM-bound: 128 bytes
// read and 128 bytes written per tile.  Every HBM access is
// non-temporal (each byte is touched once; measured +8-11% over cached
// accesses), and up to 16384 workgroups cover the 2^20-tile workload's 16384
// blocks in one pass.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"
#include "layout.hpp"

namespace fp16mc {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int NUM>
struct Words;
template <>
struct Words<1> {
  typedef unsigned int T;
  static __device__ __forceinline__ unsigned int get(const T& v, int) { return v; }
  static __device__ __forceinline__ void set(T& v, int, unsigned int w) { v = w; }
};
template <>
struct Words<2> {
  typedef u32x2 T;
  static __device__ __forceinline__ unsigned int get(const T& v, int t) { return v[t]; }
  static __device__ __forceinline__ void set(T& v, int t, unsigned int w) { v[t] = w; }
};
template <>
struct Words<4> {
  typedef u32x4 T;
  static __device__ __forceinline__ unsigned int get(const T& v, int t) { return v[t]; }
  static __device__ __forceinline__ void set(T& v, int t, unsigned int w) { v[t] = w; }
};

constexpr int kThreads = 256;
constexpr int kBlockBytes = 8 * 1024;
constexpr int kBlockChunks = kBlockBytes / 16;
constexpr int kHalfWaves = kThreads / 32;

// Word t of the fragment of lane `l32` (0..31), read from a group image in LDS.
template <int NUM, bool COL>
__device__ __forceinline__ unsigned int lds_read_word(const unsigned short* img, int l32, int t) {
  const int r = m8n8::row(l32);
  const int c = 2 * m8n8::col_pair(l32);
  if constexpr (!COL) {
    return *reinterpret_cast<const unsigned int*>(img + m8n8::image_offset(false, NUM, r, c, t));
  } else {
    const unsigned int lo = img[m8n8::image_offset(true, NUM, r, c, t)];
    const unsigned int hi = img[m8n8::image_offset(true, NUM, r, c + 1, t)];
    return lo | (hi << 16);
  }
}

template <int NUM, bool COL>
__device__ __forceinline__ void lds_write_word(unsigned short* img, int l32, int t, unsigned int w) {
  const int r = m8n8::row(l32);
  const int c = 2 * m8n8::col_pair(l32);
  if constexpr (!COL) {
    *reinterpret_cast<unsigned int*>(img + m8n8::image_offset(false, NUM, r, c, t)) = w;
  } else {
    img[m8n8::image_offset(true, NUM, r, c, t)] = static_cast<unsigned short>(w & 0xFFFFu);
    img[m8n8::image_offset(true, NUM, r, c + 1, t)] = static_cast<unsigned short>(w >> 16);
  }
}

// DIR: 0 load (image -> fragment), 1 store (fragment -> image), 2 roundtrip.
// The image side of a block always moves between HBM and LDS with 16-byte
// accesses.  Its fragment side (group g holds 32 lanes of NUM words) is as
// contiguous: the load direction stages it in LDS as well and writes it with
// 16-byte stores (num = 1 and 2 would otherwise store 4 or 8 bytes per
// lane; measured +1-2%), while the store direction reads it straight into
// the lanes' registers, every fragment of the block in flight at once
// (staging it measured 1-3% slower there).
template <int NUM, bool COL, int DIR>
__global__ void __launch_bounds__(kThreads)
frag_copy_kernel(const void* __restrict__ src, void* __restrict__ dst, int64_t groups, int64_t nblocks) {
  constexpr int kGroupBytes = 128 * NUM;
  constexpr int kGroupsPerBlock = kBlockBytes / kGroupBytes;
  constexpr int kGroupHalves = 64 * NUM;
  typedef typename Words<NUM>::T W;

  __shared__ __attribute__((aligned(16))) u32x4 lds_a[kBlockChunks];                  // image
  __shared__ __attribute__((aligned(16))) u32x4 lds_b[DIR == 1 ? 1 : kBlockChunks];   // fragments / 2nd image

  const int tid = threadIdx.x;
  const int l32 = tid & 31;
  const int hw = tid >> 5;  // half-wave: one 32-lane fragment at a time
  unsigned short* img = reinterpret_cast<unsigned short*>(lds_a);

  for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
    const int64_t g0 = blk * kGroupsPerBlock;
    const int ng = static_cast<int>((groups - g0) < kGroupsPerBlock ? (groups - g0) : kGroupsPerBlock);
    const int nchunks = ng * (kGroupBytes / 16);
    u32x4* d = static_cast<u32x4*>(dst) + g0 * (kGroupBytes / 16);

    if constexpr (DIR == 0 || DIR == 2) {
      // image: HBM -> LDS
      const u32x4* s = static_cast<const u32x4*>(src) + g0 * (kGroupBytes / 16);
      for (int c = tid; c < nchunks; c += kThreads) lds_a[c] = __builtin_nontemporal_load(s + c);
      __syncthreads();
      // image -> registers -> fragments (lane-major) or the second image, in LDS
      for (int lg = hw; lg < ng; lg += kHalfWaves) {
        W v;
#pragma unroll
        for (int t = 0; t < NUM; ++t) Words<NUM>::set(v, t, lds_read_word<NUM, COL>(img + lg * kGroupHalves, l32, t));
        if constexpr (DIR == 0) {
          reinterpret_cast<W*>(lds_b)[lg * 32 + l32] = v;
        } else {
          unsigned short* out = reinterpret_cast<unsigned short*>(lds_b) + lg * kGroupHalves;
#pragma unroll
          for (int t = 0; t < NUM; ++t) lds_write_word<NUM, COL>(out, l32, t, Words<NUM>::get(v, t));
        }
      }
      __syncthreads();
      for (int c = tid; c < nchunks; c += kThreads) __builtin_nontemporal_store(lds_b[c], d + c);
      __syncthreads();
    } else {
      // fragment: HBM -> VGPR -> LDS image.  In a full block every half-wave
      // loads all its fragments before writing any, so that its loads (num
      // words per lane each) are in flight together.
      const W* frag = static_cast<const W*>(src) + g0 * 32 + l32;
      if (ng == kGroupsPerBlock) {
        constexpr int kIt = kGroupsPerBlock / kHalfWaves;
        W v[kIt];
#pragma unroll
        for (int i = 0; i < kIt; ++i) v[i] = __builtin_nontemporal_load(frag + (hw + i * kHalfWaves) * 32);
#pragma unroll
        for (int i = 0; i < kIt; ++i)
#pragma unroll
          for (int t = 0; t < NUM; ++t)
            lds_write_word<NUM, COL>(img + (hw + i * kHalfWaves) * kGroupHalves, l32, t, Words<NUM>::get(v[i], t));
      } else {
        for (int lg = hw; lg < ng; lg += kHalfWaves) {
          const W v = __builtin_nontemporal_load(frag + lg * 32);
#pragma unroll
          for (int t = 0; t < NUM; ++t) lds_write_word<NUM, COL>(img + lg * kGroupHalves, l32, t, Words<NUM>::get(v, t));
        }
      }
      __syncthreads();
      // image: LDS -> HBM
      for (int c = tid; c < nchunks; c += kThreads) __builtin_nontemporal_store(lds_a[c], d + c);
      __syncthreads();
    }
  }
}

template <int NUM, bool COL, int DIR>
hipError_t launch_one(const void* src, void* dst, int64_t groups, hipStream_t stream) {
  constexpr int kGroupsPerBlock = kBlockBytes / (128 * NUM);
  int64_t nblocks = (groups + kGroupsPerBlock - 1) / kGroupsPerBlock;
  const int64_t grid = nblocks < 16384 ? nblocks : 16384;
  void* args[] = {const_cast<void**>(&src), &dst, &groups, &nblocks};
  return hipLaunchKernel(reinterpret_cast<const void*>(&frag_copy_kernel<NUM, COL, DIR>),
                         dim3(static_cast<unsigned>(grid)), dim3(kThreads), args, 0, stream);
}

template <int NUM, bool COL>
hipError_t launch_dir(const void* src, void* dst, int64_t groups, int dir, hipStream_t stream) {
  switch (dir) {
    case 0: return launch_one<NUM, COL, 0>(src, dst, groups, stream);
    case 1: return launch_one<NUM, COL, 1>(src, dst, groups, stream);
    default: return launch_one<NUM, COL, 2>(src, dst, groups, stream);
  }
}

template <int NUM>
hipError_t launch_num(const void* src, void* dst, int64_t groups, bool col, int dir, hipStream_t stream) {
  return col ? launch_dir<NUM, true>(src, dst, groups, dir, stream)
             : launch_dir<NUM, false>(src, dst, groups, dir, stream);
}

}  // namespace

hipError_t launch_frag_copy(const void* src, void* dst, int64_t groups, int num, bool col_major,
                            int direction, hipStream_t stream) {
  if (groups <= 0) return hipSuccess;
  switch (num) {
    case 1: return launch_num<1>(src, dst, groups, col_major, direction, stream);
    case 2: return launch_num<2>(src, dst, groups, col_major, direction, stream);
    default: return launch_num<4>(src, dst, groups, col_major, direction, stream);
  }
}

}  // namespace fp16mc
