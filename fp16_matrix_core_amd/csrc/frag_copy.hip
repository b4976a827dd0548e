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
// Each wavefront walks blocks of 1 KiB of groups on its own (no workgroup
// barrier).  Both sides of a block are contiguous 1 KiB spans in HBM: the
// image, and the fragments stored lane-major (group, lane, num words).  The
// kernel is HBM-bound: 128 bytes read and 128 bytes written per tile.  Every
// HBM access is non-temporal (each byte is touched once; measured +8-11%
// over cached accesses), and up to 16384 workgroups of eight wavefronts
// cover the 2^20-tile workload's 131072 blocks in one pass.

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

constexpr int kThreads = 512;                 // eight wavefronts per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kWaveBytes = 1024;              // image (and fragment) bytes a wavefront moves per step
constexpr int kWaveChunks = kWaveBytes / 16;  // one 16-byte chunk per lane
constexpr int kMaxGrid = 16384;

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

#define FP16MC_FRAG_INLINE __attribute__((always_inline))

// The wavefront's LDS writes become visible to its own later reads: LDS
// executes a wavefront's instructions in order; the wait and the compiler
// barrier keep the reads of other lanes' words behind the writes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), other counters untouched
  asm volatile("" ::: "memory");
}

// DIR: 0 load (image -> fragment), 1 store (fragment -> image), 2 roundtrip.
// Every wavefront works alone on its own 1 KiB spans: wave block w holds
// groups [w * 8/NUM, (w+1) * 8/NUM) -- 1 KiB of image and 1 KiB of fragments
// (lane-major, group after group), both contiguous in HBM.  Each lane moves
// one 16-byte chunk of the source span into the wavefront's LDS region, the
// two half-waves rebuild their groups' other side in a second region (the
// words each lane owns: ds_read/ds_write of 4-byte words for row-major
// images, b16 pairs for column-major ones), and each lane stores one 16-byte
// chunk of the result.  No workgroup barrier: every wavefront streams as a
// plain copy would (the access shape of the fastest plain copy measured on
// gfx950: one 16-byte chunk per lane, 512-thread workgroups, every access
// non-temporal), instead of each workgroup waiting for all of its 8 KiB to
// arrive before any of it leaves.
template <int NUM, bool COL, int DIR>
__global__ void __launch_bounds__(kThreads)
frag_copy_kernel(const void* __restrict__ src, void* __restrict__ dst, int64_t groups, int64_t nwblocks) {
  constexpr int kGroupBytes = 128 * NUM;
  constexpr int kGroupsPerWave = kWaveBytes / kGroupBytes;
  constexpr int kGroupHalves = 64 * NUM;
  typedef typename Words<NUM>::T W;

  __shared__ __attribute__((aligned(16))) u32x4 lds[kWaves][2][kWaveChunks];   // per wavefront: source, result

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int hw = lane >> 5;  // half-wave: one 32-lane fragment at a time
  u32x4* in = lds[wave][0];
  u32x4* out = lds[wave][1];
  unsigned short* in_img = reinterpret_cast<unsigned short*>(in);
  unsigned short* out_img = reinterpret_cast<unsigned short*>(out);

  for (int64_t wb = static_cast<int64_t>(blockIdx.x) * kWaves + wave; wb < nwblocks;
       wb += static_cast<int64_t>(gridDim.x) * kWaves) {
    const int64_t g0 = wb * kGroupsPerWave;
    const int ng = static_cast<int>((groups - g0) < kGroupsPerWave ? (groups - g0) : kGroupsPerWave);
    const int nchunks = ng * (kGroupBytes / 16);
    const u32x4* s = static_cast<const u32x4*>(src) + g0 * (kGroupBytes / 16);
    u32x4* d = static_cast<u32x4*>(dst) + g0 * (kGroupBytes / 16);
    if (lane < nchunks) in[lane] = __builtin_nontemporal_load(s + lane);
    wave_lds_sync();
    // A lane's words of group lg: read from the source region, then
    // written to the result region.  In a full block all reads come first
    // (one wait for all of them), then all writes.
    auto get = [&](int lg) FP16MC_FRAG_INLINE {
      W v;
      if constexpr (DIR == 1) {
        v = reinterpret_cast<const W*>(in)[lg * 32 + l32];
      } else {
#pragma unroll
        for (int t = 0; t < NUM; ++t) Words<NUM>::set(v, t, lds_read_word<NUM, COL>(in_img + lg * kGroupHalves, l32, t));
      }
      return v;
    };
    auto put = [&](int lg, const W& v) FP16MC_FRAG_INLINE {
      if constexpr (DIR == 0) {
        reinterpret_cast<W*>(out)[lg * 32 + l32] = v;
      } else {
#pragma unroll
        for (int t = 0; t < NUM; ++t) lds_write_word<NUM, COL>(out_img + lg * kGroupHalves, l32, t, Words<NUM>::get(v, t));
      }
    };
    if (ng == kGroupsPerWave) {
      constexpr int kIt = kGroupsPerWave / 2;   // groups per half-wave
      W v[kIt];
#pragma unroll
      for (int i = 0; i < kIt; ++i) v[i] = get(hw + 2 * i);
#pragma unroll
      for (int i = 0; i < kIt; ++i) put(hw + 2 * i, v[i]);
    } else {
      for (int lg = hw; lg < ng; lg += 2) put(lg, get(lg));
    }
    wave_lds_sync();
    if (lane < nchunks) __builtin_nontemporal_store(out[lane], d + lane);
    wave_lds_sync();   // this step's reads of both regions precede the next step's writes
  }
}

template <int NUM, bool COL, int DIR>
hipError_t launch_one(const void* src, void* dst, int64_t groups, hipStream_t stream) {
  constexpr int kGroupsPerWave = kWaveBytes / (128 * NUM);
  int64_t nwblocks = (groups + kGroupsPerWave - 1) / kGroupsPerWave;
  const int64_t blocks = (nwblocks + kWaves - 1) / kWaves;
  const int64_t grid = blocks < kMaxGrid ? blocks : kMaxGrid;
  void* args[] = {const_cast<void**>(&src), &dst, &groups, &nwblocks};
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
