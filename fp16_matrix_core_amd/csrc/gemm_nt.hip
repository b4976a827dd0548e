// gemm_nt.hip -- Out = A @ B.T, fp16 operands, fp32 accumulation, on gfx950.
//
// The operation is the one "Warp Matrix Instructions" and "Blackwell Tensor
// Cores" compute (Out = A @ B.T, K accumulated slice by slice into a fresh
// fp32 accumulator).  The data path is the same in spirit -- operand tiles
// staged in shared memory, moved into per-lane register fragments, multiplied
// by wavefront-collective matrix instructions -- laid out for CDNA4:
//
//   global -> LDS   each thread moves 16-byte chunks (8 fp16 of one row) with
//                   one global_load_dwordx4; 8 consecutive lanes cover one
//                   128-byte row segment, so a wavefront reads 8 full rows.
//   LDS layout      a BK = 64 slice of a row is 128 bytes = 8 chunks, placed
//                   by the XOR swizzle of layout.hpp (conflict-free for the
//                   row writes and for the fragment reads below).
//   LDS -> VGPR     one ds_read_b128 per lane per operand fragment: the 8
//                   consecutive-K fp16 that v_mfma_f32_32x32x16_f16 takes
//                   from each lane.  Both operands are K-contiguous (NT), so
//                   no transpose is needed.
//   MFMA            B's fragment is the instruction's first operand and A's
//                   the second, so the accumulator holds Out transposed:
//                   each lane owns 4 consecutive output columns of one row
//                   per 4 accumulator registers, stored with one 16-byte
//                   global store.
//   K loop          two LDS stages; the global loads of stage k+1 are issued
//                   before the MFMAs of stage k and land in LDS after them,
//                   one workgroup barrier per K step.
//   scheduler       XCD-contiguous ranges of tile ids, grouped so that the
//                   tiles an XCD runs together share A and B panels in L2.
//   edges           rows past M or N are clamped on load (their results are
//                   never stored); K past the end is zero-filled; the
//                   epilogue masks columns past N and rows past M.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"
#include "layout.hpp"

namespace fp16mc {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// BM x BN output tile per workgroup, WM x WN wavefronts, each owning a
// (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles.
template <int BM_, int BN_, int WM_, int WN_, int GROUP_M_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, GROUP_M = GROUP_M_;
  static constexpr int BK = 64;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int SI = WTM / 32, SJ = WTN / 32;
  static constexpr int A_STAGE = BM * lds_swizzle::kRowBytes;
  static constexpr int B_STAGE = BN * lds_swizzle::kRowBytes;
  static constexpr int ROWS_PER_PASS = NT / 8;  // rows covered by one 16-byte load per thread
  static constexpr int A_LOADS = BM / ROWS_PER_PASS;
  static constexpr int B_LOADS = BN / ROWS_PER_PASS;
  static constexpr int LDS_BYTES = 2 * (A_STAGE + B_STAGE);
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "rows must split evenly");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS is 160 KiB per CU");
};

using CfgWave32 = Cfg<32, 32, 1, 1, 1>;
using CfgWg128x64 = Cfg<128, 64, 4, 1, 8>;
using CfgWg256 = Cfg<256, 256, 2, 2, 4>;

// Elements [k, k+8) of a row, zero past K.  `row` points at element 0.
__device__ __forceinline__ u32x4 load_chunk(const _Float16* row, int64_t k, int64_t K) {
  if (k + 8 <= K) return *reinterpret_cast<const u32x4*>(row + k);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (k < K) {
    const unsigned short* r16 = reinterpret_cast<const unsigned short*>(row);
    unsigned int w[4] = {0u, 0u, 0u, 0u};
    for (int e = 0; e < 8; ++e) {
      if (k + e < K) w[e >> 1] |= static_cast<unsigned int>(r16[k + e]) << (16 * (e & 1));
    }
    v = u32x4{w[0], w[1], w[2], w[3]};
  }
  return v;
}

template <class C>
__global__ void __launch_bounds__(C::NT)
gemm_nt_kernel(const _Float16* __restrict__ A, const _Float16* __restrict__ B, float* __restrict__ Out,
               int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldo,
               int64_t sA, int64_t sB, int64_t sO, int64_t tiles_m, int64_t tiles_n, int64_t total) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN;
  const int wn = wave % C::WN;

  // ---- tile scheduler -------------------------------------------------------
  const int64_t lin = sched::xcd_remap(blockIdx.x, total);
  const int64_t per_problem = tiles_m * tiles_n;
  const int64_t b = lin / per_problem;
  const sched::Tile tile = sched::grouped_tile(lin - b * per_problem, tiles_m, tiles_n, C::GROUP_M);
  const int64_t i0 = tile.m * C::BM;
  const int64_t j0 = tile.n * C::BN;
  A += b * sA;
  B += b * sB;
  Out += b * sO;

  // ---- global -> LDS assignment: thread moves chunk `ch` of rows r0 + p*ROWS_PER_PASS
  const int ch = tid & 7;
  const int r0 = tid >> 3;
  const _Float16* a_src[C::A_LOADS];
  const _Float16* b_src[C::B_LOADS];
  int a_dst[C::A_LOADS];
  int b_dst[C::B_LOADS];
#pragma unroll
  for (int p = 0; p < C::A_LOADS; ++p) {
    const int r = r0 + p * C::ROWS_PER_PASS;
    const int64_t gi = (i0 + r < M) ? (i0 + r) : (M - 1);
    a_src[p] = A + gi * lda;
    a_dst[p] = lds_swizzle::offset_bytes(r, ch);
  }
#pragma unroll
  for (int p = 0; p < C::B_LOADS; ++p) {
    const int r = r0 + p * C::ROWS_PER_PASS;
    const int64_t gj = (j0 + r < N) ? (j0 + r) : (N - 1);
    b_src[p] = B + gj * ldb;
    b_dst[p] = lds_swizzle::offset_bytes(r, ch);
  }

  u32x4 ra[C::A_LOADS];
  u32x4 rb[C::B_LOADS];
  auto global_load = [&](int64_t k0) {
    const int64_t k = k0 + 8 * ch;
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) ra[p] = load_chunk(a_src[p], k, K);
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) rb[p] = load_chunk(b_src[p], k, K);
  };
  auto lds_store = [&](int stage) {
    unsigned char* as = smem + stage * C::A_STAGE;
    unsigned char* bs = smem + 2 * C::A_STAGE + stage * C::B_STAGE;
#pragma unroll
    for (int p = 0; p < C::A_LOADS; ++p) *reinterpret_cast<u32x4*>(as + a_dst[p]) = ra[p];
#pragma unroll
    for (int p = 0; p < C::B_LOADS; ++p) *reinterpret_cast<u32x4*>(bs + b_dst[p]) = rb[p];
  };

  // ---- fragment reads + MFMA ------------------------------------------------
  f32x16 acc[C::SI][C::SJ];
#pragma unroll
  for (int si = 0; si < C::SI; ++si)
#pragma unroll
    for (int sj = 0; sj < C::SJ; ++sj) acc[si][sj] = f32x16{};

  const int frow = mfma32::operand_row(lane);      // row inside a 32-row MFMA tile
  const int khalf = lane >> 5;                     // which 8-wide K group of a 16-K step
  const int key = lds_swizzle::key(frow);          // equal to key(row) for every fragment row
  const int a_row0 = (wm * C::WTM + frow) * lds_swizzle::kRowBytes;
  const int b_row0 = (wn * C::WTN + frow) * lds_swizzle::kRowBytes;

  auto compute = [&](int stage) {
    const unsigned char* as = smem + stage * C::A_STAGE + a_row0;
    const unsigned char* bs = smem + 2 * C::A_STAGE + stage * C::B_STAGE + b_row0;
#pragma unroll
    for (int kk = 0; kk < C::BK / mfma32::kK; ++kk) {
      const int pc = ((2 * kk + khalf) ^ key) << 4;
      f16x8 af[C::SI];
      f16x8 bf[C::SJ];
#pragma unroll
      for (int si = 0; si < C::SI; ++si)
        af[si] = *reinterpret_cast<const f16x8*>(as + si * 32 * lds_swizzle::kRowBytes + pc);
#pragma unroll
      for (int sj = 0; sj < C::SJ; ++sj)
        bf[sj] = *reinterpret_cast<const f16x8*>(bs + sj * 32 * lds_swizzle::kRowBytes + pc);
#pragma unroll
      for (int si = 0; si < C::SI; ++si)
#pragma unroll
        for (int sj = 0; sj < C::SJ; ++sj)
          acc[si][sj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[sj], af[si], acc[si][sj], 0, 0, 0);
    }
  };

  // ---- K loop: two LDS stages, one barrier per step ---------------------------
  const int64_t nk = (K + C::BK - 1) / C::BK;
  if (nk > 0) {
    global_load(0);
    lds_store(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
      const int stage = static_cast<int>(kt & 1);
      const bool more = kt + 1 < nk;
      if (more) global_load((kt + 1) * C::BK);
      compute(stage);
      if (more) lds_store(stage ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: accumulator (Out transposed) -> fp32 rows ---------------------
  // Element v = 4q + e of lane l in tile (si, sj) is Out[i][j] with
  // i = i0 + wm*WTM + 32 si + l%32 and j = j0 + wn*WTN + 32 sj + 8q + 4(l/32) + e.
#pragma unroll
  for (int si = 0; si < C::SI; ++si) {
    const int64_t i = i0 + wm * C::WTM + si * 32 + mfma32::acc_col(lane, 0);
    if (i >= M) continue;
    float* orow = Out + i * ldo;
#pragma unroll
    for (int sj = 0; sj < C::SJ; ++sj) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t j = j0 + wn * C::WTN + sj * 32 + mfma32::acc_row(lane, 4 * q);
        const f32x4 v = {acc[si][sj][4 * q], acc[si][sj][4 * q + 1], acc[si][sj][4 * q + 2],
                         acc[si][sj][4 * q + 3]};
        if (j + 4 <= N) {
          *reinterpret_cast<f32x4*>(orow + j) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < N) orow[j + e] = v[e];
        }
      }
    }
  }
}

template <class C>
int64_t tiles_of(int64_t M, int64_t N, int64_t batch, int64_t* tm, int64_t* tn) {
  *tm = (M + C::BM - 1) / C::BM;
  *tn = (N + C::BN - 1) / C::BN;
  return *tm * *tn * batch;
}

template <class C>
hipError_t launch(const GemmProblem& p, hipStream_t stream) {
  int64_t tm, tn;
  const int64_t total = tiles_of<C>(p.M, p.N, p.batch, &tm, &tn);
  const _Float16* A = static_cast<const _Float16*>(p.A);
  const _Float16* B = static_cast<const _Float16*>(p.B);
  float* Out = p.Out;
  int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb, ldo = p.ldo;
  int64_t sA = p.sA, sB = p.sB, sO = p.sO;
  void* args[] = {&A, &B, &Out, &M, &N, &K, &lda, &ldb, &ldo, &sA, &sB, &sO, &tm, &tn,
                  const_cast<int64_t*>(&total)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_nt_kernel<C>),
                         dim3(static_cast<unsigned>(total)), dim3(C::NT), args, 0, stream);
}

}  // namespace

GemmPlan choose_gemm_plan(int64_t M, int64_t N, int64_t /*K*/, int64_t batch) {
  if (M <= 0 || N <= 0 || batch <= 0) return GemmPlan::kNone;
  if (M <= 32 && N <= 32) return GemmPlan::kWave32;
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
    default: return nullptr;
  }
}

int64_t gemm_plan_grid(GemmPlan plan, int64_t M, int64_t N, int64_t batch) {
  int64_t tm, tn;
  switch (plan) {
    case GemmPlan::kWave32: return tiles_of<CfgWave32>(M, N, batch, &tm, &tn);
    case GemmPlan::kWg128x64: return tiles_of<CfgWg128x64>(M, N, batch, &tm, &tn);
    case GemmPlan::kWg256: return tiles_of<CfgWg256>(M, N, batch, &tm, &tn);
    default: return 0;
  }
}

hipError_t launch_gemm(GemmPlan plan, const GemmProblem& p, hipStream_t stream) {
  switch (plan) {
    case GemmPlan::kWave32: return launch<CfgWave32>(p, stream);
    case GemmPlan::kWg128x64: return launch<CfgWg128x64>(p, stream);
    case GemmPlan::kWg256: return launch<CfgWg256>(p, stream);
    default: return hipSuccess;
  }
}

}  // namespace fp16mc
