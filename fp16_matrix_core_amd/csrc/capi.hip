// capi.hip -- the extern "C" boundary of libfp16mc.so (declared in fp16mc.h).
//
// Every argument is checked on the host before any HIP call; a failed check
// returns a negative status and records a message for fp16mc_last_error().
// Each message names the argument and the rule it breaks, as the matrix-load
// lowering reports why a copy does not fit ("copy -> ldstmatrix", "What it
// accepts" and "Algorithm" step 3).  Launches go through
// hipLaunchKernel, whose return code becomes FP16MC_EHIP on failure.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/fp16mc.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return FP16MC_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The tile scheduler works in 32-bit arithmetic (grid x group strip < 2^32).
constexpr int64_t kMaxGrid = int64_t(1) << 28;

static_assert(static_cast<int>(fp16mc::Dtype::kF32) == FP16MC_F32 &&
                  static_cast<int>(fp16mc::Dtype::kF16) == FP16MC_F16 &&
                  static_cast<int>(fp16mc::Dtype::kBF16) == FP16MC_BF16,
              "internal element-type codes must match fp16mc.h");

int check_gemm(const void* A, const void* B, const void* Out, int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int64_t ldo, int64_t batch, int64_t sA, int64_t sB,
               int64_t sO, int a_order, int b_order, int ab_type, int out_type, int accumulate) {
  if ((a_order != FP16MC_K_CONTIGUOUS && a_order != FP16MC_MN_CONTIGUOUS) ||
      (b_order != FP16MC_K_CONTIGUOUS && b_order != FP16MC_MN_CONTIGUOUS))
    return fail(FP16MC_EINVAL, "a_order=%d and b_order=%d must be FP16MC_K_CONTIGUOUS or FP16MC_MN_CONTIGUOUS",
                a_order, b_order);
  if (ab_type != FP16MC_F16 && ab_type != FP16MC_BF16)
    return fail(FP16MC_EINVAL, "ab_type=%d must be FP16MC_F16 or FP16MC_BF16", ab_type);
  if (out_type != FP16MC_F32 && out_type != ab_type)
    return fail(FP16MC_EINVAL, "out_type=%d must be FP16MC_F32 or the operands' type %d", out_type, ab_type);
  if (accumulate != 0 && accumulate != 1) return fail(FP16MC_EINVAL, "accumulate must be 0 or 1");
  if (M < 0 || N < 0 || K < 0) return fail(FP16MC_EINVAL, "negative size (M=%lld, N=%lld, K=%lld)",
                                           (long long)M, (long long)N, (long long)K);
  if (batch < 0) return fail(FP16MC_EINVAL, "negative batch %lld", (long long)batch);
  const bool a_mn = a_order == FP16MC_MN_CONTIGUOUS, b_mn = b_order == FP16MC_MN_CONTIGUOUS;
  if (!a_mn && lda < K) return fail(FP16MC_EINVAL, "lda=%lld < K=%lld", (long long)lda, (long long)K);
  if (a_mn && lda < M) return fail(FP16MC_EINVAL, "lda=%lld < M=%lld (A stored K x M)", (long long)lda, (long long)M);
  if (!b_mn && ldb < K) return fail(FP16MC_EINVAL, "ldb=%lld < K=%lld", (long long)ldb, (long long)K);
  if (b_mn && ldb < N) return fail(FP16MC_EINVAL, "ldb=%lld < N=%lld (B stored K x N)", (long long)ldb, (long long)N);
  if (ldo < N) return fail(FP16MC_EINVAL, "ldo=%lld < N=%lld", (long long)ldo, (long long)N);
  if (sA < 0 || sB < 0 || sO < 0) return fail(FP16MC_EINVAL, "negative batch stride");
  const bool live = M > 0 && N > 0 && batch > 0;
  if (!live) return FP16MC_OK;
  if (K > 0 && (A == nullptr || B == nullptr)) return fail(FP16MC_EINVAL, "A or B is NULL");
  if (Out == nullptr) return fail(FP16MC_EINVAL, "Out is NULL");
  if (batch > 1) {
    // Problem b starts b * stride elements in: the last one's byte offset must be representable.
    const int64_t s_ab = sA > sB ? sA : sB;
    int64_t last = 0;
    if (__builtin_mul_overflow(batch - 1, s_ab, &last) || __builtin_mul_overflow(last, int64_t(2), &last) ||
        __builtin_mul_overflow(batch - 1, sO, &last) || __builtin_mul_overflow(last, int64_t(4), &last))
      return fail(FP16MC_EINVAL, "batch=%lld with these strides overflows 64-bit offsets", (long long)batch);
  }
  // Problems that shared output cells would race on them.
  if (batch > 1) {
    int64_t span = 0;
    if (__builtin_mul_overflow(M - 1, ldo, &span) || __builtin_add_overflow(span, N, &span))
      return fail(FP16MC_EINVAL, "M=%lld rows of ldo=%lld elements overflow 64-bit offsets", (long long)M,
                  (long long)ldo);
    if (sO < span)
      return fail(FP16MC_EINVAL, "strideO=%lld lets the problems' outputs overlap (at least (M-1)*ldo+N = %lld)",
                  (long long)sO, (long long)span);
  }
  if (!aligned16(A) || !aligned16(B))
    return fail(FP16MC_EALIGN, "A and B must be 16-byte aligned (8 fp16 per access)");
  if ((lda & 7) || (ldb & 7))
    return fail(FP16MC_EALIGN, "lda=%lld and ldb=%lld must be multiples of 8 (16-byte rows)",
                (long long)lda, (long long)ldb);
  const int64_t per16 = out_type == FP16MC_F32 ? 4 : 8;  // output elements per 16 bytes
  if (!aligned16(Out) || (ldo % per16))
    return fail(FP16MC_EALIGN, "Out must be 16-byte aligned and ldo=%lld a multiple of %lld", (long long)ldo,
                (long long)per16);
  if (batch > 1 && ((sA & 7) || (sB & 7) || (sO % per16)))
    return fail(FP16MC_EALIGN, "batch strides must keep 16-byte alignment (sA, sB %% 8, sO %% %lld)",
                (long long)per16);
  return FP16MC_OK;
}

}  // namespace

extern "C" {

int gemm_ex(const void* A, const void* B, void* Out, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
            int64_t ldo, int64_t batch, int64_t strideA, int64_t strideB, int64_t strideO, int a_order,
            int b_order, int ab_type, int out_type, int accumulate, void* stream) {
  const int rc = check_gemm(A, B, Out, M, N, K, lda, ldb, ldo, batch, strideA, strideB, strideO, a_order,
                            b_order, ab_type, out_type, accumulate);
  if (rc != FP16MC_OK) return rc;
  const bool a_mn = a_order == FP16MC_MN_CONTIGUOUS, b_mn = b_order == FP16MC_MN_CONTIGUOUS;
  const fp16mc::GemmPlan plan = fp16mc::choose_gemm_plan(M, N, K, batch, a_mn, b_mn);
  if (plan == fp16mc::GemmPlan::kNone) return ok();
  const int64_t grid = fp16mc::gemm_plan_grid(plan, M, N, batch);
  if (grid > kMaxGrid) return fail(FP16MC_EINVAL, "problem needs %lld workgroups (limit %lld)",
                                   (long long)grid, (long long)kMaxGrid);
  if (!fp16mc::gemm_plan_fits_offsets(plan, K, lda, ldb, ldo, out_type == FP16MC_F32 ? 4 : 2, a_mn, b_mn))
    return fail(FP16MC_EINVAL,
                "a %s tile spans too many bytes (operand rows of lda=%lld / ldb=%lld must stay below 2^32, "
                "output rows of ldo=%lld below 2^31)",
                fp16mc::gemm_plan_name(plan, a_mn, b_mn), (long long)lda, (long long)ldb, (long long)ldo);
  fp16mc::GemmProblem p{A,      B,       Out,     M,       N,       K,
                        lda,    ldb,     ldo,     batch,   strideA, strideB,
                        strideO, static_cast<fp16mc::Dtype>(ab_type), static_cast<fp16mc::Dtype>(out_type),
                        accumulate != 0, a_mn, b_mn};
  const hipError_t e = fp16mc::launch_gemm(plan, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FP16MC_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int gemm_nt_ex(const void* A, const void* B, void* Out, int64_t M, int64_t N, int64_t K, int64_t lda,
               int64_t ldb, int64_t ldo, int64_t batch, int64_t strideA, int64_t strideB, int64_t strideO,
               int ab_type, int out_type, int accumulate, void* stream) {
  return gemm_ex(A, B, Out, M, N, K, lda, ldb, ldo, batch, strideA, strideB, strideO, FP16MC_K_CONTIGUOUS,
                 FP16MC_K_CONTIGUOUS, ab_type, out_type, accumulate, stream);
}

int gemm_nt_f16f32_batched(const void* A, const void* B, float* Out, int64_t M, int64_t N, int64_t K,
                           int64_t lda, int64_t ldb, int64_t ldo, int64_t batch, int64_t strideA,
                           int64_t strideB, int64_t strideO, void* stream) {
  return gemm_nt_ex(A, B, Out, M, N, K, lda, ldb, ldo, batch, strideA, strideB, strideO, FP16MC_F16, FP16MC_F32, 0,
                    stream);
}

int gemm_nt_f16f32(const void* A, const void* B, float* Out, int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int64_t ldo, void* stream) {
  return gemm_nt_ex(A, B, Out, M, N, K, lda, ldb, ldo, 1, 0, 0, 0, FP16MC_F16, FP16MC_F32, 0, stream);
}

int frag_copy(const void* src, void* dst, int64_t num_tiles, int num, int col_major, int direction,
              void* stream) {
  if (num != 1 && num != 2 && num != 4)
    return fail(FP16MC_EINVAL, "num=%d: a matrix load moves 1, 2 or 4 tiles", num);
  if (num_tiles < 0) return fail(FP16MC_EINVAL, "negative num_tiles %lld", (long long)num_tiles);
  if (num_tiles % num)
    return fail(FP16MC_EINVAL, "num_tiles=%lld is not a multiple of num=%d", (long long)num_tiles, num);
  if (col_major != 0 && col_major != 1) return fail(FP16MC_EINVAL, "col_major must be 0 or 1");
  if (direction != FRAG_LOAD && direction != FRAG_STORE && direction != FRAG_ROUNDTRIP)
    return fail(FP16MC_EINVAL, "direction must be FRAG_LOAD, FRAG_STORE or FRAG_ROUNDTRIP");
  if (num_tiles == 0) return ok();
  if (src == nullptr || dst == nullptr) return fail(FP16MC_EINVAL, "src or dst is NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(FP16MC_EALIGN, "src and dst must be 16-byte aligned");
  // Each wavefront reads a whole block before writing the same block, so
  // src == dst works; a partial overlap would let one wavefront overwrite
  // what another has yet to read.
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  uintptr_t bytes = 0, s_end = 0, d_end = 0;
  if (__builtin_mul_overflow(static_cast<uintptr_t>(num_tiles), uintptr_t(128), &bytes) ||
      __builtin_add_overflow(s0, bytes, &s_end) || __builtin_add_overflow(d0, bytes, &d_end))
    return fail(FP16MC_EINVAL, "num_tiles=%lld spans past the end of the address space", (long long)num_tiles);
  if (s0 != d0 && s0 < d_end && d0 < s_end)
    return fail(FP16MC_EINVAL, "src and dst overlap without being the same buffer");
  const hipError_t e = fp16mc::launch_frag_copy(src, dst, num_tiles / num, num, col_major != 0, direction,
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FP16MC_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* gemm_nt_f16f32_plan(int64_t M, int64_t N, int64_t K, int64_t batch) {
  return fp16mc::gemm_plan_name(fp16mc::choose_gemm_plan(M, N, K, batch, false, false), false, false);
}

const char* gemm_ex_plan(int64_t M, int64_t N, int64_t K, int64_t batch, int a_order, int b_order) {
  const bool a_mn = a_order == FP16MC_MN_CONTIGUOUS, b_mn = b_order == FP16MC_MN_CONTIGUOUS;
  return fp16mc::gemm_plan_name(fp16mc::choose_gemm_plan(M, N, K, batch, a_mn, b_mn), a_mn, b_mn);
}

const char* fp16mc_last_error(void) { return g_err; }

}  // extern "C"
