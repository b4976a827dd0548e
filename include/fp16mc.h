/*
 * fp16mc.h -- C ABI of libfp16mc.so: the fp16 NT matrix product with fp32
 * accumulation, and the 8x8 fragment copy between shared memory and
 * registers, on one MI355X (gfx950) GPU.
 *
 * Conventions for every entry point
 *   - Pointers to data are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no reference after the call returns, and never
 *     synchronises the host: work is enqueued on `stream`, a hipStream_t passed
 *     as void* (NULL = the null stream).
 *   - Arguments are validated on the host before any HIP call.  A call that
 *     fails validation enqueues nothing and returns a negative status; the
 *     reason is then available from fp16mc_last_error() on the same thread.
 *   - No C++ exception crosses this interface.
 */
#ifndef FP16MC_H
#define FP16MC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP16MC_OK = 0,
  FP16MC_EINVAL = -1, /* a size, stride, count, flag or pointer is invalid   */
  FP16MC_EALIGN = -2, /* a pointer or stride breaks the 16-byte access rule   */
  FP16MC_EHIP = -3    /* the HIP runtime refused the launch                   */
} fp16mc_status;

/*
 * Out = A @ B.T with fp16 inputs and fp32 accumulation and output.
 *
 * Defined on "Warp Matrix Instructions" (introduction; the check snippet that
 * compares with a.float() @ b.float().T) and "Blackwell Tensor Cores" (the
 * 128x64x64 product, K accumulated slice by slice into a fresh accumulator).
 *
 *   Out[i*ldo + j] = sum_{k<K} A[i*lda + k] * B[j*ldb + k],  0<=i<M, 0<=j<N
 *
 * A: fp16, M rows of K, row stride lda elements.   (read only)
 * B: fp16, N rows of K, row stride ldb elements.   (read only; the product
 *    uses B transposed, so both operands are K-contiguous)
 * Out: fp32, M rows of N, row stride ldo elements. Write only: its prior
 *    contents are ignored (the first K slice starts from zero), and the cells
 *    between N and ldo of each row are never touched.
 * Result accuracy: every element within 1e-4 * sum_k |A[i,k]*B[j,k]| of the
 *    exact sum (fp32 accumulation in an unspecified order).
 *
 * Preconditions (else FP16MC_EINVAL): M, N, K >= 0; lda >= K, ldb >= K,
 *   ldo >= N; A, B non-NULL when M*K, N*K > 0; Out non-NULL when M*N > 0.
 * Alignment (else FP16MC_EALIGN): A and B 16-byte aligned, lda and ldb
 *   multiples of 8 (each 8-element fp16 run is one 16-byte access, the same
 *   rule the matrix-load page states for its tile strides); Out 16-byte
 *   aligned and ldo a multiple of 4.
 * Size limit (else FP16MC_EINVAL): the kernels address each operand tile
 *   (up to 256 rows) with 32-bit byte offsets, so 2*(255*lda + K) and
 *   2*(255*ldb + K) must stay below 2^32 (about lda, ldb < 8.4e6), and each
 *   output tile with signed 32-bit offsets: 256*ldo*4 < 2^31 (ldo < 2.1e6;
 *   256*ldo*2 for 16-bit outputs).
 * M == 0 or N == 0: nothing is enqueued, FP16MC_OK.  K == 0: Out = 0.
 * Operands may not overlap Out.
 */
int gemm_nt_f16f32(const void* A, const void* B, float* Out,
                   int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int64_t ldo, void* stream);

/*
 * `batch` independent products in one launch: the product of "Blackwell
 * Tensor Cores" ("The Accumulator's Lifetime": one 128x64 output tile from a
 * 128x64 A and a 64x64 B, K accumulated slice by slice) repeated over many
 * independent operand sets.  Problem b uses
 * A + b*strideA, B + b*strideB, Out + b*strideO (strides in elements) with
 * the shapes and row strides above.  Same preconditions per problem, plus
 * batch >= 0, strides >= 0, strideA and strideB multiples of 8, strideO a
 * multiple of 4.  batch == 1 is exactly gemm_nt_f16f32.  The operands may be
 * shared between problems (strideA or strideB 0); the outputs may not
 * overlap: with batch > 1, strideO >= (M-1)*ldo + N (else FP16MC_EINVAL).
 */
int gemm_nt_f16f32_batched(const void* A, const void* B, float* Out,
                           int64_t M, int64_t N, int64_t K,
                           int64_t lda, int64_t ldb, int64_t ldo,
                           int64_t batch, int64_t strideA, int64_t strideB,
                           int64_t strideO, void* stream);

/* Element types of gemm_nt_ex. */
typedef enum {
  FP16MC_F32 = 0,  /* IEEE binary32                                        */
  FP16MC_F16 = 1,  /* IEEE binary16                                        */
  FP16MC_BF16 = 2  /* bfloat16: the upper 16 bits of a binary32            */
} fp16mc_dtype;

/*
 * The general form: `batch` products (as gemm_nt_f16f32_batched) with a
 * choice of element types and of a fresh or an accumulating output.
 *
 *   Out[i*ldo + j] = round_out( sum_{k<K} A[i*lda + k] * B[j*ldb + k]
 *                               (+ Out[i*ldo + j] when accumulate) )
 *
 * ab_type: FP16MC_F16 or FP16MC_BF16, for both A and B -- the float16 and
 *   bfloat16 forms of the warp matrix instruction ("Warp Matrix
 *   Instructions", "Other Fragment Shapes and Transfers").  Products are
 *   exact and summed in fp32 as for gemm_nt_f16f32.
 * out_type: FP16MC_F32, or the same type as ab_type; a 16-bit output is the
 *   fp32 result rounded to nearest-even (overflow gives +-inf).
 * accumulate: 0 -- Out's previous contents are ignored (the first K slice
 *   starts from zero); 1 -- Out's previous values are read and added before
 *   the final rounding, i.e. they are the MMA's C operand (the D, A, B, C
 *   contract of "From Shared Memory to a Matrix Product", whose first issue
 *   reads C; and "Other TMEM Transfers" on the Blackwell Tensor Cores page,
 *   accumulators that start from existing values).  With K == 0 an
 *   accumulating call leaves Out's values unchanged (a 16-bit Out is
 *   rewritten with the same value).
 * Result accuracy: every element within 1e-4 * (sum_k |A[i,k]*B[j,k]| plus
 *   |previous Out| when accumulating) of the exact value, plus half a unit
 *   in the last place of a 16-bit output format.
 *
 * Preconditions and errors are those of gemm_nt_f16f32_batched, with Out's
 * alignment rule in bytes: Out 16-byte aligned and ldo (and strideO when
 * batch > 1) a multiple of 16 bytes / element size (4 for fp32, 8 for
 * 16-bit outputs).  An unknown type, an out_type that is neither F32 nor
 * ab_type, or accumulate not in {0, 1} is FP16MC_EINVAL.
 * gemm_nt_f16f32_batched(...) is exactly gemm_nt_ex(..., FP16MC_F16,
 * FP16MC_F32, 0, stream).
 */
int gemm_nt_ex(const void* A, const void* B, void* Out,
               int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int64_t ldo,
               int64_t batch, int64_t strideA, int64_t strideB, int64_t strideO,
               int ab_type, int out_type, int accumulate, void* stream);

/* Storage orders of the operands of gemm_ex. */
enum {
  FP16MC_K_CONTIGUOUS = 0,  /* rows hold K: A[i*lda + k], B[j*ldb + k]          */
  FP16MC_MN_CONTIGUOUS = 1  /* rows are K indices: A[k*lda + i], B[k*ldb + j]   */
};

/*
 * The general form: gemm_nt_ex with a choice of storage order per operand.
 *
 *   Out[i*ldo + j] = round_out( sum_{k<K} a(i,k) * b(j,k)  (+ Out[i*ldo + j]) )
 *   a(i,k) = A[i*lda + k] (a_order = FP16MC_K_CONTIGUOUS) or A[k*lda + i]
 *            (FP16MC_MN_CONTIGUOUS: A stored K x M, M contiguous)
 *   b(j,k) = B[j*ldb + k] (b_order = FP16MC_K_CONTIGUOUS) or B[k*ldb + j]
 *            (FP16MC_MN_CONTIGUOUS: B stored K x N, N contiguous)
 *
 * With both operands K-contiguous this is Out = A @ B.T (gemm_nt_ex); with B
 * stored K x N it is the plain product Out = A @ B.  An operand stored with M
 * (or N) contiguous is staged in LDS as it lies in memory and its fragments
 * are read with the LDS transpose read -- the role of the matrix load's
 * transposing variant ("Warp Matrix Instructions", "Other Fragment Shapes and
 * Transfers": the transpose acts on each 8x8 matrix of 16-bit elements; "copy
 * -> ldstmatrix", column-major shared layouts).
 *
 * Preconditions as gemm_nt_ex, except that a K x M operand needs lda >= M
 * (K x N: ldb >= N) and that an operand stored K x W addresses BK = 64 of its
 * rows at a time with 32-bit byte offsets: 2*64*ld < 2^32.  a_order and
 * b_order outside the enum are FP16MC_EINVAL.  Result accuracy as gemm_nt_ex.
 */
int gemm_ex(const void* A, const void* B, void* Out,
            int64_t M, int64_t N, int64_t K,
            int64_t lda, int64_t ldb, int64_t ldo,
            int64_t batch, int64_t strideA, int64_t strideB, int64_t strideO,
            int a_order, int b_order, int ab_type, int out_type, int accumulate, void* stream);

/* Directions of frag_copy. */
enum {
  FRAG_LOAD = 0,     /* shared image  -> fragment (the ldmatrix direction)  */
  FRAG_STORE = 1,    /* fragment      -> shared image (the stmatrix direction) */
  FRAG_ROUNDTRIP = 2 /* image -> fragment -> image, through registers       */
};

/*
 * The warp-collective 8x8 b16 matrix transfer between shared memory and the
 * per-lane register fragment, for `num` tiles at a time.
 *
 * Defined on "copy -> ldstmatrix": the demonstration program (register layout
 * (8,4,num,2):(4@lane,1@lane,2,1), row-major shared layout
 * (8,4,num,2):(8num,2,8,1)), Algorithm steps 2-4 (lane 4r+c holds row r,
 * column pair c; row- or column-major shared side with 8-element strides;
 * the store direction mirrors the load), and "How inputs change the
 * algorithm" (num in {1,2,4}).  A group is `num` tiles moved by one
 * instruction.  Registers and shared memory are not host-visible, so both
 * sides are serialised in device memory:
 *
 *   image    (shared side), 64*num b16 per group, groups back to back:
 *              row-major    element (r,c) of tile t at r*8*num + 8*t + c
 *              column-major element (r,c) of tile t at (8*t + c)*8 + r
 *   fragment (register side), 32*num uint32 per group, lane-major:
 *              word (g*32 + lane)*num + t holds elements (lane/4, 2*(lane%4))
 *              in bits 0..15 and (lane/4, 2*(lane%4)+1) in bits 16..31.
 *
 * Inside the kernel the image passes through LDS in the given layout and each
 * fragment word through a VGPR of the lane that owns it; one 64-lane
 * wavefront serves two 32-lane fragments.  Only bit patterns move: NaN
 * payloads, infinities, subnormals and -0 are preserved exactly.
 *
 * src, dst: device pointers, 16-byte aligned (else FP16MC_EALIGN), each
 *   num_tiles*128 bytes; either the same buffer (the transfer is done in
 *   place) or not overlapping at all (else FP16MC_EINVAL).  LOAD reads an
 *   image and writes a fragment; STORE the reverse; ROUNDTRIP reads an image
 *   and writes the image it reconstructs from the fragment (bit-identical to
 *   src).
 * num_tiles >= 0 and a multiple of num; num in {1,2,4}; col_major in {0,1};
 *   direction one of FRAG_*  (else FP16MC_EINVAL).  num_tiles == 0: no-op.
 */
int frag_copy(const void* src, void* dst, int64_t num_tiles, int num,
              int col_major, int direction, void* stream);

/*
 * Name of the kernel configuration gemm_nt_f16f32(_batched) would launch for
 * this shape (a static string), or NULL for an empty problem.  Pure host
 * logic, no HIP call.
 */
const char* gemm_nt_f16f32_plan(int64_t M, int64_t N, int64_t K, int64_t batch);

/* The same for gemm_ex with the given storage orders (pure host logic). */
const char* gemm_ex_plan(int64_t M, int64_t N, int64_t K, int64_t batch, int a_order, int b_order);

/*
 * Message describing the last failed call on this thread ("" if none).  The
 * pointer stays valid until the next call of this library on the thread.
 * It plays the part of the (ok, message) pair with which "copy ->
 * ldstmatrix" ("What it accepts") reports why a copy does not fit the
 * matrix load: a rejected call returns a negative status and this text
 * names the argument and the rule it breaks.
 */
const char* fp16mc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP16MC_H */
