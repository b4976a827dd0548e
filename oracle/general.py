"""Oracle for the general product: bfloat16 operands, an accumulating output
and 16-bit outputs (test infrastructure only).

Definitions followed
  accumulate  "Warp Matrix Instructions", "From Shared Memory to a Matrix
              Product": the MMA takes D, A, B, C and C is the value the sum
              starts from; "Other Fragment Shapes and Transfers": the first K
              issue reads C and later issues accumulate into the preceding D.
              "Blackwell Tensor Cores", "Other TMEM Transfers": accumulators
              that start from existing values.  Reading taken: with
              accumulation the output's previous contents are C, so
              Out = C + A @ B.T.
  bfloat16    "Warp Matrix Instructions", "Other Fragment Shapes and
              Transfers": the instruction has float16 and bfloat16 forms.  A
              bfloat16 value is, by the format's definition, the upper 16
              bits of an IEEE binary32, so widening it to float64 is exact.
              Products of two bfloat16 values have at most 16 significant bits
              and are exact in float64, as for float16.
  storage     "Warp Matrix Instructions", "Other Fragment Shapes and
  order       Transfers": the matrix load has a transposing variant that acts
              on each 8x8 matrix of 16-bit elements; "copy -> ldstmatrix"
              accepts row- and column-major shared layouts.  Reading taken: an
              operand may be stored with K indexing its rows (A as K x M,
              a(i, k) = A[k*lda + i]; B as K x N, b(j, k) = B[k*ldb + j]); the
              product is the same sum over the same logical values.
  16-bit out  the pages only produce fp32 results.  Reading taken: a float16
              or bfloat16 output is the fp32 result rounded to nearest even in
              that format (values past its range become +-inf).

Acceptance: the fp32 rule of ``oracle.gemm`` (|out - ref| <= 1e-4 * bound,
with bound = sum_k |A*B| plus |C| when accumulating) widened by half a unit in
the last place of a 16-bit output format -- the most that the final rounding
can add.
"""

import numpy as np

__all__ = ["bf16_to_f64", "operand_f64", "gemm_nt_ex", "gemm_ex", "gemm_ex_strided", "half_ulp",
           "within_bound_out"]

# significand bits (incl. the implicit one) and minimum normal exponent per format
_FORMATS = {"f16": (11, -14), "bf16": (8, -126)}


def bf16_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64: the pattern is the upper half of a binary32."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError(f"bfloat16 values are passed as uint16 bit patterns, got {bits.dtype}")
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def operand_f64(x, fmt):
    """An operand array in format ``fmt`` ('f16': float16 values, 'bf16': uint16 bit patterns) -> float64."""
    if fmt == "f16":
        x = np.asarray(x)
        if x.dtype != np.float16:
            raise TypeError(f"float16 operand expected, got {x.dtype}")
        return x.astype(np.float64)
    if fmt == "bf16":
        return bf16_to_f64(x)
    raise ValueError(f"unknown operand format {fmt!r}")


def gemm_nt_ex(A, B, C=None, ab="f16", c_fmt="f32"):
    """Reference and bound for Out = A @ B.T (+ C).

    A: (M, K), B: (N, K) in format ``ab``; C: None (fresh output) or the
    output's previous contents, (M, N), given as float32 ('f32'), float16
    ('f16') or bfloat16 bit patterns ('bf16').
    Returns (ref, bound), float64 (M, N):
      ref   = sum_k A[i,k] B[j,k] (+ C[i,j])
      bound = sum_k |A[i,k] B[j,k]| (+ |C[i,j]|)
    A float64 library matmul is the summation step (products exact).
    """
    a = operand_f64(A, ab)
    b = operand_f64(B, ab)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shape mismatch: A {a.shape}, B {b.shape}")
    ref = a @ b.T
    bound = np.abs(a) @ np.abs(b).T
    if C is not None:
        if c_fmt == "f32":
            c = np.asarray(C, dtype=np.float32).astype(np.float64)
        else:
            c = operand_f64(C, c_fmt)
        if c.shape != ref.shape:
            raise ValueError(f"C has shape {c.shape}, expected {ref.shape}")
        ref = ref + c
        bound = bound + np.abs(c)
    return ref, bound


def gemm_ex(A, B, C=None, ab="f16", a_order="k", b_order="k", c_fmt="f32"):
    """Reference and bound for Out = a @ b^T (+ C) with either storage order per operand.

    a_order 'k': A is (M, K), a(i, k) = A[i, k]; 'mn': A is stored (K, M),
    a(i, k) = A[k, i].  Likewise b_order for B ((N, K) or stored (K, N)).
    """
    A = np.asarray(A)
    B = np.asarray(B)
    if a_order not in ("k", "mn") or b_order not in ("k", "mn"):
        raise ValueError("storage orders are 'k' or 'mn'")
    a = A if a_order == "k" else A.T
    b = B if b_order == "k" else B.T
    return gemm_nt_ex(np.ascontiguousarray(a), np.ascontiguousarray(b), C, ab=ab, c_fmt=c_fmt)


def gemm_ex_strided(a_flat, b_flat, M, N, K, lda, ldb, ab="f16", a_order="k", b_order="k", C=None):
    """Oracle seen through the library's buffer view, element by element.

    a(i, k) = a_flat[i*lda + k] ('k') or a_flat[k*lda + i] ('mn'); b(j, k) =
    b_flat[j*ldb + k] or b_flat[k*ldb + j].  Elements outside these index sets
    (the padding between rows) are never read.
    """
    a_flat = np.asarray(a_flat)
    b_flat = np.asarray(b_flat)
    a = np.empty((M, K), dtype=a_flat.dtype)
    b = np.empty((N, K), dtype=b_flat.dtype)
    for i in range(M):
        for k in range(K):
            a[i, k] = a_flat[i * lda + k] if a_order == "k" else a_flat[k * lda + i]
    for j in range(N):
        for k in range(K):
            b[j, k] = b_flat[j * ldb + k] if b_order == "k" else b_flat[k * ldb + j]
    return gemm_nt_ex(a, b, C, ab=ab)


def half_ulp(x, fmt):
    """Half the spacing of format ``fmt`` at |x| (0 for 'f32', whose rounding the 1e-4 rule covers).

    For a value of magnitude in [2^e, 2^(e+1)) the spacing is 2^(e - p + 1)
    with p significand bits; below the smallest normal 2^emin it stays
    2^(emin - p + 1) (the subnormal spacing).
    """
    x = np.abs(np.asarray(x, dtype=np.float64))
    if fmt == "f32":
        return np.zeros_like(x)
    p, emin = _FORMATS[fmt]
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    e = np.maximum(np.where(x > 0, e, emin), emin)
    return np.ldexp(1.0, (e - p).astype(np.int64))


def within_bound_out(out, ref, bound, fmt, rel=1e-4):
    """Acceptance for an output of format ``fmt`` ('f32', 'f16' or 'bf16'; values as float64).

    Passes iff every element is finite and
      |out - ref| <= rel * bound + half_ulp(max(|out|, |ref|), fmt).
    Returns (ok, worst, n_bad) with ``worst`` the largest error divided by
    its allowance.
    """
    out64 = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    if out64.shape != ref.shape:
        raise ValueError(f"shape mismatch {out64.shape} vs {ref.shape}")
    finite = np.isfinite(out64)
    err = np.abs(np.where(finite, out64, 0.0) - ref)
    allow = rel * bound + half_ulp(np.maximum(np.abs(np.where(finite, out64, 0.0)), np.abs(ref)), fmt)
    bad = (~finite) | (err > allow)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(allow > 0, err / np.where(allow > 0, allow, 1.0), np.where(err > 0, np.inf, 0.0))
    ratio = np.where(finite, ratio, np.inf)
    worst = float(ratio.max()) if ratio.size else 0.0
    n_bad = int(bad.sum())
    return n_bad == 0, worst, n_bad
