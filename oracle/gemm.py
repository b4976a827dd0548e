"""Oracle for Out = A @ B.T with fp16 inputs (test infrastructure only).

Definition followed: "Warp Matrix Instructions", introduction and the check
snippet at the end of "From Shared Memory to a Matrix Product" (Out = A @ B.T,
A (M,K) and B (N,K) fp16, compared with a.float() @ b.float().T); the same
product at 128x64x64 in "Blackwell Tensor Cores", "The Accumulator's
Lifetime".  Row i of Out pairs row i of A with row j of B over the shared K
index, i.e. Out[i, j] = sum_k A[i, k] * B[j, k].

Precision: inputs are read as fp16 and widened to float64 (exact).  Each
product of two fp16 values has at most 22 significant bits and is exact in
float64; the sum over K rounds in float64 only (relative error ~K * 2**-53,
about 1e-12 at K = 8192, far below the 1e-4 acceptance bound).

Acceptance (the parity bar): a device result ``out`` passes iff every element
is finite and |out[i,j] - ref[i,j]| <= 1e-4 * bound[i,j] with
bound[i,j] = sum_k |A[i,k] * B[j,k]|.  Any summation order within that bound is
a correct result; the bound is order-free, so it does not favour one order.
"""

import numpy as np

__all__ = ["gemm_nt", "gemm_nt_loops", "gemm_nt_strided", "gemm_nt_rows", "gemm_nt_batched",
           "within_bound"]


def _f64(x):
    """fp16 array -> float64 (exact widening)."""
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError(f"oracle expects float16 inputs, got {x.dtype}")
    return x.astype(np.float64)


def gemm_nt(A, B):
    """Reference and bound for Out = A @ B.T.

    A: (M, K) float16, B: (N, K) float16.
    Returns (ref, bound), both (M, N) float64:
      ref[i, j]   = sum_k A[i, k] * B[j, k]
      bound[i, j] = sum_k |A[i, k] * B[j, k]| = (|A| @ |B|.T)[i, j]
    A float64 library matmul serves as the summation step (products exact).
    """
    a = _f64(A)
    b = _f64(B)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shape mismatch: A {a.shape}, B {b.shape}")
    ref = a @ b.T
    bound = np.abs(a) @ np.abs(b).T
    return ref, bound


def gemm_nt_loops(A, B):
    """The same definition written as an explicit triple loop (small shapes only).

    Used to pin ``gemm_nt``'s library step: one term per (i, j, k), in K order.
    """
    a = _f64(A)
    b = _f64(B)
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise ValueError("K mismatch")
    ref = np.zeros((M, N), dtype=np.float64)
    bound = np.zeros((M, N), dtype=np.float64)
    for i in range(M):
        for j in range(N):
            s = 0.0
            t = 0.0
            for k in range(K):
                p = a[i, k] * b[j, k]
                s += p
                t += abs(p)
            ref[i, j] = s
            bound[i, j] = t
    return ref, bound


def gemm_nt_strided(a_flat, b_flat, M, N, K, lda, ldb):
    """Oracle seen through the library's buffer view.

    Element A[i, k] lives at a_flat[i * lda + k] and B[j, k] at
    b_flat[j * ldb + k] (row-major with leading dimensions lda >= K,
    ldb >= K); elements between K and the leading dimension are never read.
    """
    a_flat = np.asarray(a_flat)
    b_flat = np.asarray(b_flat)
    A = np.empty((M, K), dtype=np.float16)
    B = np.empty((N, K), dtype=np.float16)
    for i in range(M):
        A[i, :] = a_flat[i * lda: i * lda + K]
    for j in range(N):
        B[j, :] = b_flat[j * ldb: j * ldb + K]
    return gemm_nt(A, B)


def gemm_nt_rows(A, B, rows):
    """Oracle for a subset of output rows (for sampled checks at full size)."""
    rows = np.asarray(rows, dtype=np.int64)
    return gemm_nt(np.asarray(A)[rows, :], B)


def gemm_nt_batched(A, B):
    """Independent products: ref[p], bound[p] = gemm_nt(A[p], B[p]) for every problem p."""
    A = np.asarray(A)
    B = np.asarray(B)
    if A.ndim != 3 or B.ndim != 3 or A.shape[0] != B.shape[0]:
        raise ValueError(f"batched shapes {A.shape}, {B.shape}")
    P, M, _ = A.shape
    N = B.shape[1]
    ref = np.empty((P, M, N))
    bound = np.empty((P, M, N))
    for p in range(P):
        ref[p], bound[p] = gemm_nt(A[p], B[p])
    return ref, bound


def within_bound(out, ref, bound, rel=1e-4):
    """Apply the acceptance rule element by element.

    Returns (ok, worst, n_bad): ``worst`` is max |out - ref| / bound over the
    elements (0/0 counts as 0, x/0 for x > 0 as inf), ``n_bad`` the number of
    elements that break the rule or are not finite.
    """
    out64 = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    if out64.shape != ref.shape:
        raise ValueError(f"shape mismatch {out64.shape} vs {ref.shape}")
    finite = np.isfinite(out64)
    err = np.abs(out64 - ref)
    bad = (~finite) | (err > rel * bound)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
    ratio = np.where(finite, ratio, np.inf)
    worst = float(ratio.max()) if ratio.size else 0.0
    n_bad = int(bad.sum())
    return n_bad == 0, worst, n_bad
