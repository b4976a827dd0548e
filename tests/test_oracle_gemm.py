"""Pins of the GEMM oracle against facts fixed by the pages and by arithmetic.

Each test is chosen so that a plausible mistake in ``oracle.gemm`` (a dropped
term, a transposed operand, a wrong index, a sign error, a loose tolerance)
fails at least one of them.  None of them calls the HIP library.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from fp16_matrix_core_amd import inputs


def _exact(A, B):
    """Exact rational Out = A @ B.T (fp16 values are dyadic rationals)."""
    M, K = A.shape
    N = B.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(A[i, k])) * Fraction(float(B[j, k]))
            out[i][j] = s
    return out


def test_worked_shapes(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "worked_shapes.json")))
    rng = np.random.default_rng(11)
    for case in spec["cases"]:
        A = inputs.uniform_f16(tuple(case["A"]), rng)
        B = inputs.uniform_f16(tuple(case["B"]), rng)
        ref, bound = oracle.gemm_nt(A, B)
        assert ref.shape == tuple(case["Out"]) and bound.shape == tuple(case["Out"])


def test_brute_force_exact_single_tile():
    """16x16 by 8x16 (seed 0): fp64 oracle equals the exact rational sum (K=16: no rounding at all)."""
    A, B = inputs.single_tile(0)
    ref, bound = oracle.gemm_nt(A, B)
    ex = _exact(A, B)
    for i in range(16):
        for j in range(8):
            assert Fraction(ref[i, j]) == ex[i][j]
            assert bound[i, j] >= abs(ref[i, j])


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (17, 9, 33), (8, 16, 70), (70, 33, 1), (5, 64, 40)])
def test_library_step_vs_triple_loop(shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    A = inputs.uniform_f16((M, K), rng)
    B = inputs.uniform_f16((N, K), rng)
    ref, bound = oracle.gemm_nt(A, B)
    ref2, bound2 = oracle.gemm_nt_loops(A, B)
    # both sum exact fp64 products; only the fp64 summation order differs
    tol = K * 2.0 ** -52 * bound2
    assert np.all(np.abs(ref - ref2) <= tol)
    assert np.all(np.abs(bound - bound2) <= tol)


def test_exact_rational_small_random():
    rng = np.random.default_rng(7)
    A = inputs.uniform_f16((6, 40), rng)
    B = inputs.uniform_f16((5, 40), rng)
    ref, bound = oracle.gemm_nt(A, B)
    ex = _exact(A, B)
    for i in range(6):
        for j in range(5):
            assert abs(Fraction(ref[i, j]) - ex[i][j]) <= Fraction(40 * 2.0 ** -52) * Fraction(bound[i, j])


def test_identity_b_is_exact_copy():
    A, _, I, _, _ = inputs.single_workgroup()
    ref, _ = oracle.gemm_nt(A, I)
    assert np.array_equal(ref, A.astype(np.float64))


def test_permutation_b_permutes_columns():
    A, _, _, P, perm = inputs.single_workgroup()
    ref, _ = oracle.gemm_nt(A, P)
    assert np.array_equal(ref, A.astype(np.float64)[:, perm])
    # a transposed operand would give the inverse permutation instead
    inv = np.argsort(perm)
    assert not np.array_equal(ref, A.astype(np.float64)[:, inv])


def test_rank_one_closed_form():
    """A[i,k] = a_i c_k, B[j,k] = b_j d_k  =>  Out[i,j] = a_i b_j sum_k c_k d_k (small integers: exact)."""
    a = np.array([1, -2, 3, 0, 5], dtype=np.float64)
    b = np.array([2, 1, -1], dtype=np.float64)
    c = np.arange(1, 9, dtype=np.float64)
    d = np.array([1, -1, 2, 0, 3, 1, -2, 1], dtype=np.float64)
    A = np.outer(a, c).astype(np.float16)
    B = np.outer(b, d).astype(np.float16)
    ref, bound = oracle.gemm_nt(A, B)
    assert np.array_equal(ref, np.outer(a, b) * float(c @ d))
    assert np.array_equal(bound, np.outer(np.abs(a), np.abs(b)) * float(np.abs(c) @ np.abs(d)))


def test_all_ones_gives_k():
    for K in (1, 16, 64, 1000):
        ref, bound = oracle.gemm_nt(np.ones((3, K), np.float16), np.ones((2, K), np.float16))
        assert np.all(ref == K) and np.all(bound == K)


def test_k_slice_accumulation_matches_whole():
    """K = 64 as four K = 16 slices accumulated into D (the sm_100a example's split): exact for integers."""
    rng = np.random.default_rng(5)
    A = rng.integers(-8, 9, size=(128, 64)).astype(np.float16)
    B = rng.integers(-8, 9, size=(64, 64)).astype(np.float16)
    whole, _ = oracle.gemm_nt(A, B)
    acc = np.zeros((128, 64))
    for kr in range(4):
        part, _ = oracle.gemm_nt(A[:, 16 * kr:16 * kr + 16], B[:, 16 * kr:16 * kr + 16])
        acc += part
    assert np.array_equal(acc, whole)


def test_swapping_operands_transposes():
    rng = np.random.default_rng(9)
    A = inputs.uniform_f16((12, 20), rng)
    B = inputs.uniform_f16((7, 20), rng)
    r1, b1 = oracle.gemm_nt(A, B)
    r2, b2 = oracle.gemm_nt(B, A)
    assert np.array_equal(r1, r2.T) and np.array_equal(b1, b2.T)


def test_strided_view_never_reads_padding():
    rng = np.random.default_rng(12)
    M, N, K, lda, ldb = 9, 5, 13, 24, 16
    A = inputs.uniform_f16((M, K), rng)
    B = inputs.uniform_f16((N, K), rng)
    a_flat = np.full(M * lda, np.nan, dtype=np.float16)
    b_flat = np.full(N * ldb, np.nan, dtype=np.float16)
    for i in range(M):
        a_flat[i * lda:i * lda + K] = A[i]
    for j in range(N):
        b_flat[j * ldb:j * ldb + K] = B[j]
    ref, bound = oracle.gemm_nt_strided(a_flat, b_flat, M, N, K, lda, ldb)
    ref2, bound2 = oracle.gemm_nt(A, B)
    assert np.array_equal(ref, ref2) and np.array_equal(bound, bound2)


def test_rows_subset():
    rng = np.random.default_rng(13)
    A = inputs.uniform_f16((40, 24), rng)
    B = inputs.uniform_f16((11, 24), rng)
    rows = [0, 7, 39]
    ref, _ = oracle.gemm_nt(A, B)
    sub, _ = oracle.gemm_nt_rows(A, B, rows)
    assert np.array_equal(sub, ref[rows])


def test_acceptance_rule_catches_planted_mistakes():
    """Mistakes planted in a copy of the oracle's result must fail the 1e-4 rule."""
    A, B, _, _, _ = inputs.single_workgroup()
    a = A.astype(np.float64)
    b = B.astype(np.float64)
    ref, bound = oracle.gemm_nt(A, B)
    # the correct answer passes, also after fp32 rounding of the output
    assert oracle.within_bound(ref.astype(np.float32), ref, bound)[0]
    dropped_term = ref - np.outer(a[:, 5], b[:, 5])
    assert not oracle.within_bound(dropped_term, ref, bound)[0]
    wrong_sign = ref - 2 * np.outer(a[:, 0], b[:, 0])
    assert not oracle.within_bound(wrong_sign, ref, bound)[0]
    shifted_k = a[:, 1:] @ b[:, :-1].T
    assert not oracle.within_bound(shifted_k, ref, bound)[0]
    transposed = (a[:64] @ b.T).T
    assert not oracle.within_bound(transposed, ref[:64], bound[:64])[0]
    with_nan = ref.copy()
    with_nan[3, 4] = np.nan
    ok, worst, n_bad = oracle.within_bound(with_nan, ref, bound)
    assert not ok and n_bad == 1 and worst == np.inf


def test_fp32_accumulation_fits_the_bound():
    """A serial fp32 sum (the worst plain order) of the large-square recipe stays inside 1e-4 * bound.

    Rows of a K = 8192 problem drawn like the 8192^3 workload; shows the bar is
    reachable by any fp32 accumulation order, not only the oracle's.
    """
    rng = np.random.default_rng(4)
    K = 8192
    A = inputs.normal_f16((4, K), rng)
    B = inputs.normal_f16((4, K), rng)
    ref, bound = oracle.gemm_nt(A, B)
    prods = A.astype(np.float32)[:, None, :] * B.astype(np.float32)[None, :, :]   # exact in fp32
    acc = np.zeros((4, 4), dtype=np.float32)
    for k in range(K):
        acc = (acc + prods[:, :, k]).astype(np.float32)
    ok, worst, _ = oracle.within_bound(acc, ref, bound)
    assert ok and worst < 1e-5


def test_batched_is_per_problem():
    rng = np.random.default_rng(14)
    A = inputs.uniform_f16((3, 5, 16), rng)
    B = inputs.uniform_f16((3, 4, 16), rng)
    ref, bound = oracle.gemm_nt_batched(A, B)
    for p in range(3):
        r, b = oracle.gemm_nt_loops(A[p], B[p])
        assert np.allclose(ref[p], r, rtol=0, atol=1e-15) and np.allclose(bound[p], b, rtol=0, atol=1e-15)
