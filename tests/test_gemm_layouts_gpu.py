"""GPU parity of gemm_ex with operands stored with K indexing their rows
(A as K x M, B as K x N), against the CPU oracle, through the C ABI.

Same bar as the K-contiguous product: every element within 1e-4 * bound (plus
half an ulp of a 16-bit output), identity and permutation products exact,
padding of Out untouched.  Stored operands carry NaN patterns in the gaps
between their rows: a kernel that let one reach a stored output would fail.
"""

import numpy as np
import pytest

import oracle
from fp16_matrix_core_amd import inputs
from fullcheck import check_all_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

K_C, MN_C = 0, 1
ORDER = {"k": K_C, "mn": MN_C}
CODE = {"f32": 0, "f16": 1, "bf16": 2}
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}
LAYOUTS = [("k", "mn"), ("mn", "k"), ("mn", "mn")]     # NN, TT, TN (NT is covered elsewhere)


@pytest.fixture(scope="module")
def f():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp16_matrix_core_amd as f
    f.lib()
    return f


def _bits(X, fmt):
    return X.view(np.uint16) if fmt == "f16" else np.asarray(X, dtype=np.uint16)


def _draw(shape, rng, fmt):
    return inputs.uniform_f16(shape, rng) if fmt == "f16" else inputs.uniform_bf16(shape, rng)


def _stored(X, order, fmt, extra=0):
    """The logical operand X ((M, K) or (N, K)) as stored: rows of K values or, for
    'mn', rows of M values per K index; row stride a multiple of 8 plus `extra`
    multiples of 8, NaN patterns in the gaps."""
    S = X if order == "k" else np.ascontiguousarray(X.T)
    R, W = S.shape
    ld = max(8, W + (-W) % 8) + 8 * extra
    buf = np.full((max(R, 1), ld), NAN_BITS[fmt], np.uint16)
    buf[:R, :W] = _bits(S, fmt)
    return torch.from_numpy(buf.view(np.int16)).cuda(), ld


def _to_f64(t):
    return t.float().double().cpu().numpy()


def _run(f, A, B, ab, out_fmt, a_order, b_order, C=None, ldo_pad=0, extra=0):
    M, K = A.shape
    N = B.shape[0]
    per16 = 4 if out_fmt == "f32" else 8
    ldo = N + ldo_pad
    ldo += (-ldo) % per16
    out = torch.full((M, ldo), float("nan"), dtype=TORCH[out_fmt], device="cuda")
    if C is not None:
        out[:, :N] = torch.from_numpy(np.asarray(C, np.float64)).to(TORCH[out_fmt]).cuda()
    pad_before = out[:, N:].clone()
    a, lda = _stored(A, a_order, ab, extra)
    b, ldb = _stored(B, b_order, ab, extra)
    f.gemm_ex_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldo, 1, 0, 0, 0,
                  ORDER[a_order], ORDER[b_order], CODE[ab], CODE[out_fmt], C is not None,
                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    view = torch.int16 if out_fmt != "f32" else torch.int32
    pad_same = torch.equal(out[:, N:].view(view), pad_before.view(view))
    return _to_f64(out[:, :N]), pad_same


def _c_values(shape, out_fmt, seed):
    return torch.from_numpy(inputs.accumulator_f32(shape, seed)).to(TORCH[out_fmt]).double().numpy()


SHAPES = [
    (16, 8, 16), (5, 7, 3), (31, 29, 70),                      # one wavefront
    (100, 5, 64), (77, 16, 200), (33, 17, 70),                 # tall tiles (N <= 32)
    (300, 520, 200), (129, 65, 64), (1000, 999, 136), (2049, 3000, 72),
    (4100, 2050, 100), (4096, 4096, 64), (2304, 4608, 130),    # 128x128 tiles (short K)
    (4100, 2050, 40),                                          # 128x128, K < 64: the partial slice alone
]


@pytest.mark.parametrize("a_order,b_order", LAYOUTS)
@pytest.mark.parametrize("ab,out_fmt,acc", [("f16", "f32", False), ("bf16", "bf16", True),
                                            ("f16", "f16", True), ("bf16", "f32", False)])
def test_ragged_shapes(f, a_order, b_order, ab, out_fmt, acc):
    rng = np.random.default_rng(41)
    plans = set()
    for (M, N, K) in SHAPES:
        A = _draw((M, K), rng, ab)
        B = _draw((N, K), rng, ab)
        C = _c_values((M, N), out_fmt, seed=M * 3 + N) if acc else None
        got, pad_same = _run(f, A, B, ab, out_fmt, a_order, b_order, C, ldo_pad=5, extra=1)
        assert pad_same, f"padding of Out written at {(M, N, K)}"
        ref, bound = oracle.gemm_nt_ex(A, B, C, ab=ab)
        ok, worst, n_bad = oracle.within_bound_out(got, ref, bound, out_fmt)
        assert ok, f"{(M, N, K)}: {n_bad} elements outside the bound (worst {worst:.3g})"
        plans.add(f.plan_ex(M, N, K, 1, ORDER[a_order], ORDER[b_order]).split("_")[0])
    assert plans == {"wave32x32", "tall64x32", "wg128x64", "wg128x128"}


@pytest.mark.parametrize("a_order,b_order", LAYOUTS)
@pytest.mark.parametrize("M,N", [(1024, 512), (8192, 1024)])
def test_identity_and_permutation_exact(f, a_order, b_order, M, N):
    rng = np.random.default_rng(42)
    A = _draw((M, N), rng, "f16")
    perm = rng.permutation(N)
    P = inputs.permutation_f16(perm)
    got, _ = _run(f, A, inputs.identity_f16(N), "f16", "f32", a_order, b_order)
    assert np.array_equal(got, A.astype(np.float64))
    got, _ = _run(f, A, P, "f16", "f32", a_order, b_order)
    assert np.array_equal(got, A.astype(np.float64)[:, perm])


@pytest.mark.parametrize("a_order,b_order", LAYOUTS)
def test_one_hot_products_locate_every_cell(f, a_order, b_order):
    M, N, K = 300, 260, 192
    ka = (np.arange(M) * 5) % K
    kb = (np.arange(N) * 7) % K
    A = np.zeros((M, K), np.float16)
    B = np.zeros((N, K), np.float16)
    A[np.arange(M), ka] = 1
    B[np.arange(N), kb] = 1
    got, _ = _run(f, A, B, "f16", "f32", a_order, b_order)
    assert np.array_equal(got, (ka[:, None] == kb[None, :]).astype(np.float64))


@pytest.mark.parametrize("a_order,b_order", LAYOUTS)
def test_full_size_every_element(f, a_order, b_order):
    """8192^3 with the stored operands, every element checked."""
    n = 8192
    A, B = inputs.large_square(n)
    a = torch.from_numpy((A if a_order == "k" else np.ascontiguousarray(A.T)).view(np.int16)).cuda()
    b = torch.from_numpy((B if b_order == "k" else np.ascontiguousarray(B.T)).view(np.int16)).cuda()
    out = torch.full((n, n), float("nan"), dtype=torch.float32, device="cuda")
    assert f.plan_ex(n, n, n, 1, ORDER[a_order], ORDER[b_order]).startswith("wg256")
    f.gemm_ex_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), n, n, n, n, n, n, 1, 0, 0, 0,
                  ORDER[a_order], ORDER[b_order], 1, 0, False, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check_all_rows(out, lambda r0, r1: oracle.gemm_nt(A[r0:r1], B))


def test_batched_transposed(f):
    """4096 problems of 128x64x64 with B stored K x N (the plain product per problem)."""
    P, M, N, K = 4096, 128, 64, 64
    rng = np.random.default_rng(44)
    A = inputs.uniform_f16((P, M, K), rng)
    B = inputs.uniform_f16((P, N, K), rng)
    Bs = np.ascontiguousarray(np.transpose(B, (0, 2, 1)))      # (P, K, N)
    a = torch.from_numpy(A).cuda()
    b = torch.from_numpy(Bs).cuda()
    out = torch.empty((P, M, N), dtype=torch.float32, device="cuda")
    f.gemm_ex_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, K, N, N, P, M * K, K * N, M * N,
                  K_C, MN_C, 1, 0, False, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    for p in range(0, P, 131):
        ref, bound = oracle.gemm_nt(A[p], B[p])
        assert oracle.within_bound(got[p], ref, bound)[0], p


def test_matmul_binding_reads_storage_order_from_strides(f):
    rng = np.random.default_rng(45)
    A = inputs.uniform_f16((96, 80), rng)      # logical (M, K)
    B = inputs.uniform_f16((72, 80), rng)      # logical (N, K)
    a_km = torch.from_numpy(np.ascontiguousarray(A.T)).cuda()    # stored K x M
    b_kn = torch.from_numpy(np.ascontiguousarray(B.T)).cuda()    # stored K x N
    a_mk = torch.from_numpy(A).cuda()
    b_nk = torch.from_numpy(B).cuda()
    ref, bound = oracle.gemm_nt(A, B)
    for a, b in ((a_mk, b_nk.t()), (a_mk, b_kn), (a_km.t(), b_nk.t()), (a_km.t(), b_kn)):
        out = f.matmul(a, b)
        torch.cuda.synchronize()
        assert oracle.within_bound(out.double().cpu().numpy(), ref, bound)[0]
    with pytest.raises(ValueError):
        f.matmul(a_mk[:, ::2], b_kn[:40])           # no unit stride


@pytest.mark.parametrize("a_order,b_order", [("k", "k")] + LAYOUTS)
@pytest.mark.parametrize("M,N", [(4096, 4096), (300, 520)])          # 128x128 and 128x64 tiles
@pytest.mark.parametrize("ab,out_fmt,acc", [("f16", "f32", False), ("bf16", "bf16", False), ("f16", "f16", True)])
def test_k_zero(f, a_order, b_order, M, N, ab, out_fmt, acc):
    """K = 0: no MFMA runs, so the output is the zero sum (fresh) or the previous
    values (accumulating), exactly, in every storage order; padding untouched."""
    rng = np.random.default_rng(M + N)
    A = _draw((M, 0), rng, ab)
    B = _draw((N, 0), rng, ab)
    C = _c_values((M, N), out_fmt, seed=M + 2 * N) if acc else None
    got, pad_same = _run(f, A, B, ab, out_fmt, a_order, b_order, C, ldo_pad=3)
    assert pad_same, "padding of Out written"
    assert np.array_equal(got, C if acc else np.zeros((M, N)))


@pytest.mark.parametrize("a_order,b_order,ab,out_fmt", [("mn", "mn", "bf16", "bf16"), ("k", "mn", "f16", "f16")])
def test_full_size_16bit_outputs_every_element(f, a_order, b_order, ab, out_fmt):
    """8192^3 with MN-contiguous operands and a 16-bit output (tied accumulators,
    transposed for the LDS-staged epilogue), every element checked."""
    n = 8192
    A, B = inputs.large_square_bf16(n) if ab == "bf16" else inputs.large_square(n)
    a = torch.from_numpy(np.ascontiguousarray(_bits(A if a_order == "k" else A.T, ab)).view(np.int16)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(_bits(B if b_order == "k" else B.T, ab)).view(np.int16)).cuda()
    out = torch.full((n, n), float("nan"), dtype=TORCH[out_fmt], device="cuda")
    assert f.plan_ex(n, n, n, 1, ORDER[a_order], ORDER[b_order]).startswith("wg256")
    f.gemm_ex_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), n, n, n, n, n, n, 1, 0, 0, 0,
                  ORDER[a_order], ORDER[b_order], CODE[ab], CODE[out_fmt], False,
                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check_all_rows(out, lambda r0, r1: oracle.gemm_nt_ex(A[r0:r1], B, ab=ab), out_fmt)
