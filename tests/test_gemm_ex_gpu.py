"""GPU parity of gemm_nt_ex (bfloat16 operands, accumulation, 16-bit outputs)
against the CPU oracle, through the C ABI.

Bar: every element finite and |gpu - ref| <= 1e-4 * (sum_k |A B| + |C|) plus
half a unit in the last place of a 16-bit output (oracle.within_bound_out);
identity and permutation products exact; the padding cells of Out never
touched; with accumulation the previous contents are the C operand, without
it they are ignored.
"""

import numpy as np
import pytest

import oracle
from fp16_matrix_core_amd import inputs
from fullcheck import check_all_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32, F16, BF16 = 0, 1, 2
CODE = {"f32": F32, "f16": F16, "bf16": BF16}
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}
TYPE_COMBOS = [("f16", "f32"), ("f16", "f16"), ("bf16", "f32"), ("bf16", "bf16")]


@pytest.fixture(scope="module")
def f():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp16_matrix_core_amd as f
    f.lib()
    return f


def _bits(X, fmt):
    """Operand values -> uint16 bit patterns (float16 arrays or bfloat16 patterns as given)."""
    return X.view(np.uint16) if fmt == "f16" else np.asarray(X, dtype=np.uint16)


def _draw(shape, rng, fmt):
    return inputs.uniform_f16(shape, rng) if fmt == "f16" else inputs.uniform_bf16(shape, rng)


def _dev_bits(X, fmt):
    """Rows of X in a device buffer with row stride a multiple of 8 and NaN patterns in the gaps."""
    R, K = X.shape
    ld = max(8, K + (-K) % 8)
    buf = np.full((R, ld), NAN_BITS[fmt], np.uint16)
    buf[:, :K] = _bits(X, fmt)
    return torch.from_numpy(buf.view(np.int16)).cuda(), ld


def _to_f64(t):
    return t.double().cpu().numpy() if t.dtype != torch.bfloat16 else t.float().double().cpu().numpy()


def _run(f, A, B, ab, out_fmt, C=None, ldo_pad=0):
    """Out prefilled with C (accumulating) or NaN (fresh); padding cells NaN in both cases."""
    M, K = A.shape
    N = B.shape[0]
    per16 = 4 if out_fmt == "f32" else 8
    ldo = N + ldo_pad
    ldo += (-ldo) % per16
    out = torch.full((M, ldo), float("nan"), dtype=TORCH[out_fmt], device="cuda")
    if C is not None:
        out[:, :N] = torch.from_numpy(np.asarray(C, dtype=np.float64)).to(TORCH[out_fmt]).cuda()
    pad_before = out[:, N:].clone()
    a, lda = _dev_bits(A, ab)
    b, ldb = _dev_bits(B, ab)
    f.gemm_nt_ex_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldo, 1, 0, 0, 0,
                     CODE[ab], CODE[out_fmt], C is not None, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    pad_same = torch.equal(out[:, N:].view(torch.int16 if out_fmt != "f32" else torch.int32),
                           pad_before.view(torch.int16 if out_fmt != "f32" else torch.int32))
    return _to_f64(out[:, :N]), pad_same


def _c_values(shape, out_fmt, seed):
    """Previous Out contents, representable in the output format."""
    c = inputs.accumulator_f32(shape, seed)
    return torch.from_numpy(c).to(TORCH[out_fmt]).double().numpy()


def _check(got, A, B, ab, out_fmt, C=None):
    ref, bound = oracle.gemm_nt_ex(A, B, C, ab=ab, c_fmt="f32")
    ok, worst, n_bad = oracle.within_bound_out(got, ref, bound, out_fmt)
    assert ok, f"{n_bad} elements outside the bound (worst ratio {worst:.3g})"


SHAPES = [
    (16, 8, 16), (5, 7, 3), (31, 32, 64),                       # one wavefront
    (1000, 8, 300), (333, 16, 1000), (77, 3, 129), (33, 17, 70),  # tall tiles (N <= 32)
    (300, 520, 200), (129, 65, 64),                              # 128x64 tiles
    (4100, 2050, 100), (2049, 3000, 136), (4096, 4096, 64),     # 128x128 tiles (short K)
]


@pytest.mark.parametrize("ab,out_fmt", TYPE_COMBOS)
@pytest.mark.parametrize("acc", [False, True])
def test_ragged_shapes_all_plans(f, ab, out_fmt, acc):
    rng = np.random.default_rng(31)
    plans = set()
    for (M, N, K) in SHAPES:
        A = _draw((M, K), rng, ab)
        B = _draw((N, K), rng, ab)
        C = _c_values((M, N), out_fmt, seed=M + N) if acc else None
        got, pad_same = _run(f, A, B, ab, out_fmt, C, ldo_pad=3)
        assert pad_same, f"padding of Out written at {(M, N, K)}"
        _check(got, A, B, ab, out_fmt, C)
        plans.add(f.plan(M, N, K).split("_")[0])
    assert plans == {"wave32x32", "tall64x32", "wg128x64", "wg128x128"}


@pytest.mark.parametrize("ab,out_fmt", TYPE_COMBOS)
def test_identity_and_permutation_exact(f, ab, out_fmt):
    rng = np.random.default_rng(32)
    M, N = 1024, 512        # 128x64 tiles
    A = _draw((M, N), rng, ab)
    a64 = oracle.operand_f64(A, ab)
    eye = np.eye(N)
    I = eye.astype(np.float16) if ab == "f16" else inputs.to_bf16_bits(eye)
    got, _ = _run(f, A, I, ab, out_fmt)
    assert np.array_equal(got, a64)                  # every operand value is representable in the output
    perm = rng.permutation(N)
    P = np.zeros((N, N))
    P[np.arange(N), perm] = 1
    P = P.astype(np.float16) if ab == "f16" else inputs.to_bf16_bits(P)
    got, _ = _run(f, A, P, ab, out_fmt)
    assert np.array_equal(got, a64[:, perm])


@pytest.mark.parametrize("ab,out_fmt", TYPE_COMBOS)
def test_permutation_on_256_tiles_exact(f, ab, out_fmt):
    rng = np.random.default_rng(33)
    M, N = 4096, 3072       # 16 x 12 = 192 tiles of 256 x 256
    A = _draw((M, N), rng, ab)
    perm = rng.permutation(N)
    P = np.zeros((N, N))
    P[np.arange(N), perm] = 1
    P = P.astype(np.float16) if ab == "f16" else inputs.to_bf16_bits(P)
    assert f.plan(M, N, N).startswith("wg256")
    got, _ = _run(f, A, P, ab, out_fmt)
    assert np.array_equal(got, oracle.operand_f64(A, ab)[:, perm])


@pytest.mark.parametrize("ab,out_fmt", TYPE_COMBOS)
def test_accumulate_with_k0_keeps_out(f, ab, out_fmt):
    for (M, N) in [(16, 8), (100, 12), (300, 200), (1024, 1024)]:
        C = _c_values((M, N), out_fmt, seed=M)
        A = np.zeros((M, 0), np.float16 if ab == "f16" else np.uint16)
        B = np.zeros((N, 0), np.float16 if ab == "f16" else np.uint16)
        got, pad_same = _run(f, A, B, ab, out_fmt, C)
        assert pad_same and np.array_equal(got, C)


@pytest.mark.parametrize("ab,out_fmt", TYPE_COMBOS)
def test_accumulate_twice_is_two_products(f, ab, out_fmt):
    """Out += A1 B1^T then Out += A2 B2^T equals C + [A1 A2] [B1 B2]^T within the bound."""
    rng = np.random.default_rng(34)
    M, N, K = 700, 600, 96
    A1, B1 = _draw((M, K), rng, ab), _draw((N, K), rng, ab)
    A2, B2 = _draw((M, K), rng, ab), _draw((N, K), rng, ab)
    C = _c_values((M, N), out_fmt, seed=35)
    per16 = 4 if out_fmt == "f32" else 8
    ldo = N + (-N) % per16
    out = torch.zeros((M, ldo), dtype=TORCH[out_fmt], device="cuda")
    out[:, :N] = torch.from_numpy(C).to(TORCH[out_fmt]).cuda()
    s = torch.cuda.current_stream().cuda_stream
    for A, B in ((A1, B1), (A2, B2)):
        a, lda = _dev_bits(A, ab)
        b, ldb = _dev_bits(B, ab)
        f.gemm_nt_ex_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldo, 1, 0, 0, 0,
                         CODE[ab], CODE[out_fmt], True, s)
    torch.cuda.synchronize()
    got = _to_f64(out[:, :N])
    A = np.concatenate([A1, A2], axis=1)
    B = np.concatenate([B1, B2], axis=1)
    ref, bound = oracle.gemm_nt_ex(A, B, C, ab=ab)
    # Two roundings of a 16-bit output: the first at the intermediate value
    # C + A1 B1^T (which can exceed the final one in magnitude), the second at
    # the result; the second call's bound also counts |intermediate|.
    ref1, bound1 = oracle.gemm_nt_ex(A1, B1, C, ab=ab)
    mid = np.abs(ref1) + 1e-4 * bound1
    allow = (1e-4 * (bound + mid) + oracle.half_ulp(mid, out_fmt)
             + oracle.half_ulp(np.maximum(np.abs(got), np.abs(ref)), out_fmt))
    assert (np.abs(got - ref) <= allow).all()


@pytest.mark.parametrize("ab,out_fmt,acc", [("bf16", "f32", False), ("f16", "f16", False),
                                            ("f16", "f32", True), ("bf16", "bf16", True)])
def test_full_size_every_element(f, ab, out_fmt, acc):
    """The 8192^3 launch (the measured configuration) with other types, every element checked."""
    n = 8192
    if ab == "bf16":
        A, B = inputs.large_square_bf16(n)
    else:
        A, B = inputs.large_square(n)
    a = torch.from_numpy(_bits(A, ab).view(np.int16)).cuda()
    b = torch.from_numpy(_bits(B, ab).view(np.int16)).cuda()
    out = torch.empty((n, n), dtype=TORCH[out_fmt], device="cuda")
    C = None
    if acc:
        C = _c_values((n, n), out_fmt, seed=7)
        out.copy_(torch.from_numpy(C).to(TORCH[out_fmt]))
    else:
        out.fill_(float("nan"))
    assert f.plan(n, n, n).startswith("wg256")
    f.gemm_nt_ex_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), n, n, n, n, n, n, 1, 0, 0, 0,
                     CODE[ab], CODE[out_fmt], acc, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check_all_rows(out, lambda r0, r1: oracle.gemm_nt_ex(A[r0:r1], B, C[r0:r1] if acc else None, ab=ab), out_fmt)


@pytest.mark.parametrize("ab,out_fmt", [("bf16", "bf16"), ("f16", "f16")])
def test_batched_accumulate(f, ab, out_fmt):
    """The 4096-problem 128x64x64 batch with 16-bit, accumulating outputs."""
    P, M, N, K = 4096, 128, 64, 64
    rng = np.random.default_rng(37)
    A = _draw((P, M, K), rng, ab)
    B = _draw((P, N, K), rng, ab)
    C = _c_values((P, M, N), out_fmt, seed=38)
    a = torch.from_numpy(_bits(A, ab).view(np.int16)).cuda()
    b = torch.from_numpy(_bits(B, ab).view(np.int16)).cuda()
    out = torch.from_numpy(C).to(TORCH[out_fmt]).cuda()
    f.gemm_nt_ex_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, K, K, N, P, M * K, N * K, M * N,
                     CODE[ab], CODE[out_fmt], True, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = _to_f64(out)
    for p in range(0, P, 97):       # 43 problems spread over the batch
        ref, bound = oracle.gemm_nt_ex(A[p], B[p], C[p], ab=ab)
        ok, worst, n_bad = oracle.within_bound_out(got[p], ref, bound, out_fmt)
        assert ok, f"problem {p}: {n_bad} bad (worst {worst:.3g})"


def test_binding_types(f):
    rng = np.random.default_rng(39)
    A = inputs.uniform_bf16((70, 40), rng)
    B = inputs.uniform_bf16((50, 40), rng)
    a = torch.from_numpy(A.view(np.int16)).cuda().view(torch.bfloat16)
    b = torch.from_numpy(B.view(np.int16)).cuda().view(torch.bfloat16)
    out = f.gemm_nt(a, b, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16 and tuple(out.shape) == (70, 50)
    torch.cuda.synchronize()
    ref, bound = oracle.gemm_nt_ex(A, B, ab="bf16")
    assert oracle.within_bound_out(_to_f64(out), ref, bound, "bf16")[0]
    C = _c_values((70, 50), "f32", seed=40)
    out32 = torch.zeros((70, 52), dtype=torch.float32, device="cuda")[:, :50]   # 16-byte rows
    out32.copy_(torch.from_numpy(C.astype(np.float32)))
    f.gemm_nt(a, b, out32, accumulate=True)
    torch.cuda.synchronize()
    ref, bound = oracle.gemm_nt_ex(A, B, C, ab="bf16")
    assert oracle.within_bound_out(out32.double().cpu().numpy(), ref, bound, "f32")[0]
    with pytest.raises(TypeError):
        f.gemm_nt(a, b, out_dtype=torch.float16)
    with pytest.raises(ValueError):
        f.gemm_nt(a, b, accumulate=True)
