"""GPU parity of gemm_nt_f16f32 against the CPU oracle (through the C ABI).

Bar: every element finite and |gpu - ref| <= 1e-4 * sum_k |A[i,k] B[j,k]|
(fp64 oracle); the identity and permutation cases are exact; padding cells
of Out (between N and ldo) and the prior contents of Out never leak.
"""

import numpy as np
import pytest

import oracle
from fp16_matrix_core_amd import inputs
from fullcheck import check_all_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENTINEL = float("nan")


@pytest.fixture(scope="module")
def f():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp16_matrix_core_amd as f
    f.lib()
    return f


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _padded(X):
    """Rows of X in a buffer whose row stride is a multiple of 8, NaN in the gaps (never read)."""
    R, K = X.shape
    ld = max(8, K + (-K) % 8)
    buf = np.full((R, ld), np.nan, np.float16)
    buf[:, :K] = X
    return buf, ld


def _run(f, A, B, ldo_pad=0):
    """Call the C ABI with Out prefilled with NaN (prior contents must be ignored)."""
    M, K = A.shape
    N = B.shape[0]
    ldo = N + ldo_pad
    ldo += (-ldo) % 4
    out = torch.full((M, ldo), SENTINEL, dtype=torch.float32, device="cuda")
    a_buf, lda = _padded(A)
    b_buf, ldb = _padded(B)
    a, b = _dev(a_buf), _dev(b_buf)
    f.gemm_nt_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldo,
                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    full = out.cpu().numpy()
    return full[:M, :N], full[:M, N:]


def _assert_parity(got, A, B):
    ref, bound = oracle.gemm_nt(A, B)
    ok, worst, n_bad = oracle.within_bound(got, ref, bound)
    assert ok, f"{n_bad} elements outside 1e-4 * bound (worst ratio {worst:.3g})"
    return worst


def test_single_tile_one_wavefront(f):
    A, B = inputs.single_tile(0)
    assert f.plan(16, 8, 16).startswith("wave32")      # one 64-lane wavefront
    got, _ = _run(f, A, B)
    assert got.shape == (16, 8)
    _assert_parity(got, A, B)


def test_single_workgroup(f):
    A, B, _, _, _ = inputs.single_workgroup()
    got, _ = _run(f, A, B)
    _assert_parity(got, A, B)


def test_identity_b_exact(f):
    A, _, I, _, _ = inputs.single_workgroup()
    got, _ = _run(f, A, I)
    assert np.array_equal(got, A.astype(np.float32))


def test_permutation_b_exact(f):
    A, _, _, P, perm = inputs.single_workgroup()
    got, _ = _run(f, A, P)
    assert np.array_equal(got, A.astype(np.float32)[:, perm])


@pytest.mark.parametrize("M,N,plan", [(4096, 3072, "wg256x256"), (4096, 5120, "wg256x128"),
                                      (8192, 1024, "wg128x128")])
def test_permutation_large_tiles_exact(f, M, N, plan):
    """A permutation product on each large-tile configuration: any lane-map mistake permutes the output."""
    rng = np.random.default_rng(21)
    A = inputs.uniform_f16((M, N), rng)
    perm = rng.permutation(N)
    P = inputs.permutation_f16(perm)
    assert f.plan(M, N, N).startswith(plan)
    got, _ = _run(f, A, P)
    assert np.array_equal(got, A.astype(np.float32)[:, perm])


def test_one_hot_products_locate_every_cell(f):
    """A = rows of distinct one-hot K positions, B likewise: Out[i, j] = 1 iff their K positions match."""
    M, N, K = 96, 80, 128
    ka = np.arange(M) % K
    kb = (np.arange(N) * 7) % K
    A = np.zeros((M, K), np.float16)
    B = np.zeros((N, K), np.float16)
    A[np.arange(M), ka] = 1
    B[np.arange(N), kb] = 1
    got, _ = _run(f, A, B)
    assert np.array_equal(got, (ka[:, None] == kb[None, :]).astype(np.float32))


RAGGED = [
    (1, 1, 1), (1, 17, 9), (17, 1, 33), (5, 7, 3), (33, 17, 70), (31, 32, 64), (64, 64, 1000),
    (129, 65, 64), (300, 520, 200), (257, 255, 130), (1000, 1000, 72), (513, 700, 257),
    (4100, 2050, 100), (4096, 4096, 64), (2049, 3000, 136),
]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged_shapes(f, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 7 + N * 13 + K)
    A = inputs.uniform_f16((M, K), rng)
    B = inputs.uniform_f16((N, K), rng)
    got, pad = _run(f, A, B, ldo_pad=5)
    _assert_parity(got, A, B)
    assert np.isnan(pad).all(), "ldo padding was written"


def test_k_zero_writes_zeros(f):
    A = np.zeros((40, 0), np.float16)
    B = np.zeros((24, 0), np.float16)
    M, N = 40, 24
    out = torch.full((M, N), SENTINEL, dtype=torch.float32, device="cuda")
    a = torch.empty(8, dtype=torch.float16, device="cuda")
    f.gemm_nt_raw(a.data_ptr(), a.data_ptr(), out.data_ptr(), M, N, 0, 8, 8, N,
                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert (out == 0).all()
    del A, B


def test_strided_operands_never_read_padding(f):
    """lda, ldb > K with NaN in the gaps: a single NaN read would poison the output."""
    rng = np.random.default_rng(31)
    M, N, K, lda, ldb = 300, 270, 100, 136, 112
    A = inputs.uniform_f16((M, K), rng)
    B = inputs.uniform_f16((N, K), rng)
    a_full = np.full((M, lda), np.nan, np.float16)
    b_full = np.full((N, ldb), np.nan, np.float16)
    a_full[:, :K] = A
    b_full[:, :K] = B
    a, b = _dev(a_full), _dev(b_full)
    ldo = N + 6
    out = torch.full((M, ldo), SENTINEL, dtype=torch.float32, device="cuda")
    f.gemm_nt_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldo,
                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    full = out.cpu().numpy()
    _assert_parity(full[:, :N], A, B)
    assert np.isnan(full[:, N:]).all()


def test_torch_binding_matches_raw(f):
    rng = np.random.default_rng(41)
    A = inputs.uniform_f16((200, 96), rng)
    B = inputs.uniform_f16((150, 96), rng)
    out = f.gemm_nt(_dev(A), _dev(B))
    torch.cuda.synchronize()
    _assert_parity(out.cpu().numpy(), A, B)


def test_large_square_every_element(f):
    """M = N = K = 8192, normal(0,1)*0.1 (seed 4), the launch the benchmark times; every element checked."""
    A, B = inputs.large_square()
    a, b = _dev(A), _dev(B)
    out = torch.full((8192, 8192), SENTINEL, dtype=torch.float32, device="cuda")
    assert f.plan(8192, 8192, 8192).startswith("wg256")
    f.gemm_nt_f16f32(a.data_ptr(), b.data_ptr(), out.data_ptr(), 8192, 8192, 8192, 8192, 8192, 8192,
                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check_all_rows(out, lambda r0, r1: oracle.gemm_nt(A[r0:r1], B))


def test_row_shard_every_element(f):
    """A's first 1024 rows against the whole 8192 x 8192 B (what each of 8 GPUs
    would run with the product split by rows), through a 1032-row buffer whose
    last 8 rows must stay untouched; every element checked."""
    A, B = inputs.large_square()
    a, b = _dev(A), _dev(B)
    m, n = 1024, 8192
    buf = torch.full((m + 8, n), SENTINEL, dtype=torch.float32, device="cuda")
    f.gemm_nt_raw(a.data_ptr(), b.data_ptr(), buf.data_ptr(), m, n, n, n, n, n,
                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert bool(torch.isnan(buf[m:]).all()), "rows past M written"
    check_all_rows(buf[:m], lambda r0, r1: oracle.gemm_nt(A[r0:r1], B))


def test_batched_small(f):
    """4096 independent 128x64 by 64x64 problems (seed 5), one launch; every element checked,
    through the tensor binding and through the C entry point."""
    A, B = inputs.batched_small()
    ref, bound = oracle.gemm_nt_batched(A, B)
    a, b = _dev(A), _dev(B)
    out = f.gemm_nt_batched(a, b)
    torch.cuda.synchronize()
    ok, worst, n_bad = oracle.within_bound(out.cpu().numpy(), ref, bound)
    assert ok, f"{n_bad} bad, worst {worst:.3g}"
    P, M, K = A.shape
    N = B.shape[1]
    raw = torch.full((P, M, N), SENTINEL, dtype=torch.float32, device="cuda")
    f.gemm_nt_f16f32_batched(a.data_ptr(), b.data_ptr(), raw.data_ptr(), M, N, K, K, K, N, P, M * K, N * K, M * N,
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(raw, out), "the C entry point and the tensor binding differ"


def test_batched_equals_single_calls(f):
    rng = np.random.default_rng(51)
    A = inputs.uniform_f16((3, 70, 40), rng)
    B = inputs.uniform_f16((3, 50, 40), rng)
    out = f.gemm_nt_batched(_dev(A), _dev(B))
    torch.cuda.synchronize()
    for p in range(3):
        _assert_parity(out[p].cpu().numpy(), A[p], B[p])


def test_skinny(f):
    """M = 16384, N = 8, K = 16384 (seed 5) on the tall tiles; every element checked."""
    A, B = inputs.skinny()
    assert f.plan(16384, 8, 16384).startswith("tall64x32")
    got, pad = _run(f, A, B, ldo_pad=3)
    _assert_parity(got, A, B)
    assert np.isnan(pad).all()


SKINNY = [(64, 1, 128), (65, 8, 129), (1000, 16, 1000), (33, 3, 7), (4097, 5, 2048), (200, 16, 0), (128, 12, 4100),
          (500, 32, 300), (301, 24, 100), (70, 17, 64)]


@pytest.mark.parametrize("shape", SKINNY, ids=lambda s: "x".join(map(str, s)))
def test_skinny_ragged(f, shape):
    """N <= 32 shapes on the tall tiles: ragged M, N, K (incl. K = 0 and K not a multiple of 8)."""
    M, N, K = shape
    assert f.plan(M, N, K).startswith("tall64x32") or (M <= 32 and N <= 32)
    rng = np.random.default_rng(M + 31 * N + 7 * K)
    A = inputs.uniform_f16((M, K), rng)
    B = inputs.uniform_f16((N, K), rng)
    if K == 0:
        out = torch.full((M, 36), SENTINEL, dtype=torch.float32, device="cuda")
        a = torch.empty(8, dtype=torch.float16, device="cuda")
        f.gemm_nt_raw(a.data_ptr(), a.data_ptr(), out.data_ptr(), M, N, 0, 8, 8, 36,
                      torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        full = out.cpu().numpy()
        assert (full[:, :N] == 0).all() and np.isnan(full[:, N:]).all()
        return
    got, pad = _run(f, A, B, ldo_pad=4)
    _assert_parity(got, A, B)
    assert np.isnan(pad).all()


SMALL_GRID = [(512, 512, 16384), (300, 500, 4100), (100, 200, 8200), (256, 1000, 4096), (1000, 1000, 600), (40, 3000, 2000)]


@pytest.mark.parametrize("shape", SMALL_GRID, ids=lambda s: "x".join(map(str, s)))
def test_small_grid_64x64_tiles(f, shape):
    """K >= 512 with at most 256 tiles of 64x64: at most one tile per CU
    (ragged M, N and K); every element checked."""
    M, N, K = shape
    assert f.plan(M, N, K).startswith("wg64x64_")
    rng = np.random.default_rng(M + 31 * N + 7 * K)
    A = inputs.uniform_f16((M, K), rng)
    B = inputs.uniform_f16((N, K), rng)
    got, pad = _run(f, A, B, ldo_pad=4)
    _assert_parity(got, A, B)
    assert np.isnan(pad).all()


WIDE = [(8, 4097, 1000), (32, 3000, 4100), (1, 777, 333), (17, 2048, 2048), (5, 65, 640)]


@pytest.mark.parametrize("shape", WIDE, ids=lambda s: "x".join(map(str, s)))
def test_wide_ragged(f, shape):
    """M <= 32 shapes on the wide tiles (B streamed): ragged N and K; K spans
    several slices, so each workgroup's staggered K sweep wraps around, and
    most end with a partial slice."""
    M, N, K = shape
    assert f.plan(M, N, K).startswith("wide32x64")
    rng = np.random.default_rng(M + 31 * N + 7 * K)
    A = inputs.uniform_f16((M, K), rng)
    B = inputs.uniform_f16((N, K), rng)
    got, pad = _run(f, A, B, ldo_pad=4)
    _assert_parity(got, A, B)
    assert np.isnan(pad).all()


def test_skinny_batched(f):
    rng = np.random.default_rng(61)
    A = inputs.uniform_f16((3, 130, 256), rng)
    B = inputs.uniform_f16((3, 8, 256), rng)
    out = f.gemm_nt_batched(_dev(A), _dev(B))
    torch.cuda.synchronize()
    ref, bound = oracle.gemm_nt_batched(A, B)
    ok, worst, n_bad = oracle.within_bound(out.cpu().numpy(), ref, bound)
    assert ok, f"{n_bad} bad, worst {worst:.3g}"


def test_small_grid_batched(f):
    """A batch on the 64x64 tiles (3 problems of 300x200x1000: 60 tiles in all)
    and on the wide tiles (M <= 32), each problem checked."""
    rng = np.random.default_rng(62)
    for (P, M, N, K), plan in (((3, 300, 200, 1000), "wg64x64_"), ((2, 20, 700, 640), "wide32x64_")):
        assert f.plan(M, N, K, P).startswith(plan)
        A = inputs.uniform_f16((P, M, K), rng)
        B = inputs.uniform_f16((P, N, K), rng)
        out = f.gemm_nt_batched(_dev(A), _dev(B))
        torch.cuda.synchronize()
        ref, bound = oracle.gemm_nt_batched(A, B)
        ok, worst, n_bad = oracle.within_bound(out.cpu().numpy(), ref, bound)
        assert ok, f"{plan} batch: {n_bad} bad, worst {worst:.3g}"


def test_two_streams_at_once(f):
    """The library keeps no device state between calls: products and fragment
    copies enqueued on two streams (default priority) that run concurrently
    give the results each gives alone."""
    rng = np.random.default_rng(61)
    A1, B1 = inputs.uniform_f16((1000, 600), rng), inputs.uniform_f16((700, 600), rng)
    A2, B2 = inputs.uniform_f16((2304, 384), rng), inputs.uniform_f16((2048, 384), rng)
    img = inputs.random_bits_u16(64 * 4 * 4096, rng)
    a1, b1, a2, b2 = _dev(A1), _dev(B1), _dev(A2), _dev(B2)
    src = torch.from_numpy(img.view(np.int16)).cuda()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs1, outs2, frags = [], [], []
    for _ in range(4):
        with torch.cuda.stream(s1):
            outs1.append(f.gemm_nt(a1, b1))
            frags.append(f.frag_copy(src, torch.empty_like(src), 4, False, 0))
        with torch.cuda.stream(s2):
            outs2.append(f.gemm_nt(a2, b2))
    torch.cuda.synchronize()
    want_frag = oracle.frag_load(img, 4, False)
    for o1, o2, fr in zip(outs1, outs2, frags):
        _assert_parity(o1.cpu().numpy(), A1, B1)
        _assert_parity(o2.cpu().numpy(), A2, B2)
        assert np.array_equal(fr.cpu().numpy().view(np.uint32), want_frag)
    assert all(torch.equal(o, outs1[0]) for o in outs1) and all(torch.equal(o, outs2[0]) for o in outs2)


def test_hip_graph_replays(f):
    """The calls enqueue kernels only (no allocation, no host synchronisation), so
    they can be captured in a HIP graph: each replay, with new operand values
    written eagerly between replays, matches the oracle."""
    rng = np.random.default_rng(71)
    M, N, K = 640, 384, 320
    a = torch.empty((M, K), dtype=torch.float16, device="cuda")
    b = torch.empty((N, K), dtype=torch.float16, device="cuda")
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    src = torch.empty(64 * 2 * 1000, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm the binding and library on the side stream
        f.gemm_nt(a, b, out=out)
        f.frag_copy(src, dst, 2, True, 0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f.gemm_nt(a, b, out=out)
        f.frag_copy(src, dst, 2, True, 0)
    for _ in range(3):
        A, B = inputs.uniform_f16((M, K), rng), inputs.uniform_f16((N, K), rng)
        img = inputs.random_bits_u16(src.numel(), rng)
        a.copy_(torch.from_numpy(A))
        b.copy_(torch.from_numpy(B))
        src.copy_(torch.from_numpy(img.view(np.int16)))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _assert_parity(out.cpu().numpy(), A, B)
        assert np.array_equal(dst.cpu().numpy().view(np.uint32), oracle.frag_load(img, 2, True))
