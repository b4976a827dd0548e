"""Every kernel configuration (plan) of the product, under every storage order
and two type combinations, against the CPU oracle through the C ABI.

Each shape below is chosen so that the plan logic picks the named
configuration (asserted); shapes are ragged in M, N and K.  Every element
is checked, plus all-finite and untouched padding.  Out is
followed by GUARD rows of NaN that must stay untouched: the last row tile of
every shape reaches past M, and the kernels rely on the output buffer's
range to drop those rows.
"""

import zlib

import numpy as np
import pytest

import oracle
from fp16_matrix_core_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ORDER = {"k": 0, "mn": 1}
CODE = {"f32": 0, "f16": 1, "bf16": 2}
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}

PLAN_SHAPES = {
    "wave32x32": (31, 29, 70),
    "wg64x64": (300, 500, 4100),
    "tall64x32": (1000, 17, 300),
    "wide32x64": (20, 1000, 77),
    "wg128x64": (300, 520, 200),
    "wg128x128": (4100, 2050, 100),
    "wg256x128": (1003, 4105, 8200),
    "wg256x256": (8100, 2003, 4100),      # N % 8 = 3: 16-bit row pieces straddle N
}
ORDERS = [("k", "k"), ("k", "mn"), ("mn", "k"), ("mn", "mn")]
GUARD = 37
TYPES = [("f16", "f32", False), ("bf16", "bf16", True), ("f16", "f16", False)]


@pytest.fixture(scope="module")
def f():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp16_matrix_core_amd as f
    f.lib()
    return f


def _bits(X, fmt):
    return X.view(np.uint16) if fmt == "f16" else np.asarray(X, dtype=np.uint16)


def _stored(X, order, fmt):
    S = X if order == "k" else np.ascontiguousarray(X.T)
    R, W = S.shape
    ld = W + (-W) % 8 + 8
    buf = np.full((R, ld), NAN_BITS[fmt], np.uint16)
    buf[:, :W] = _bits(S, fmt)
    return torch.from_numpy(buf.view(np.int16)).cuda(), ld


@pytest.mark.parametrize("plan", list(PLAN_SHAPES))
@pytest.mark.parametrize("a_order,b_order", ORDERS)
@pytest.mark.parametrize("ab,out_fmt,acc", TYPES)
def test_plan(f, plan, a_order, b_order, ab, out_fmt, acc):
    M, N, K = PLAN_SHAPES[plan]
    _check_case(f, plan, M, N, K, a_order, b_order, ab, out_fmt, acc)


@pytest.mark.parametrize("K", [3136, 3140], ids=["49_slices", "49_slices_and_4"])
@pytest.mark.parametrize("a_order,b_order", ORDERS)
@pytest.mark.parametrize("ab,out_fmt,acc", TYPES)
def test_wg256x256_odd_slice_count(f, K, a_order, b_order, ab, out_fmt, acc):
    """The 256x256 K loop with an odd number of whole slices (no trailing phase
    after the paired ones), with and without a partial slice after them."""
    _check_case(f, "wg256x256", 4100, 2200, K, a_order, b_order, ab, out_fmt, acc)


def _check_case(f, plan, M, N, K, a_order, b_order, ab, out_fmt, acc):
    assert f.plan_ex(M, N, K, 1, ORDER[a_order], ORDER[b_order]).split("_")[0] == plan
    rng = np.random.default_rng(zlib.crc32(f"{plan}/{M}x{N}x{K}/{a_order}/{b_order}/{ab}".encode()))
    draw = inputs.uniform_f16 if ab == "f16" else inputs.uniform_bf16
    A = draw((M, K), rng)
    B = draw((N, K), rng)
    per16 = 4 if out_fmt == "f32" else 8
    ldo = N + 3
    ldo += (-ldo) % per16
    buf = torch.full((M + GUARD, ldo), float("nan"), dtype=TORCH[out_fmt], device="cuda")
    out = buf[:M]
    C = None
    if acc:
        C = torch.from_numpy(inputs.accumulator_f32((M, N), seed=M)).to(TORCH[out_fmt])
        out[:, :N] = C.cuda()
        C = C.double().numpy()
    pad_before = out[:, N:].clone()
    guard_before = buf[M:].clone()
    a, lda = _stored(A, a_order, ab)
    b, ldb = _stored(B, b_order, ab)
    f.gemm_ex_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldo, 1, 0, 0, 0,
                  ORDER[a_order], ORDER[b_order], CODE[ab], CODE[out_fmt], acc,
                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    view = torch.int16 if out_fmt != "f32" else torch.int32
    assert torch.equal(out[:, N:].view(view), pad_before.view(view)), "padding of Out written"
    assert torch.equal(buf[M:].view(view), guard_before.view(view)), "rows past M written"
    assert bool(torch.isfinite(out[:, :N]).all())
    got = out[:, :N].float().double().cpu().numpy()
    ref, bound = oracle.gemm_nt_ex(A, B, C, ab=ab)
    ok, worst, n_bad = oracle.within_bound_out(got, ref, bound, out_fmt)
    assert ok, f"{plan} {a_order}{b_order} {ab}->{out_fmt}: {n_bad} bad (worst {worst:.3g})"
