"""Host-only checks: the layout module (compiled for the host), the C ABI's
exported symbols, its argument validation and its plan selection.  No call
here reaches the GPU: every call either fails validation or is empty, and
both return before any HIP runtime call."""

import ctypes
import os
import re
import subprocess

import pytest

from fp16_matrix_core_amd import build as fbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp16mc.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fbuild.LIB_PATH):
        fbuild.build()
    import fp16_matrix_core_amd as f
    return f.lib()


def test_layout_module_on_host(tmp_path):
    exe = tmp_path / "test_layout"
    cmd = [fbuild.HIPCC, "-x", "hip", f"--offload-arch={fbuild.ARCH}", "-O1", "-std=c++17",
           "-I", fbuild.CSRC, os.path.join(ROOT, "tests", "host", "test_layout.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    out = subprocess.run([str(exe)], stdout=subprocess.PIPE, text=True)
    assert out.returncode == 0, out.stdout
    assert out.stdout.startswith("OK"), out.stdout


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert {"gemm_nt_f16f32", "gemm_nt_f16f32_batched", "gemm_nt_ex", "gemm_ex", "frag_copy",
            "fp16mc_last_error", "gemm_nt_f16f32_plan", "gemm_ex_plan"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    nm = subprocess.run(["nm", "-D", "--defined-only", fbuild.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, flags=re.M), f"{n} is not a defined text symbol"


def test_binding_has_every_entry_point_by_its_c_name():
    """The Python binding offers each declared function under its C name (frag_copy's
    pointer-level form is frag_copy_raw; fp16mc_last_error feeds the exceptions)."""
    import inspect
    import fp16_matrix_core_amd as f
    for n in _declared_functions():
        if n == "fp16mc_last_error":
            continue
        py = "frag_copy_raw" if n == "frag_copy" else n
        assert callable(getattr(f, py, None)), f"binding lacks {py}"
    # pointer-level functions take the C arguments in the C order (stream last, optional)
    assert list(inspect.signature(f.gemm_nt_f16f32).parameters)[:9] == \
        ["a_ptr", "b_ptr", "out_ptr", "M", "N", "K", "lda", "ldb", "ldo"]
    assert list(inspect.signature(f.gemm_ex).parameters)[-1] == "stream"


def test_binding_c_names_validate_like_the_library(L):
    import fp16_matrix_core_amd as f
    with pytest.raises(f.Fp16mcError, match="lda=8 < K=16"):
        f.gemm_nt_f16f32(FAKE, FAKE, FAKE, 8, 8, 16, 8, 16, 8)
    with pytest.raises(f.Fp16mcError, match="overlap"):
        f.gemm_nt_f16f32_batched(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 2, 128, 128, 0)
    with pytest.raises(f.Fp16mcError, match="ab_type=3"):
        f.gemm_nt_ex(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 1, 0, 0, 0, 3, 0, 0)
    with pytest.raises(f.Fp16mcError, match="a_order=2"):
        f.gemm_ex(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 1, 0, 0, 0, 2, 0, 1, 0, 0)
    assert f.gemm_nt_f16f32_plan(8192, 8192, 8192) == L.gemm_nt_f16f32_plan(8192, 8192, 8192, 1).decode()
    assert f.gemm_ex_plan(8192, 8192, 8192, 1, 1, 1) == L.gemm_ex_plan(8192, 8192, 8192, 1, 1, 1).decode()


FAKE = 0x1000       # never dereferenced: every call below fails validation first
MISALIGNED = 0x1002


@pytest.mark.parametrize("args,code,needle", [
    ((FAKE, FAKE, FAKE, -1, 8, 8, 8, 8, 8), -1, "negative size"),
    ((FAKE, FAKE, FAKE, 8, 8, 16, 8, 16, 8), -1, "lda=8 < K=16"),
    ((FAKE, FAKE, FAKE, 8, 8, 16, 16, 8, 8), -1, "ldb=8 < K=16"),
    ((FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 4), -1, "ldo=4 < N=8"),
    ((0, FAKE, FAKE, 8, 8, 16, 16, 16, 8), -1, "NULL"),
    ((FAKE, FAKE, 0, 8, 8, 16, 16, 16, 8), -1, "Out is NULL"),
    ((MISALIGNED, FAKE, FAKE, 8, 8, 16, 16, 16, 8), -2, "16-byte aligned"),
    ((FAKE, FAKE, FAKE, 8, 8, 12, 12, 16, 8), -2, "multiples of 8"),
    ((FAKE, FAKE, FAKE, 8, 6, 16, 16, 16, 6), -2, "ldo=6"),
    ((FAKE, FAKE, MISALIGNED, 8, 8, 16, 16, 16, 8), -2, "Out must be 16-byte aligned"),
])
def test_gemm_validation(L, args, code, needle):
    rc = L.gemm_nt_f16f32(*args, None)
    assert rc == code
    assert needle in L.fp16mc_last_error().decode()


def test_gemm_rejects_tiles_beyond_32bit_offsets(L):
    # 8192 x 8192 problem with a huge row stride: validated before any HIP call
    ld = 1 << 24
    assert L.gemm_nt_f16f32(FAKE, FAKE, FAKE, 8192, 8192, 8192, ld, ld, 8192, None) == -1
    assert "2^32" in L.fp16mc_last_error().decode()


def test_gemm_rejects_output_tiles_beyond_31bit_offsets(L):
    # 8192^3 runs 256x256 tiles: 256 rows of Out at ldo = 2^21 fp32 or 2^22
    # fp16 elements span 2^31 bytes, rejected before any HIP call
    n, ld = 8192, 1 << 21
    assert L.gemm_nt_f16f32_plan(n, n, n, 1).decode().startswith("wg256x256")
    assert L.gemm_nt_f16f32(FAKE, FAKE, FAKE, n, n, n, n, n, ld, None) == -1
    assert "2^31" in L.fp16mc_last_error().decode()
    assert L.gemm_nt_ex(FAKE, FAKE, FAKE, n, n, n, n, n, 2 * ld, 1, 0, 0, 0, 1, 1, 0, None) == -1
    assert "2^31" in L.fp16mc_last_error().decode()


def test_gemm_batched_validation(L):
    assert L.gemm_nt_f16f32_batched(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, -1, 0, 0, 0, None) == -1
    assert L.gemm_nt_f16f32_batched(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 2, 12, 128, 64, None) == -2
    assert L.gemm_nt_f16f32_batched(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 2, -8, 128, 64, None) == -1


def test_huge_sizes_are_refused_not_wrapped(L):
    # sizes whose tile counts or byte offsets would overflow 64-bit arithmetic
    big = 1 << 62
    assert L.gemm_nt_f16f32(FAKE, FAKE, FAKE, big, big, 16, 16, 16, big, None) == -1
    assert "workgroups" in L.fp16mc_last_error().decode()
    assert L.gemm_nt_f16f32_batched(FAKE, FAKE, FAKE, 1 << 40, 1 << 40, 16, 16, 16, 1 << 40, 1, 0, 0, 0,
                                    None) == -1
    assert "workgroups" in L.fp16mc_last_error().decode()
    assert L.gemm_nt_f16f32(FAKE, FAKE, FAKE, 4096, 4096, 16, 1 << 60, 16, 4096, None) == -1
    assert "2^32" in L.fp16mc_last_error().decode()
    assert L.gemm_nt_f16f32(FAKE, FAKE, FAKE, 4096, 4096, 16, 16, 16, 1 << 61, None) == -1
    assert "2^31" in L.fp16mc_last_error().decode()
    assert L.gemm_nt_f16f32_batched(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 1 << 20, 1 << 50, 0, 64, None) == -1
    assert "overflows" in L.fp16mc_last_error().decode()


def test_gemm_batched_outputs_may_not_overlap(L):
    # M = 8 rows of N = 8 at ldo = 8: a problem's output spans 64 elements
    for so in (0, 8, 60):
        assert L.gemm_nt_f16f32_batched(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 2, 128, 128, so, None) == -1
        assert "overlap" in L.fp16mc_last_error().decode()
    # with ldo = 12 the last row ends at 7*12 + 8 = 92 elements
    assert L.gemm_nt_f16f32_batched(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 12, 2, 128, 128, 88, None) == -1
    # shared operands (strides 0) do not excuse overlapping outputs
    assert L.gemm_nt_f16f32_batched(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 2, 0, 0, 30, None) == -1
    assert "overlap" in L.fp16mc_last_error().decode()
    # an output span past 64-bit offsets is refused, not wrapped
    big = 1 << 40
    assert L.gemm_nt_f16f32_batched(FAKE, FAKE, FAKE, big, 8, 16, 16, 16, big, 2, 0, 0, 0, None) == -1
    assert "overflow" in L.fp16mc_last_error().decode()


# gemm_nt_ex(A, B, Out, M, N, K, lda, ldb, ldo, batch, sA, sB, sO, ab_type, out_type, accumulate)
EX_OK = (FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 1, 0, 0, 0)


@pytest.mark.parametrize("tail,code,needle", [
    ((0, 0, 0), -1, "ab_type=0"),
    ((3, 0, 0), -1, "ab_type=3"),
    ((1, 2, 0), -1, "out_type=2"),
    ((2, 1, 0), -1, "out_type=1"),
    ((1, 0, 2), -1, "accumulate"),
    ((1, 0, -1), -1, "accumulate"),
])
def test_gemm_ex_type_validation(L, tail, code, needle):
    assert L.gemm_nt_ex(*EX_OK, *tail, None) == code
    assert needle in L.fp16mc_last_error().decode()


def test_gemm_ex_output_alignment_follows_the_output_type(L):
    # ldo = 12: a multiple of 4 (16 bytes of fp32) but not of 8 (16 bytes of fp16 / bf16)
    base = (FAKE, FAKE, FAKE, 8, 12, 16, 16, 16, 12, 1, 0, 0, 0)
    for ab, out in ((1, 1), (2, 2)):
        assert L.gemm_nt_ex(*base, ab, out, 0, None) == -2
        assert "multiple of 8" in L.fp16mc_last_error().decode()
    # batched: strideO must be a multiple of 8 for 16-bit outputs
    assert L.gemm_nt_ex(FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 2, 128, 128, 68, 1, 1, 1, None) == -2
    # the old entry points are gemm_nt_ex(F16, F32, fresh): same checks, same codes
    assert L.gemm_nt_ex(*EX_OK[:8], 4, 1, 0, 0, 0, 1, 0, 0, None) == -1
    assert L.gemm_nt_f16f32(*EX_OK[:8], 4, None) == -1


def test_gemm_ex_storage_order_validation(L):
    # gemm_ex(..., a_order, b_order, ab_type, out_type, accumulate)
    base = (FAKE, FAKE, FAKE, 8, 8, 16, 16, 16, 8, 1, 0, 0, 0)
    assert L.gemm_ex(*base, 2, 0, 1, 0, 0, None) == -1
    assert "a_order=2" in L.fp16mc_last_error().decode()
    assert L.gemm_ex(*base, 0, -1, 1, 0, 0, None) == -1
    # A stored K x M needs lda >= M (not K); B stored K x N needs ldb >= N
    assert L.gemm_ex(FAKE, FAKE, FAKE, 64, 8, 16, 32, 16, 8, 1, 0, 0, 0, 1, 0, 1, 0, 0, None) == -1
    assert "lda=32 < M=64" in L.fp16mc_last_error().decode()
    assert L.gemm_ex(FAKE, FAKE, FAKE, 8, 64, 16, 16, 32, 64, 1, 0, 0, 0, 0, 1, 1, 0, 0, None) == -1
    assert "ldb=32 < N=64" in L.fp16mc_last_error().decode()
    # ... while lda < K is fine: this call passes the stride checks and stops at the NULL Out
    assert L.gemm_ex(FAKE, FAKE, 0, 64, 8, 4096, 64, 4096, 8, 1, 0, 0, 0, 1, 0, 1, 0, 0, None) == -1
    assert "Out is NULL" in L.fp16mc_last_error().decode()
    # a K x W operand is addressed 64 rows at a time: 2 * 64 * ld must stay below 2^32
    ld = 1 << 25
    assert L.gemm_ex(FAKE, FAKE, FAKE, 8192, 8192, 8192, ld, 8192, 8192, 1, 0, 0, 0, 1, 0, 1, 0, 0, None) == -1
    assert "2^32" in L.fp16mc_last_error().decode()


def test_plans_by_storage_order(L):
    import fp16_matrix_core_amd as f
    for order in ((0, 0), (1, 0), (0, 1), (1, 1)):
        assert f.plan_ex(100, 8, 64, 1, *order).startswith("tall64x32")
        assert f.plan_ex(100, 40, 64, 1, *order).startswith("wg128x64_")
        assert f.plan_ex(16, 8, 16, 1, *order).startswith("wave32x32")
        assert f.plan_ex(8192, 8192, 8192, 1, *order).startswith("wg256x256")
    # large tiles use 16x16x32 instructions for K-contiguous operands; with an
    # MN-contiguous operand the 256x256, 256x128 and 128x128 tiles do too, the
    # 128x64 ones 32x32x16
    for shape, name in (((8192, 8192, 8192), "wg256x256_w4"), ((8192, 1024, 8192), "wg256x128_w4"),
                        ((6144, 6144, 2048), "wg128x128_w4"), ((2048, 2048, 2048), "wg128x64_w4")):
        assert f.plan_ex(*shape, 1, 0, 0) == name + "_mfma16x16x32"
        assert f.plan(*shape) == name + "_mfma16x16x32"
        for order in ((1, 0), (0, 1), (1, 1)):
            mn_mfma = "_mfma32x32x16" if name == "wg128x64_w4" else "_mfma16x16x32"
            assert f.plan_ex(*shape, 1, *order) == name + mn_mfma
    assert f.plan(128, 64, 64, 4096) == "wg128x64s_w4_mfma32x32x16"
    assert f.plan(16384, 8, 16384) == "tall64x32_w2_mfma32x32x16"


def test_gemm_ex_empty_problems(L):
    for ab, out, acc in ((1, 0, 0), (1, 1, 1), (2, 0, 1), (2, 2, 0)):
        assert L.gemm_nt_ex(0, 0, 0, 0, 8, 16, 16, 16, 8, 1, 0, 0, 0, ab, out, acc, None) == 0
        assert L.gemm_nt_ex(0, 0, 0, 8, 8, 16, 16, 16, 8, 0, 0, 0, 0, ab, out, acc, None) == 0


def test_empty_problems_enqueue_nothing(L):
    # M == 0 or N == 0 or batch == 0: OK without touching pointers or the GPU
    assert L.gemm_nt_f16f32(0, 0, 0, 0, 8, 16, 16, 16, 8, None) == 0
    assert L.gemm_nt_f16f32(0, 0, 0, 8, 0, 16, 16, 16, 0, None) == 0
    assert L.gemm_nt_f16f32_batched(0, 0, 0, 8, 8, 16, 16, 16, 8, 0, 0, 0, 0, None) == 0
    assert L.frag_copy(0, 0, 0, 4, 0, 0, None) == 0


@pytest.mark.parametrize("args,code,needle", [
    ((FAKE, FAKE, 8, 3, 0, 0), -1, "1, 2 or 4 tiles"),
    ((FAKE, FAKE, 6, 4, 0, 0), -1, "not a multiple of num=4"),
    ((FAKE, FAKE, -4, 4, 0, 0), -1, "negative"),
    ((FAKE, FAKE, 8, 2, 2, 0), -1, "col_major"),
    ((FAKE, FAKE, 8, 2, 0, 3), -1, "direction"),
    ((0, FAKE, 8, 2, 0, 0), -1, "NULL"),
    ((MISALIGNED, FAKE, 8, 2, 0, 1), -2, "16-byte aligned"),
    ((FAKE, FAKE + 512, 8, 2, 0, 0), -1, "overlap"),          # 8 tiles = 1 KiB: dst starts inside src
    ((FAKE + 1008, FAKE, 8, 2, 0, 2), -1, "overlap"),         # dst's last 16 bytes are src's first
    ((FAKE, FAKE, 1 << 60, 4, 0, 0), -1, "address space"),    # 2^67 bytes
])
def test_frag_copy_validation(L, args, code, needle):
    assert L.frag_copy(*args, None) == code
    assert needle in L.fp16mc_last_error().decode()


def test_plans(L):
    import fp16_matrix_core_amd as f
    assert f.plan(0, 8, 8) is None
    assert f.plan(16, 8, 16).startswith("wave32x32")
    # K >= 512 and at most 256 tiles of 64x64: at most one 64x64 tile per CU
    assert f.plan(512, 512, 16384) == "wg64x64_w4_mfma16x16x32"
    assert f.plan(1024, 1024, 4096).startswith("wg64x64_")
    assert f.plan(1024, 1024, 512).startswith("wg64x64_")
    assert f.plan(1024, 1088, 4096).startswith("wg128x64_")
    assert f.plan(1024, 1024, 511).startswith("wg128x64_")
    assert f.plan_ex(1024, 1024, 4096, 1, 1, 0) == "wg64x64_w4_mfma32x32x16"
    assert f.plan(128, 64, 64).startswith("wg128x64_")
    assert f.plan(128, 64, 64, 4096).startswith("wg128x64s_")      # one-tile problems: streamed
    assert f.plan(129, 64, 64, 4096).startswith("wg128x64_")
    assert f.plan(8192, 8192, 8192).startswith("wg256x256")
    assert f.plan(8192, 1024, 8192).startswith("wg256x128")    # 256x256 tiles would fill half the CUs
    assert f.plan(6144, 6144, 2048).startswith("wg128x128")    # two workgroups per CU
    assert f.plan(3000, 5000, 704).startswith("wg128x128")
    assert f.plan(12288, 12288, 1024).startswith("wg256x256")  # many waves of tiles: largest tiles
    assert f.plan(2048, 2048, 2048).startswith("wg128x64_")
    assert f.plan(16384, 64, 4096).startswith("wg64x64_")      # 256 tiles of 64x64: one per CU
    assert f.plan(16384, 128, 4096).startswith("wg128x64_")    # 512 of them: the larger tiles win again
    assert f.plan(8, 16384, 16384).startswith("wide32x64")
    assert f.plan(16384, 8, 16384).startswith("tall64x32")
    assert f.plan(100, 32, 64).startswith("tall64x32")
    assert f.plan(100, 33, 64).startswith("wg128x64_")


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import fp16_matrix_core_amd as f
    monkeypatch.setattr(f, "_lib", None)
    monkeypatch.setattr(f, "_HERE", str(tmp_path))
    with pytest.raises(RuntimeError, match="not built"):
        f.lib()


def test_binding_rejects_host_tensors_before_any_call(monkeypatch):
    """Host tensors never reach the library: their addresses would be handed to the kernels."""
    torch = pytest.importorskip("torch")
    import fp16_matrix_core_amd as f

    def no_call():
        raise AssertionError("the library was reached with a host tensor")
    monkeypatch.setattr(f, "lib", no_call)
    a = torch.zeros((16, 16), dtype=torch.float16)
    b = torch.zeros((8, 16), dtype=torch.float16)
    out = torch.zeros((16, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        f.gemm_nt(a, b, out)
    with pytest.raises(ValueError, match="GPU tensor"):
        f.gemm_nt(a, b)
    with pytest.raises(ValueError, match="GPU tensor"):
        f.gemm_nt_batched(a[None], b[None], out[None])
    with pytest.raises(ValueError, match="GPU tensor"):
        f.matmul(a, b.t(), out)
    src = torch.zeros(64, dtype=torch.int16)
    with pytest.raises(ValueError, match="GPU tensor"):
        f.frag_copy(src, torch.zeros_like(src), 1, False, f.FRAG_LOAD)
