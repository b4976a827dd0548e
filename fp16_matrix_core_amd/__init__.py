"""fp16_matrix_core_amd -- Python binding of libfp16mc.so (MI355X / gfx950).

The binding marshals arguments only: every step of the product and of the
fragment copy runs in the HIP kernels of ``libfp16mc.so``.  PyTorch supplies
device memory and the current stream; nothing here computes on the CPU, and
every entry point raises if the library is not built.

    gemm_nt(a, b, out)             Out = A @ B.T  (fp16 or bf16 in, fp32 or the
                                   input type out; accumulate=True adds to out)
    gemm_nt_batched(a, b, out)     the same for (batch, M, K) x (batch, N, K)
    matmul(a, b, out)              Out = a @ b for (M,K) x (K,N) views with any
                                   contiguous dimension (the storage order of
                                   each operand is read from its strides)
    frag_copy(src, dst, num, col_major, direction)
    plan(M, N, K, batch=1)         name of the kernel configuration used

Pointer-level calls with the C ABI's names and argument order (integer
device pointers, the stream as an integer handle): gemm_nt_f16f32,
gemm_nt_f16f32_batched, gemm_nt_ex, gemm_ex, frag_copy_raw (the C frag_copy),
gemm_nt_f16f32_plan, gemm_ex_plan.  Status codes are those of
include/fp16mc.h; a nonzero status raises Fp16mcError with the library's
message.
"""

import ctypes
import os

__all__ = [
    "FRAG_LOAD", "FRAG_STORE", "FRAG_ROUNDTRIP", "Fp16mcError", "lib", "lib_path",
    "gemm_nt", "gemm_nt_batched", "frag_copy", "plan", "gemm_nt_raw", "gemm_nt_ex_raw", "frag_copy_raw",
    "F32", "F16", "BF16", "K_CONTIGUOUS", "MN_CONTIGUOUS", "matmul", "gemm_ex_raw", "plan_ex",
    "gemm_nt_f16f32", "gemm_nt_f16f32_batched", "gemm_nt_ex", "gemm_ex", "gemm_nt_f16f32_plan", "gemm_ex_plan",
]

FRAG_LOAD, FRAG_STORE, FRAG_ROUNDTRIP = 0, 1, 2
F32, F16, BF16 = 0, 1, 2
K_CONTIGUOUS, MN_CONTIGUOUS = 0, 1
STATUS = {0: "FP16MC_OK", -1: "FP16MC_EINVAL", -2: "FP16MC_EALIGN", -3: "FP16MC_EHIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfp16mc.so"
_lib = None


class Fp16mcError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib_path():
    return os.path.join(_HERE, _LIB_NAME)


def lib():
    """Load libfp16mc.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built; run `python -m fp16_matrix_core_amd.build` "
                "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.gemm_nt_f16f32.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
        L.gemm_nt_f16f32.restype = ci
        L.gemm_nt_f16f32_batched.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64, i64, vp]
        L.gemm_nt_f16f32_batched.restype = ci
        L.gemm_nt_ex.argtypes = [vp, vp, vp] + [i64] * 10 + [ci, ci, ci, vp]
        L.gemm_nt_ex.restype = ci
        L.gemm_ex.argtypes = [vp, vp, vp] + [i64] * 10 + [ci, ci, ci, ci, ci, vp]
        L.gemm_ex.restype = ci
        L.gemm_ex_plan.argtypes = [i64, i64, i64, i64, ci, ci]
        L.gemm_ex_plan.restype = ctypes.c_char_p
        L.frag_copy.argtypes = [vp, vp, i64, ci, ci, ci, vp]
        L.frag_copy.restype = ci
        L.gemm_nt_f16f32_plan.argtypes = [i64, i64, i64, i64]
        L.gemm_nt_f16f32_plan.restype = ctypes.c_char_p
        L.fp16mc_last_error.argtypes = []
        L.fp16mc_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise Fp16mcError(status, lib().fp16mc_last_error().decode())


def _require_device(ref, **tensors):
    """Every tensor must live on the GPU that holds ``ref``.

    The kernels take raw addresses: a host tensor's address handed to them
    would fault on the device instead of raising here.
    """
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the operands on {ref.device}")


def _stream_ptr(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _ld(t, rows, cols):
    """Row stride of a 2-D view; a single row may use any stride (it is never stepped)."""
    if t.stride(-1) != 1 and cols > 1:
        raise ValueError("innermost dimension must be contiguous")
    if rows > 1:
        return t.stride(-2)
    return max(cols, 1) + (-max(cols, 1)) % 8


def gemm_nt_raw(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, stream=0):
    """Direct call of gemm_nt_f16f32 with integer device pointers."""
    _check(lib().gemm_nt_f16f32(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, stream))


def gemm_nt_ex_raw(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, batch=1, sa=0, sb=0, so=0,
                   ab_type=F16, out_type=F32, accumulate=False, stream=0):
    """Direct call of gemm_nt_ex with integer device pointers."""
    _check(lib().gemm_nt_ex(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, batch, sa, sb, so,
                            ab_type, out_type, int(bool(accumulate)), stream))


def gemm_ex_raw(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, batch=1, sa=0, sb=0, so=0,
                a_order=K_CONTIGUOUS, b_order=K_CONTIGUOUS, ab_type=F16, out_type=F32, accumulate=False,
                stream=0):
    """Direct call of gemm_ex with integer device pointers."""
    _check(lib().gemm_ex(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, batch, sa, sb, so,
                         a_order, b_order, ab_type, out_type, int(bool(accumulate)), stream))


def frag_copy_raw(src_ptr, dst_ptr, num_tiles, num, col_major, direction, stream=0):
    """Direct call of frag_copy with integer device pointers."""
    _check(lib().frag_copy(src_ptr, dst_ptr, num_tiles, num, int(col_major), direction, stream))


def gemm_nt_f16f32(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, stream=0):
    """gemm_nt_f16f32 of the C ABI (integer device pointers)."""
    _check(lib().gemm_nt_f16f32(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, stream))


def gemm_nt_f16f32_batched(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, batch, stride_a, stride_b, stride_o,
                           stream=0):
    """gemm_nt_f16f32_batched of the C ABI (integer device pointers, strides in elements)."""
    _check(lib().gemm_nt_f16f32_batched(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, batch, stride_a,
                                        stride_b, stride_o, stream))


def gemm_nt_ex(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, batch, stride_a, stride_b, stride_o, ab_type,
               out_type, accumulate, stream=0):
    """gemm_nt_ex of the C ABI (integer device pointers)."""
    _check(lib().gemm_nt_ex(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, batch, stride_a, stride_b, stride_o,
                            ab_type, out_type, int(accumulate), stream))


def gemm_ex(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, batch, stride_a, stride_b, stride_o, a_order, b_order,
            ab_type, out_type, accumulate, stream=0):
    """gemm_ex of the C ABI (integer device pointers)."""
    _check(lib().gemm_ex(a_ptr, b_ptr, out_ptr, M, N, K, lda, ldb, ldo, batch, stride_a, stride_b, stride_o,
                         a_order, b_order, ab_type, out_type, int(accumulate), stream))


def gemm_nt_f16f32_plan(M, N, K, batch=1):
    """gemm_nt_f16f32_plan of the C ABI: the kernel configuration's name, or None."""
    return plan(M, N, K, batch)


def gemm_ex_plan(M, N, K, batch=1, a_order=K_CONTIGUOUS, b_order=K_CONTIGUOUS):
    """gemm_ex_plan of the C ABI."""
    return plan_ex(M, N, K, batch, a_order, b_order)


def _types(a, b, out_dtype):
    import torch
    codes = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    if a.dtype not in (torch.float16, torch.bfloat16) or b.dtype != a.dtype:
        raise TypeError("a and b must both be float16 or both bfloat16")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if out_dtype not in (torch.float32, a.dtype):
        raise TypeError("out must be float32 or the inputs' dtype")
    return codes[a.dtype], codes[out_dtype], out_dtype


def gemm_nt(a, b, out=None, accumulate=False, out_dtype=None):
    """Out = A @ B.T (+ out if accumulate) on the GPU.

    a: (M,K), b: (N,K), both float16 or both bfloat16; out: (M,N) float32 or
    the inputs' dtype (allocated, with 16-byte-aligned rows, if None; then
    ``out_dtype`` picks its type and accumulate must be False).
    """
    import torch
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} do not form A @ B.T")
    M, K = a.shape
    N = b.shape[0]
    _require_device(a, a=a, b=b)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out")
        ab, ot, odt = _types(a, b, out_dtype)
        per16 = 16 // torch.empty((), dtype=odt).element_size()
        out = torch.empty((M, N + (-N) % per16), dtype=odt, device=a.device)[:, :N]
    else:
        ab, ot, _ = _types(a, b, out.dtype)
    _require_device(a, out=out)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must have shape (M, N)")
    _check(lib().gemm_nt_ex(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                            _ld(a, M, K), _ld(b, N, K), _ld(out, M, N), 1, 0, 0, 0,
                            ab, ot, int(bool(accumulate)), _stream_ptr(a)))
    return out


def gemm_nt_batched(a, b, out=None, accumulate=False, out_dtype=None):
    """Batched Out[p] = A[p] @ B[p].T (+ out[p]). a: (P,M,K), b: (P,N,K); types as gemm_nt."""
    import torch
    if a.dim() != 3 or b.dim() != 3 or a.shape[0] != b.shape[0] or a.shape[2] != b.shape[2]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} do not form batched A @ B.T")
    P, M, K = a.shape
    N = b.shape[1]
    _require_device(a, a=a, b=b)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out")
        ab, ot, odt = _types(a, b, out_dtype)
        per16 = 16 // torch.empty((), dtype=odt).element_size()
        out = torch.empty((P, M, N + (-N) % per16), dtype=odt, device=a.device)[:, :, :N]
    else:
        ab, ot, _ = _types(a, b, out.dtype)
    _require_device(a, out=out)
    if tuple(out.shape) != (P, M, N):
        raise ValueError("out must have shape (P, M, N)")
    _check(lib().gemm_nt_ex(
        a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
        _ld(a, M, K), _ld(b, N, K), _ld(out, M, N), P,
        a.stride(0) if P > 1 else 0, b.stride(0) if P > 1 else 0, out.stride(0) if P > 1 else 0,
        ab, ot, int(bool(accumulate)), _stream_ptr(a)))
    return out


def _order(t, contiguous_dim):
    """(storage order, leading dimension) of a 2-D operand view.

    ``contiguous_dim`` is the view dimension that indexes K.  A view whose K
    dimension has stride 1 is K-contiguous; one whose other dimension has
    stride 1 is stored with K indexing its rows.
    """
    other = 1 - contiguous_dim
    rows_k, rows_o = t.shape[contiguous_dim], t.shape[other]
    if t.stride(contiguous_dim) == 1 or rows_k <= 1:
        return K_CONTIGUOUS, (t.stride(other) if rows_o > 1 else max(rows_k, 1) + (-max(rows_k, 1)) % 8)
    if t.stride(other) == 1 or rows_o <= 1:
        return MN_CONTIGUOUS, (t.stride(contiguous_dim) if rows_k > 1 else max(rows_o, 1) + (-max(rows_o, 1)) % 8)
    raise ValueError("operand views need one dimension with stride 1")


def matmul(a, b, out=None, accumulate=False, out_dtype=None):
    """Out = a @ b (+ out if accumulate) for a (M, K) and b (K, N) views.

    Either operand may be K-contiguous or stored with K indexing its rows
    (e.g. ``x.t()`` of a row-major tensor); the storage order is read from the
    strides.  Types as gemm_nt.
    """
    import torch
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} do not form a @ b")
    M, K = a.shape
    N = b.shape[1]
    _require_device(a, a=a, b=b)
    a_order, lda = _order(a, 1)
    b_order, ldb = _order(b, 0)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out")
        ab, ot, odt = _types(a, b, out_dtype)
        per16 = 16 // torch.empty((), dtype=odt).element_size()
        out = torch.empty((M, N + (-N) % per16), dtype=odt, device=a.device)[:, :N]
    else:
        ab, ot, _ = _types(a, b, out.dtype)
    _require_device(a, out=out)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must have shape (M, N)")
    _check(lib().gemm_ex(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, _ld(out, M, N),
                         1, 0, 0, 0, a_order, b_order, ab, ot, int(bool(accumulate)), _stream_ptr(a)))
    return out


def frag_copy(src, dst, num, col_major, direction):
    """Fragment copy between two contiguous device buffers of num_tiles * 128 bytes each."""
    _require_device(src, src=src, dst=dst)
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or nbytes % 128:
        raise ValueError("src and dst must both hold a whole number of 128-byte tiles, same size")
    _check(lib().frag_copy(src.data_ptr(), dst.data_ptr(), nbytes // 128, num, int(bool(col_major)),
                           direction, _stream_ptr(src)))
    return dst


def plan(M, N, K, batch=1):
    name = lib().gemm_nt_f16f32_plan(M, N, K, batch)
    return name.decode() if name is not None else None


def plan_ex(M, N, K, batch=1, a_order=K_CONTIGUOUS, b_order=K_CONTIGUOUS):
    name = lib().gemm_ex_plan(M, N, K, batch, a_order, b_order)
    return name.decode() if name is not None else None
