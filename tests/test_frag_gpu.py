"""GPU parity of frag_copy against the bit-exact oracle (through the C ABI).

Bar: bit-exact, every word, every direction, for num in {1,2,4} and both
shared layouts; bytes past the end of dst stay untouched.
"""

import numpy as np
import pytest

import oracle
from fp16_matrix_core_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOAD, STORE, ROUNDTRIP = 0, 1, 2
TAIL = 256          # bytes of sentinel after dst
SENT = 0x5A


@pytest.fixture(scope="module")
def f():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp16_matrix_core_amd as f
    f.lib()
    return f


@pytest.fixture(scope="module")
def bits():
    return inputs.frag_bits()          # 2^20 tiles of random 16-bit patterns (seed 3)


def _copy(f, src_np, num, col, direction):
    """Run frag_copy on a byte copy of src_np; return dst bytes and the sentinel tail."""
    raw = np.ascontiguousarray(src_np).view(np.uint8)
    nbytes = raw.size
    src = torch.from_numpy(raw.copy()).cuda()
    dst = torch.full((nbytes + TAIL,), SENT, dtype=torch.uint8, device="cuda")
    f.frag_copy_raw(src.data_ptr(), dst.data_ptr(), nbytes // 128, num, col, direction,
                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = dst.cpu().numpy()
    return out[:nbytes], out[nbytes:]


def _check(got_bytes, want, tail):
    want_b = np.ascontiguousarray(want).view(np.uint8)
    if not np.array_equal(got_bytes, want_b):
        bad = np.flatnonzero(got_bytes != want_b)
        raise AssertionError(f"{bad.size} bytes differ, first at byte {bad[0]}")
    assert (tail == SENT).all(), "wrote past the end of dst"


@pytest.mark.parametrize("num", [1, 2, 4])
@pytest.mark.parametrize("col", [0, 1], ids=["row", "col"])
def test_full_size(f, bits, num, col):
    """2^20 tiles: load, store and roundtrip, bit-exact."""
    print(f"frag_copy full num={num} col={col}", flush=True)
    want_frag = oracle.frag_load(bits, num, col)
    got, tail = _copy(f, bits, num, col, LOAD)
    _check(got, want_frag, tail)
    words = bits.view(np.uint32)       # the same random patterns read as fragment words
    got, tail = _copy(f, words, num, col, STORE)
    _check(got, oracle.frag_store(words, num, col), tail)
    got, tail = _copy(f, bits, num, col, ROUNDTRIP)
    _check(got, bits, tail)


@pytest.mark.parametrize("num", [1, 2, 4])
@pytest.mark.parametrize("col", [0, 1], ids=["row", "col"])
@pytest.mark.parametrize("groups", [1, 2, 3, 31, 33, 127, 129, 1000])
def test_ragged_counts(f, num, col, groups):
    rng = np.random.default_rng(1000 * num + 10 * groups + col)
    img = inputs.random_bits_u16(groups * 64 * num, rng)
    got, tail = _copy(f, img, num, col, LOAD)
    _check(got, oracle.frag_load(img, num, col), tail)
    words = rng.integers(0, 1 << 32, size=groups * 32 * num, dtype=np.uint32)
    got, tail = _copy(f, words, num, col, STORE)
    _check(got, oracle.frag_store(words, num, col), tail)
    got, tail = _copy(f, img, num, col, ROUNDTRIP)
    _check(got, img, tail)


def test_special_patterns_survive(f):
    """NaN payloads, infinities, subnormals and -0 move as bits."""
    specials = np.array([0x7C00, 0xFC00, 0x7E00, 0x7C01, 0xFE37, 0x0001, 0x8001, 0x03FF, 0x8000, 0x0000,
                         0x7FFF, 0xFFFF], dtype=np.uint16)
    img = np.resize(specials, 64 * 4 * 8)
    for col in (0, 1):
        got, tail = _copy(f, img, 4, col, LOAD)
        _check(got, oracle.frag_load(img, 4, col), tail)
        got, tail = _copy(f, img, 4, col, ROUNDTRIP)
        _check(got, img, tail)


def test_torch_binding(f):
    rng = np.random.default_rng(77)
    img = inputs.random_bits_u16(64 * 2 * 50, rng)
    src = torch.from_numpy(img.view(np.int16)).cuda()
    dst = torch.empty_like(src)
    f.frag_copy(src, dst, 2, True, LOAD)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().view(np.uint32), oracle.frag_load(img, 2, True))


@pytest.mark.parametrize("num", [1, 2, 4])
@pytest.mark.parametrize("col", [0, 1], ids=["row", "col"])
def test_in_place(f, num, col):
    """src == dst: each direction gives what it gives out of place (a whole-block
    count and a ragged one, so a partial last block is covered too)."""
    for groups in (4096, 4099):
        rng = np.random.default_rng(500 + 10 * num + col + groups)
        img = inputs.random_bits_u16(groups * 64 * num, rng)
        for direction, want in ((LOAD, oracle.frag_load(img, num, col)),
                                (STORE, oracle.frag_store(img.view(np.uint32), num, col)),
                                (ROUNDTRIP, img)):
            buf = torch.from_numpy(img.view(np.uint8).copy()).cuda()
            f.frag_copy_raw(buf.data_ptr(), buf.data_ptr(), groups * num, num, col, direction,
                            torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            got = buf.cpu().numpy()
            assert np.array_equal(got, np.ascontiguousarray(want).view(np.uint8)), (groups, direction)
