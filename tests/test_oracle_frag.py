"""Pins of the fragment-copy oracle (the ldmatrix/stmatrix model).

Pinned against: the ldstmatrix page's demo and its step-2/step-3 rules, a
closed form on index-valued tiles, the page-1 fragment layouts (an independent
statement of the same lane map), row/column-major equivalence, and the
inverse pair load/store on raw bit patterns including NaN payloads.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import page1
from fp16_matrix_core_amd import inputs


def _tiles_index_valued(G, num):
    """tiles[g, t, r, c] = a distinct 16-bit label per element: (g*num + t) * 64 + 8 r + c (mod 2**16)."""
    g = np.arange(G)[:, None, None, None]
    t = np.arange(num)[None, :, None, None]
    r = np.arange(8)[None, None, :, None]
    c = np.arange(8)[None, None, None, :]
    return (((g * num + t) * 64 + 8 * r + c) % 65536).astype(np.uint16)


def _image_row_major(tiles):
    """Group image with the tiles side by side: an 8 x (8 num) row-major matrix per group."""
    G, num = tiles.shape[:2]
    return np.concatenate([tiles[:, t] for t in range(num)], axis=2).reshape(G, -1).reshape(-1)


def _image_col_major(tiles):
    """Group image with each tile stored column by column (its transpose row-major), tiles back to back."""
    G, num = tiles.shape[:2]
    return np.ascontiguousarray(tiles.transpose(0, 1, 3, 2)).reshape(-1)


def _closed_form_fragment(tiles):
    """F[g, lane, t] = tile(lane//4, 2 (lane%4)) | tile(lane//4, 2 (lane%4) + 1) << 16."""
    G, num = tiles.shape[:2]
    F = np.zeros((G, 32, num), dtype=np.uint32)
    for lane in range(32):
        r, cp = divmod(lane, 4)
        lo = tiles[:, :, r, 2 * cp].astype(np.uint32)
        hi = tiles[:, :, r, 2 * cp + 1].astype(np.uint32)
        F[:, lane, :] = lo | (hi << 16)
    return F.reshape(-1)


def test_demo_fit_and_register_rule(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "ldstmatrix_demo.json")))
    num = spec["num"]
    shape, strides = oracle.shared_layout(num, col_major=False)
    assert list(shape) == spec["shared_layout_row_major"]["shape"]
    assert list(strides) == spec["shared_layout_row_major"]["strides"]
    assert oracle.fit_shared_layout(strides) == (spec["expected_fit"]["trans"], spec["expected_fit"]["p"])
    rshape, rstrides = oracle.register_layout(num)
    assert list(rshape) == spec["register_layout"]["shape"]
    lane_st = [s if k == "lane" else 0 for k, s in rstrides]
    reg_st = [s if k == "reg" else 0 for k, s in rstrides]
    assert lane_st == spec["register_layout"]["lane_strides"]
    assert reg_st == spec["register_layout"]["reg_strides"]
    # step 2: the (8, 4, 2) strides of the register side
    assert (rstrides[0][1], rstrides[1][1], rstrides[3][1]) == tuple(spec["register_strides_required"])
    # "lane i holds row i // 4, column pair i % 4" on the demo's 8 x 16 matrix
    M, N = spec["M"], spec["N"]
    mat = (np.arange(M * N) % 65536).astype(np.uint16)           # element (r, c) labelled r * N + c
    F = oracle.frag_load(mat, num, col_major=False).reshape(32, num)
    for lane in range(32):
        r, cp = divmod(lane, 4)
        for t in range(num):
            c = 8 * t + 2 * cp
            assert F[lane, t] == (r * N + c) | ((r * N + c + 1) << 16)


@pytest.mark.parametrize("num", [1, 2, 4])
def test_col_major_layout_fits_transposing_form(num):
    _, st = oracle.shared_layout(num, col_major=True)
    assert oracle.fit_shared_layout(st) == (True, 8)
    _, st = oracle.shared_layout(num, col_major=False)
    assert oracle.fit_shared_layout(st) == (False, 8 * num)
    # layouts that break step 3 are refused
    assert oracle.fit_shared_layout((12, 2, 8, 1)) is None      # row stride not a multiple of 8
    assert oracle.fit_shared_layout((1, 8, 64, 4)) is None      # column stride not a multiple of 8
    assert oracle.fit_shared_layout((1, 24, 64, 8)) is None     # s4 != 2 s2


@pytest.mark.parametrize("num", [1, 2, 4])
@pytest.mark.parametrize("col_major", [False, True])
def test_closed_form_on_labelled_tiles(num, col_major):
    G = 5
    tiles = _tiles_index_valued(G, num)
    img = _image_col_major(tiles) if col_major else _image_row_major(tiles)
    F = oracle.frag_load(img, num, col_major)
    assert np.array_equal(F, _closed_form_fragment(tiles))
    assert np.array_equal(oracle.frag_store(F, num, col_major), img)


@pytest.mark.parametrize("num", [1, 2, 4])
def test_row_and_col_major_give_the_same_fragment(num):
    rng = np.random.default_rng(20 + num)
    G = 64
    tiles = rng.integers(0, 1 << 16, size=(G, num, 8, 8), dtype=np.uint16)
    f_row = oracle.frag_load(_image_row_major(tiles), num, False)
    f_col = oracle.frag_load(_image_col_major(tiles), num, True)
    assert np.array_equal(f_row, f_col)


def _special_bits(n, rng):
    bits = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    specials = np.array([0x7C00, 0xFC00, 0x7E00, 0x7C01, 0xFE37, 0x0001, 0x8001, 0x03FF, 0x8000, 0x0000],
                        dtype=np.uint16)
    bits[:specials.size] = specials
    return bits


@pytest.mark.parametrize("num", [1, 2, 4])
@pytest.mark.parametrize("col_major", [False, True])
def test_load_store_are_inverse_on_raw_bits(num, col_major):
    rng = np.random.default_rng(30 + num + 10 * col_major)
    img = _special_bits(96 * 64 * num, rng)
    F = oracle.frag_load(img, num, col_major)
    assert np.array_equal(oracle.frag_store(F, num, col_major), img)
    assert np.array_equal(oracle.frag_roundtrip(img, num, col_major), img)
    words = rng.integers(0, 1 << 32, size=96 * 32 * num, dtype=np.uint32)
    assert np.array_equal(oracle.frag_load(oracle.frag_store(words, num, col_major), num, col_major), words)
    # the load only moves 16-bit patterns: the multiset of halves is unchanged
    halves = np.concatenate([(F & 0xFFFF).astype(np.uint16), (F >> 16).astype(np.uint16)])
    assert np.array_equal(np.sort(halves), np.sort(img))


def test_recipe_bits_include_nan_payloads():
    bits = inputs.frag_bits(n_tiles=4096)
    exp = (bits >> 10) & 0x1F
    mant = bits & 0x3FF
    assert np.any((exp == 31) & (mant != 0))          # NaNs
    assert np.any((exp == 0) & (mant != 0))           # subnormals
    F = oracle.frag_load(bits, 4, True)
    assert np.array_equal(oracle.frag_store(F, 4, True), bits)


def test_page1_a_fragment_matches_ldstmatrix_model():
    """x4 load of A's four 8x8 word matrices = frag_load(num=4) of the same matrices as one group."""
    A, _ = inputs.single_tile(0)
    words = page1.a_words(A)                                     # (4, 8, 4) uint32
    regs = page1.load_fragments(words, page1.A_LOAD, 4)          # (32 lanes, 4 regs)
    halves = words.view(np.uint16).reshape(4, 8, 8)              # tile t = matrix t, little-endian pairs
    group = _image_row_major(halves[None])
    F = oracle.frag_load(group, 4, False).reshape(32, 4)
    assert np.array_equal(F, regs)


def test_page1_b_fragment_matches_ldstmatrix_model():
    _, B = inputs.single_tile(0)
    words = page1.b_words(B)
    regs = page1.load_fragments(words, page1.B_LOAD, 2)
    halves = words.view(np.uint16).reshape(2, 8, 8)
    F = oracle.frag_load(_image_row_major(halves[None]), 2, False).reshape(32, 2)
    assert np.array_equal(F, regs)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.frag_load(np.zeros(64 * 3, np.uint16), 3, False)
    with pytest.raises(ValueError):
        oracle.frag_load(np.zeros(64 * 2 + 8, np.uint16), 2, False)
    with pytest.raises(ValueError):
        oracle.frag_store(np.zeros(33, np.uint32), 1, False)


@pytest.mark.parametrize("num", [1, 2, 4])
@pytest.mark.parametrize("col_major", [False, True])
def test_image_index_names_the_element_the_image_builders_place(num, col_major):
    """image_index against images built by concatenation / transposition (no stride arithmetic):
    every (r, c, t) lands on its own label, and the offsets cover one group image exactly once."""
    tiles = _tiles_index_valued(1, num)
    image = _image_col_major(tiles) if col_major else _image_row_major(tiles)
    seen = []
    for t in range(num):
        for r in range(8):
            for c in range(8):
                off = oracle.image_index(num, col_major, r, c, t)
                assert image[off] == tiles[0, t, r, c], (num, col_major, r, c, t, off)
                seen.append(off)
    assert sorted(seen) == list(range(64 * num))
