"""Pins of the page-1 lane-map model, and through it of the GEMM oracle's orientation."""

import json
import os

import numpy as np

import oracle
from oracle import page1
from fp16_matrix_core_amd import inputs


def test_lane0_cells(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "page1_lane0.json")))
    cells = [list(page1.scatter_cell(spec["lane"], r)) for r in range(4)]
    assert cells == spec["cells_for_dr_0_to_3"]


def test_d_layout_equals_scatter_formula():
    for i in range(16):
        for j in range(8):
            lane, reg = page1.evaluate(page1.D_MMA, (0, 0, i // 8, i % 8, j // 2, j % 2))
            assert page1.scatter_cell(lane, reg) == (i, j)


def test_scatter_covers_out_once():
    cells = {page1.scatter_cell(lane, r) for lane in range(32) for r in range(4)}
    assert cells == {(i, j) for i in range(16) for j in range(8)}


def test_a_load_and_a_mma_place_every_word_identically():
    """Word (i, kw) of A: where the x4 load puts it == where the MMA view reads it."""
    A = np.arange(256, dtype=np.uint16).view(np.float16).reshape(16, 16)
    regs = page1.load_fragments(page1.a_words(A), page1.A_LOAD, 4)
    wA = A.view(np.uint32)                                  # (16, 8) words
    for i in range(16):
        for kw in range(8):
            lane, reg = page1.evaluate(page1.A_MMA, (0, 0, i // 8, i % 8, kw // 4, kw % 4))
            assert regs[lane, reg] == wA[i, kw]


def test_b_load_and_b_mma_place_every_word_identically():
    B = np.arange(128, dtype=np.uint16).view(np.float16).reshape(8, 16)
    regs = page1.load_fragments(page1.b_words(B), page1.B_LOAD, 2)
    wB = B.view(np.uint32)
    for j in range(8):
        for kw in range(8):
            lane, reg = page1.evaluate(page1.B_MMA, (0, 0, j, kw // 4, kw % 4))
            assert regs[lane, reg] == wB[j, kw]


def test_simulated_example_equals_oracle():
    """The page-1 data flow (load, MMA view, D layout, scatter) reproduces oracle.gemm_nt exactly (K=16)."""
    A, B = inputs.single_tile(0)
    out = page1.simulate_warp_matmul(A, B)
    ref, _ = oracle.gemm_nt(A, B)
    assert np.array_equal(out, ref)
    # and with integer-valued inputs where any mistaken routing changes the value
    rng = np.random.default_rng(99)
    A = rng.integers(-50, 50, size=(16, 16)).astype(np.float16)
    B = rng.integers(-50, 50, size=(8, 16)).astype(np.float16)
    assert np.array_equal(page1.simulate_warp_matmul(A, B), oracle.gemm_nt(A, B)[0])


def test_fragment_sizes_match_table():
    """ar: 4 words, br: 2 words, dr: 4 floats per lane over 32 lanes (the page's fragment table)."""
    a_regs = {page1.evaluate(page1.A_LOAD, idx) for idx in np.ndindex(4, 8, 4)}
    b_regs = {page1.evaluate(page1.B_LOAD, idx) for idx in np.ndindex(2, 8, 4)}
    d_regs = {page1.evaluate(page1.D_MMA, idx) for idx in np.ndindex(1, 1, 2, 8, 4, 2)}
    assert a_regs == {(l, r) for l in range(32) for r in range(4)}
    assert b_regs == {(l, r) for l in range(32) for r in range(2)}
    assert d_regs == {(l, r) for l in range(32) for r in range(4)}
