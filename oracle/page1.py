"""The single-warp m16n8k16 example, evaluated as written (test infrastructure only).

Follows "Warp Matrix Instructions", section "From Shared Memory to a Matrix
Product": the fragment table (ar: four uint32 words, br: two, dr: four
float32), the five layouts a_load, b_load, a_mma, b_mma, d_mma, the two uint32
rearranges that regroup the staged A and B into 8x8 matrices, the MMA's
(D, A, B, C) operand order with C = 0, and the final scatter of dr into Out
(the loop after the MMA and the prose that names lane 0's four cells).

Nothing here is used by the product path.  The module exists to pin the
``gemm`` and ``frag`` oracles to the pages: the fragment routes that the
page-1 layouts describe must agree with the ``frag`` model of the
ldstmatrix page, and the product they feed must equal the ``gemm`` definition.

A layout is written S[(shape) : (strides)]; a stride is either an int (a step
in the register index) or ("lane", k), meaning k @ laneid.
"""

import numpy as np

__all__ = [
    "A_LOAD", "B_LOAD", "A_MMA", "B_MMA", "D_MMA", "evaluate", "a_words", "b_words",
    "load_fragments", "simulate_warp_matmul", "scatter_cell",
]

L = "lane"

# The five layouts of the example, strides as printed on the page.
A_LOAD = ((4, 8, 4), (1, (L, 4), (L, 1)))
B_LOAD = ((2, 8, 4), (1, (L, 4), (L, 1)))
A_MMA = ((1, 1, 2, 8, 2, 4), (4, 4, 1, (L, 4), 2, (L, 1)))
B_MMA = ((1, 1, 8, 2, 4), (2, 2, (L, 4), 1, (L, 1)))
D_MMA = ((1, 1, 2, 8, 4, 2), (4, 4, 2, (L, 4), (L, 1), 1))


def evaluate(layout, coord):
    """(lane, register index) that a layout assigns to a coordinate."""
    shape, strides = layout
    if len(coord) != len(shape):
        raise ValueError("coordinate rank")
    lane = 0
    reg = 0
    for x, n, s in zip(coord, shape, strides):
        if not 0 <= x < n:
            raise IndexError(f"coordinate {coord} outside shape {shape}")
        if isinstance(s, tuple):
            lane += x * s[1]
        else:
            reg += x * s
    return lane, reg


def _u32_view(h):
    """fp16 (R, C) -> uint32 (R, C/2): bit view, two fp16 per word."""
    return np.ascontiguousarray(h, dtype=np.float16).view(np.uint32)


def a_words(A):
    """A (16,16) fp16 -> (4, 8, 4) uint32: "(group row) (chunk word) -> (chunk group) row word"."""
    w = _u32_view(A).reshape(2, 8, 2, 4)            # group, row, chunk, word
    return w.transpose(2, 0, 1, 3).reshape(4, 8, 4)  # (chunk group), row, word


def b_words(B):
    """B (8,16) fp16 -> (2, 8, 4) uint32: "row (chunk word) -> chunk row word"."""
    w = _u32_view(B).reshape(8, 2, 4)                # row, chunk, word
    return w.transpose(1, 0, 2).copy()


def load_fragments(words, layout, n_regs):
    """The ldmatrix step: place each (matrix, row, word) of ``words`` by ``layout``.

    Returns regs[lane, reg] uint32 for 32 lanes.
    """
    regs = np.zeros((32, n_regs), dtype=np.uint32)
    seen = np.zeros((32, n_regs), dtype=bool)
    for idx in np.ndindex(*words.shape):
        lane, reg = evaluate(layout, idx)
        if seen[lane, reg]:
            raise AssertionError("load layout not injective")
        seen[lane, reg] = True
        regs[lane, reg] = words[idx]
    if not seen.all():
        raise AssertionError("load layout leaves registers unset")
    return regs


def _halves(word):
    """uint32 -> (low fp16, high fp16) as float64 (bit view, little-endian pair)."""
    pair = np.array([word], dtype=np.uint32).view(np.float16)
    return float(pair[0]), float(pair[1])


def simulate_warp_matmul(A, B):
    """Run the example's data flow on the CPU and return Out (16, 8) float64.

    1. regroup A and B into 8x8 matrices of words and load them by A_LOAD/B_LOAD;
    2. read the same registers through A_MMA/B_MMA as A[i, k] and B[j, k];
    3. D[i, j] = C + sum_k A[i, k] * B[j, k] with C = 0;
    4. place D by D_MMA into dr[lane, r];
    5. scatter dr into Out with the page's formula.
    """
    ar = load_fragments(a_words(A), A_LOAD, 4)
    br = load_fragments(b_words(B), B_LOAD, 2)
    a = np.zeros((16, 16))
    b = np.zeros((8, 16))
    for i in range(16):
        for kw in range(8):
            lane, reg = evaluate(A_MMA, (0, 0, i // 8, i % 8, kw // 4, kw % 4))
            a[i, 2 * kw], a[i, 2 * kw + 1] = _halves(ar[lane, reg])
    for j in range(8):
        for kw in range(8):
            lane, reg = evaluate(B_MMA, (0, 0, j, kw // 4, kw % 4))
            b[j, 2 * kw], b[j, 2 * kw + 1] = _halves(br[lane, reg])
    d = np.zeros((16, 8))
    for i in range(16):
        for j in range(8):
            acc = 0.0                      # C = T.float32(0)
            for k in range(16):
                acc += a[i, k] * b[j, k]
            d[i, j] = acc
    dr = np.full((32, 4), np.nan)
    for i in range(16):
        for j in range(8):
            lane, reg = evaluate(D_MMA, (0, 0, i // 8, i % 8, j // 2, j % 2))
            dr[lane, reg] = d[i, j]
    out = np.full((16, 8), np.nan)
    for lane in range(32):
        for r in range(4):
            row, col = scatter_cell(lane, r)
            out[row, col] = dr[lane, r]
    return out


def scatter_cell(lane, r):
    """Output cell of dr[r] in ``lane``: row lane//4 + 8 (r//2), column 2 (lane%4) + r%2."""
    return lane // 4 + 8 * (r // 2), 2 * (lane % 4) + r % 2
