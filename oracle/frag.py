"""Bit-exact model of the m8n8 matrix load/store (test infrastructure only).

Follows "copy -> ldstmatrix" (the ldstmatrix lowering page): sections
"Demonstration program" (the register layout and the row-major shared
layout), "Algorithm" steps 1-4 (regroup to [8 rows, 4 column pairs, num tiles,
2 b16 elements]; the register side must be the m8n8 fragment; the shared side
decides transpose and tile stride), and "How inputs change the algorithm"
(num in {1, 2, 4}; the store direction mirrors the load).  Also "Warp Matrix
Instructions", "From Shared Memory to a Matrix Product": the uint32 views pack
two fp16 elements per word and keep their bits.

Objects
  tile t of a group, element (r, c), r, c in [0, 8): a 16-bit pattern.
  group image: the shared-memory side, 64 * num b16 values per group.
    row-major    offset(r, c, t) = r * 8 * num + 8 * t + c
                 (the demo's shared layout, strides (8 num, 2, 8, 1) over
                 (row, column pair, tile, element))
    column-major offset(r, c, t) = (8 * t + c) * 8 + r
                 (strides (1, 2 p, 8 p, p) with p = 8: row stride 1, column
                 stride p, the 8-multiple required by step 3; tiles are stacked
                 along the columns.  The page fixes s8 = 1 and s4 = 2 s2 but not
                 the tile stride; 8 p = 64 elements, tiles packed back to back,
                 is the plain reading.)
  fragment: the register side, for each of the 32 lanes of a warp ``num``
    uint32 words.  The register layout (8, 4, num, 2) : (4@lane, 1@lane, 2, 1)
    puts element (r, 2 cp + e) of tile t into lane 4 r + cp, b16 slot 2 t + e.
    Word t of a lane is slots (2 t, 2 t + 1), the even column in the low 16
    bits.  Serialised lane-major: word index (g * 32 + lane) * num + t.

Only uint16/uint32 gathers and scatters; no value is ever converted, so NaN
payloads, infinities, subnormals and -0 pass through unchanged.
"""

import numpy as np

__all__ = [
    "register_layout", "shared_layout", "fit_shared_layout", "image_index",
    "frag_load", "frag_store", "frag_roundtrip",
]

LANES = 32        # a warp: the fragment is defined over 32 lanes
ROWS = 8          # rows of an m8n8 tile
PAIRS = 4         # column pairs per row
NUMS = (1, 2, 4)  # matrix counts the instruction accepts


def register_layout(num):
    """(shape, strides) of the register side; strides are (kind, value).

    kind "lane" = the stride is on the lane index, "reg" = on the b16 slot.
    Written as the demo gives it: S[(8, 4, num, 2) : (4@lane, 1@lane, 2, 1)].
    """
    _check_num(num)
    return (ROWS, PAIRS, num, 2), (("lane", 4), ("lane", 1), ("reg", 2), ("reg", 1))


def shared_layout(num, col_major):
    """(shape, strides) of the shared side over (row, column pair, tile, element)."""
    _check_num(num)
    if not col_major:
        return (ROWS, PAIRS, num, 2), (8 * num, 2, 8, 1)
    p = 8
    return (ROWS, PAIRS, num, 2), (1, 2 * p, 8 * p, p)


def fit_shared_layout(strides):
    """Step 3 of the lowering: which form fits a shared layout.

    strides = (s8, s4, s_num, s2).  Row-major fits when (s4, s2) == (2, 1) and
    s8 is a positive multiple of 8: plain form, per-lane row stride p = s8.
    Column-major fits when s8 == 1, s2 is a positive multiple of 8 and
    s4 == 2 * s2: transposing form, p = s2.  Returns (trans, p) or None.
    """
    s8, s4, _s_num, s2 = strides
    if (s4, s2) == (2, 1) and s8 > 0 and s8 % 8 == 0:
        return False, s8
    if s8 == 1 and s2 > 0 and s2 % 8 == 0 and s4 == 2 * s2:
        return True, s2
    return None


def image_index(num, col_major, r, c, t):
    """Offset (in b16 units, inside one group image) of element (r, c) of tile t."""
    _, st = shared_layout(num, col_major)
    cp, e = divmod(c, 2)
    return r * st[0] + cp * st[1] + t * st[2] + e * st[3]


def _slot_table(num, col_major):
    """table[lane, slot] = image offset feeding that register slot.

    Evaluates both layouts over every coordinate (r, cp, t, e): the register
    layout names the destination (lane, slot), the shared layout the source.
    """
    shape, rst = register_layout(num)
    _, sst = shared_layout(num, col_major)
    table = np.full((LANES, 2 * num), -1, dtype=np.int64)
    for r in range(shape[0]):
        for cp in range(shape[1]):
            for t in range(shape[2]):
                for e in range(shape[3]):
                    coord = (r, cp, t, e)
                    lane = sum(x * s for x, (kind, s) in zip(coord, rst) if kind == "lane")
                    slot = sum(x * s for x, (kind, s) in zip(coord, rst) if kind == "reg")
                    off = sum(x * s for x, s in zip(coord, sst))
                    if table[lane, slot] != -1:
                        raise AssertionError("register layout is not injective")
                    table[lane, slot] = off
    if (table < 0).any():
        raise AssertionError("register layout does not cover every slot")
    return table


def _check_num(num):
    if num not in NUMS:
        raise ValueError(f"num={num}: a matrix load moves 1, 2 or 4 tiles")


def _groups(n_items, per_group, what):
    if n_items % per_group:
        raise ValueError(f"{what}: {n_items} elements is not a whole number of groups of {per_group}")
    return n_items // per_group


def frag_load(image, num, col_major):
    """Shared image -> fragment (the ldmatrix direction).

    image: flat uint16 array of G * 64 * num values (G groups back to back).
    Returns a flat uint32 array of G * 32 * num words, lane-major per group:
    word (g * 32 + lane) * num + t = slot(2t) | slot(2t + 1) << 16.
    """
    img = np.ascontiguousarray(image).view(np.uint16).reshape(-1)
    G = _groups(img.size, 64 * num, "image")
    table = _slot_table(num, col_major)
    slots = img.reshape(G, 64 * num)[:, table]          # (G, 32, 2 num) uint16
    lo = slots[:, :, 0::2].astype(np.uint32)
    hi = slots[:, :, 1::2].astype(np.uint32)
    return (lo | (hi << np.uint32(16))).reshape(-1)


def frag_store(frag, num, col_major):
    """Fragment -> shared image (the stmatrix direction): the exact inverse of frag_load."""
    words = np.ascontiguousarray(frag).view(np.uint32).reshape(-1)
    G = _groups(words.size, 32 * num, "fragment")
    w = words.reshape(G, LANES, num)
    slots = np.empty((G, LANES, 2 * num), dtype=np.uint16)
    slots[:, :, 0::2] = (w & np.uint32(0xFFFF)).astype(np.uint16)
    slots[:, :, 1::2] = (w >> np.uint32(16)).astype(np.uint16)
    table = _slot_table(num, col_major)
    img = np.empty((G, 64 * num), dtype=np.uint16)
    img[:, table] = slots
    return img.reshape(-1)


def frag_roundtrip(image, num, col_major):
    """Load then store through the fragment, both with the same shared layout."""
    return frag_store(frag_load(image, num, col_major), num, col_major)
