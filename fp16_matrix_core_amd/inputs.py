"""Seeded synthetic inputs for the shapes the pages work through.

These generators are the only code that the device path and the CPU oracle
both consume.  They hold none of the product's or the copy's arithmetic: they
draw numbers, round them to fp16 (or draw raw 16-bit patterns), and return
numpy arrays.

Recipe: numpy ``default_rng(seed)`` (PCG64); uniform draws on [-1, 1] and
normal draws scaled by 0.1 are made in float64 and rounded to float16
(round-to-nearest-even); raw bit patterns are uniform over [0, 65536), so NaN,
infinity, subnormal and -0 patterns occur at their natural rates.  bfloat16
inputs are the same float64 draws rounded to float32 and then to the upper 16
bits of the float32 pattern, nearest-even; they are returned as uint16 bit
patterns (numpy has no bfloat16 type).
"""

import numpy as np

__all__ = [
    "uniform_f16", "normal_f16", "random_bits_u16", "identity_f16", "permutation_f16",
    "single_tile", "single_workgroup", "frag_bits", "large_square", "batched_small", "skinny",
    "FRAG_TILES", "to_bf16_bits", "uniform_bf16", "normal_bf16", "large_square_bf16", "accumulator_f32",
]

FRAG_TILES = 1 << 20   # 8x8 tiles in the fragment-copy workload


def uniform_f16(shape, rng):
    return rng.uniform(-1.0, 1.0, size=shape).astype(np.float16)


def normal_f16(shape, rng, scale=0.1):
    return (rng.standard_normal(size=shape) * scale).astype(np.float16)


def to_bf16_bits(x):
    """float64/float32 values -> bfloat16 bit patterns (uint16), via float32, nearest-even (finite inputs)."""
    bits = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def uniform_bf16(shape, rng):
    return to_bf16_bits(rng.uniform(-1.0, 1.0, size=shape))


def normal_bf16(shape, rng, scale=0.1):
    return to_bf16_bits(rng.standard_normal(size=shape) * scale)


def random_bits_u16(n, rng):
    return rng.integers(0, 1 << 16, size=n, dtype=np.uint16)


def identity_f16(n):
    return np.eye(n, dtype=np.float16)


def permutation_f16(perm):
    """Matrix P with P[j, perm[j]] = 1, so that (A @ P.T)[i, j] = A[i, perm[j]]."""
    perm = np.asarray(perm)
    n = perm.size
    p = np.zeros((n, n), dtype=np.float16)
    p[np.arange(n), perm] = 1.0
    return p


def single_tile(seed=0):
    """A (16,16), B (8,16), uniform [-1, 1], one generator (A drawn first)."""
    rng = np.random.default_rng(seed)
    return uniform_f16((16, 16), rng), uniform_f16((8, 16), rng)


def single_workgroup(seed=1, perm_seed=2):
    """A (128,64), B (64,64) uniform; plus identity-B and a permutation-B of 64."""
    rng = np.random.default_rng(seed)
    A = uniform_f16((128, 64), rng)
    B = uniform_f16((64, 64), rng)
    perm = np.random.default_rng(perm_seed).permutation(64)
    return A, B, identity_f16(64), permutation_f16(perm), perm


def frag_bits(n_tiles=FRAG_TILES, seed=3):
    """n_tiles * 64 random 16-bit patterns (n_tiles 8x8 tiles)."""
    return random_bits_u16(n_tiles * 64, np.random.default_rng(seed))


def large_square(n=8192, seed=4):
    """A (n,n), B (n,n), normal(0,1) * 0.1 rounded to fp16."""
    rng = np.random.default_rng(seed)
    return normal_f16((n, n), rng), normal_f16((n, n), rng)


def batched_small(batch=4096, seed=5):
    """batch independent problems A (128,64), B (64,64), uniform [-1, 1]."""
    rng = np.random.default_rng(seed)
    return uniform_f16((batch, 128, 64), rng), uniform_f16((batch, 64, 64), rng)


def skinny(m=16384, n=8, k=16384, seed=5):
    """A (m,k), B (n,k), uniform [-1, 1]."""
    rng = np.random.default_rng(seed)
    return uniform_f16((m, k), rng), uniform_f16((n, k), rng)


def large_square_bf16(n=8192, seed=6):
    """The large product with bfloat16 operands: A, B (n, n) ~ N(0,1)*0.1 as bfloat16 bit patterns."""
    rng = np.random.default_rng(seed)
    return normal_bf16((n, n), rng), normal_bf16((n, n), rng)


def accumulator_f32(shape, seed=7):
    """Previous output contents for accumulating products: float32 ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal(size=shape).astype(np.float32)
