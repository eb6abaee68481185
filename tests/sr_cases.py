"""Inputs that put every stochastic rounding decision one step from its carry.

For each element with 22 random bits r (the oracle's sr_bits22 for its logical
index), the value is lo + (hi - lo) * t / 2^22 with t = 2^22 - r - 1 (the sum
t + r stays below 2^22: round down) or t = 2^22 - r (it reaches 2^22: round
up), over every interval [lo, hi) of the E2M1 grid, random signs and block
scales 2^s.  Element 0 of each block is the anchor 6 * 2^s, so the block scale
is exactly 2^s.  Every value is exact in float32 (at most 23 fraction bits
above the interval's binade)."""
import numpy as np

import oracle as O


def carry_boundary_case(rows, cols, axis, seed, rng):
    """Returns (x [rows, cols] float32, expected codes [outer, inner] before
    packing, expected scale bytes [outer, inner / 32])."""
    idx = O.block_indices(rows, cols, axis)          # [outer, nblk, 32]
    r = O.sr_bits22(seed, idx)
    grid = O.E2M1_MAGNITUDES
    lo = rng.integers(0, 7, r.shape)
    up = rng.integers(0, 2, r.shape)
    up[r == 0] = 0                                   # t = 2^22 is out of range
    t = (1 << 22) - r - 1 + up
    a = grid[lo] + (grid[lo + 1] - grid[lo]) * t / float(1 << 22)
    a[..., 0] = 6.0
    mag = np.where(np.arange(32) == 0, 7, lo + up)
    s = rng.integers(-100, 100, r.shape[:-1])
    neg = rng.integers(0, 2, r.shape)
    v = np.where(neg == 1, -a, a) * np.exp2(s)[..., None]
    v32 = v.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), v), "boundary values must be exact"
    m = v32.reshape(idx.shape[0], -1)
    x = m if axis == O.ROW else np.ascontiguousarray(m.T)
    codes = ((neg << 3) | mag).astype(np.uint8).reshape(idx.shape[0], -1)
    scales = (s + 127).astype(np.uint8)
    return x, codes, scales
