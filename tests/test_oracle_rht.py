"""Pins of the oracle's rotated (random-sign block Hadamard) linear layer.

Inputs are tiled with 32 x 32 blocks B = D H diag(v) H D / 1024 (H the Sylvester
Hadamard from scipy, D the sign matrix of the mask, v from the E2M1 grid).  Such a
block rotated along its rows is D H diag(v) / 32 and along its columns
diag(v) H D / 32: both are exactly representable MXFP4 blocks, so every quantizer of
the rotated layer (RNE or stochastic) is exact and the layer must reproduce the
textbook products Y = X W^T, dX = dY W, dW = dY^T X exactly.  A wrong axis, sign,
mask bit order or alpha breaks the equality."""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle as O

GRID = np.array([1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def signs(mask):
    return np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(32)])


def rotatable(rows, cols, mask, rng):
    H = hadamard(32).astype(np.float64)
    D = np.diag(signs(mask))
    out = np.zeros((rows, cols))
    for bi in range(rows // 32):
        for bj in range(cols // 32):
            v = rng.choice(GRID, 32) * rng.choice([-1.0, 1.0], 32)
            v[0] = 6.0
            v *= 2.0 ** int(rng.integers(-8, 8))
            out[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32] = D @ H @ np.diag(v) @ H @ D / 1024
    x = out.astype(np.float32)
    assert np.array_equal(x.astype(np.float64), out)  # exact in float32
    return x


@pytest.mark.parametrize("mask", [0x0, 0x8000_0001, 0x5A3C_96E1])
def test_rotated_layer_is_exact_on_doubly_rotatable_inputs(mask):
    rng = np.random.default_rng(mask & 0xFFFF)
    M, N, K = 64, 96, 128
    x = rotatable(M, K, mask, rng)
    w = rotatable(N, K, mask, rng)
    dy = rotatable(M, N, mask, rng)
    y, xq, wq = O.linear_fwd_rht(x, w, mask)
    assert np.array_equal(y, x.astype(np.float64) @ w.astype(np.float64).T)
    dx, dw, _ = O.linear_bwd_rht(dy, xq, wq, M, N, K, seed=3, sign_mask=mask)
    assert np.array_equal(dx, dy.astype(np.float64) @ w.astype(np.float64))
    assert np.array_equal(dw, dy.astype(np.float64).T @ x.astype(np.float64))


def test_rotated_double_quantization_undoes_the_forward_rotation():
    """requantize_rht of Q_D(H_K W) equals quantizing W itself along the other axis
    with the rotation (exact inputs), and differs from the plain requantize."""
    mask = 0x0F0F_3355
    rng = np.random.default_rng(5)
    N, K = 64, 96
    w = rotatable(N, K, mask, rng)
    wq = O.quantize(w, O.ROW, O.RNE, 0, True, mask)
    got = O.requantize_rht(wq[0], wq[1], N, K, O.SR, 11, mask)
    want = O.quantize(w, O.COL, O.SR, 11, True, mask)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    plain = O.requantize(wq[0], wq[1], N, K, O.SR, 11)
    assert not np.array_equal(plain[0], want[0])


def test_rotated_layer_is_close_to_the_plain_layer_on_gaussian_inputs():
    """On ordinary inputs both layers approximate the exact product; the rotation
    changes the rounding, not the result it approximates."""
    rng = np.random.default_rng(9)
    M, N, K = 64, 64, 256
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    y_rot, _, _ = O.linear_fwd_rht(x, w, 0x1234_5678)
    y_plain, _, _ = O.linear_fwd(x, w)
    scale = np.abs(exact).mean()
    assert np.abs(y_rot - exact).mean() < 0.2 * scale
    assert np.abs(y_plain - exact).mean() < 0.2 * scale
    assert not np.array_equal(y_rot, y_plain)
