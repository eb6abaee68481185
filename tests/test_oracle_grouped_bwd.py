"""Pins of the oracle's grouped (MoE) linear backward: one group is the dense
backward, and on exactly representable inputs every product is the textbook one
per expert, with ragged and empty token segments."""
import numpy as np

import oracle as O


def test_one_group_is_the_dense_backward():
    rng = np.random.default_rng(0)
    R, N, K = 96, 64, 128
    x = rng.standard_normal((R, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    dy = (rng.standard_normal((R, N)) * 1e-3).astype(np.float32)
    _, xq, wq = O.linear_fwd(x, w)
    gdx, gdw, _ = O.grouped_linear_bwd(dy, xq, wq, [0, R], N, K, seed=7)
    ddx, ddw, _ = O.linear_bwd(dy, xq, wq, R, N, K, seed=7)
    assert np.array_equal(gdx, ddx)
    assert np.array_equal(gdw[0], ddw)


def grid_values(rng, shape, e0):
    """Values in {0, +-1, +-2, +-3, +-4, +-6} * 2^e0: every 1x32 or 32x1 block of them
    is exactly representable, whatever its largest magnitude."""
    g = rng.choice(np.array([0.0, 1, 2, 3, 4, 6, -1, -2, -3, -4, -6]), shape)
    return (g * 2.0 ** e0).astype(np.float32)


def test_exact_inputs_give_textbook_products_per_expert():
    rng = np.random.default_rng(1)
    N, K = 64, 96
    offs = [0, 0, 37, 100, 100, 261]          # empty, ragged and 32-misaligned segments
    E, R = len(offs) - 1, offs[-1]
    x = grid_values(rng, (R, K), -3)
    w = grid_values(rng, (E * N, K), -6)
    dy = grid_values(rng, (R, N), -9)
    xq = O.quantize(x, O.ROW, O.RNE)
    wq = O.quantize(w, O.ROW, O.RNE)
    assert np.array_equal(O.dequantize(*xq, R, K), x)
    dx, dw, (q3, q4, q5, q6) = O.grouped_linear_bwd(dy, xq, wq, offs, N, K, seed=3)
    x64, w64, dy64 = (a.astype(np.float64) for a in (x, w, dy))
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        we = w64[e * N:(e + 1) * N]
        assert np.array_equal(dx[r0:r1], dy64[r0:r1] @ we), e
        assert np.array_equal(dw[e], dy64[r0:r1].T @ x64[r0:r1]), e
        P = (r1 - r0 + 31) // 32 * 32
        assert q5[e][0].shape == (N, P // 2) and q6[e][0].shape == (K, P // 2)
    assert not dw[0].any() and not dw[3].any()  # experts without tokens


def test_segment_padding_rounds_to_zero_codes():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 64)).astype(np.float32)
    (codes, scales), = O.quantize_segments(x, [0, 50], O.SR, 5)
    c = O.unpack_codes(codes)                    # [64, 64]: tokens 50..63 are padding
    assert codes.shape == (64, 32) and scales.shape == (64, 2)
    assert not (c[:, 50:] & 7).any()
    # the real part equals quantizing the first 50 tokens' blocks with global indices
    want_c, want_s = O.quantize_blocks(np.pad(x.T, ((0, 0), (0, 14))).reshape(64, 2, 32),
                                       (np.arange(64)[None, :] * 64 + np.arange(64)[:, None]
                                        ).reshape(64, 2, 32), O.SR, 5)
    assert np.array_equal(c, want_c.reshape(64, 64)) and np.array_equal(scales, want_s)
