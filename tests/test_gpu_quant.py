"""GPU parity of the quantizer kernels against the oracle (bit-exact codes and scales)."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_microscaling_quantization_amd import mx, synth
from tests.gpu_util import (DEV, assert_bytes_equal, host, oracle_input, to_dev_u8, upload)

pytestmark = pytest.mark.gpu


def mixed_input(rows, cols, seed, dtype):
    """Student-t values over many binades, with outliers, exact zeros, negative
    zeros, an all-zero row block and tiny (subnormal) values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, (rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, (rows, 1))).astype(np.float32)
    k = max(1, rows * cols // 500)
    pos = rng.choice(rows * cols, k, replace=False)
    x.reshape(-1)[pos] *= 100.0
    x.reshape(-1)[rng.choice(rows * cols, k, replace=False)] = 0.0
    x.reshape(-1)[rng.choice(rows * cols, k, replace=False)] = -0.0
    x[: min(rows, 32), : min(cols, 32)] = 0.0
    if rows > 64 and cols > 64:
        x[32:64, 32:64] = (rng.standard_normal((32, 32)) * 1e-39).astype(np.float32)  # subnormal
        x[40, 40] = 3e38
    if dtype == "bf16":
        return synth.f32_to_bf16_bits(x)
    return x


SHAPES_ROW = [(1, 32), (37, 96), (300, 224)]
SHAPES_COL = [(32, 8), (96, 72), (544, 200)]   # ragged against the 256 x 64 column tile


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("axis", [mx.MX_ROW, mx.MX_COL])
@pytest.mark.parametrize("rnd", [mx.MX_RNE, mx.MX_SR])
@pytest.mark.parametrize("had", [0, 1])
def test_quantize_matches_oracle(dtype, axis, rnd, had):
    shapes = SHAPES_ROW if axis == mx.MX_ROW else SHAPES_COL
    for i, (rows, cols) in enumerate(shapes):
        x = mixed_input(rows, cols, 100 + i, dtype)
        seed, mask = 0xDEADBEEF12345 + i, 0x9E3779B9 ^ i
        codes, scales = mx.quantize(upload(x, dtype), axis, rnd, seed, had, mask)
        wc, ws = O.quantize(oracle_input(x, dtype), axis, rnd, seed, bool(had), mask)
        assert_bytes_equal(host(scales), ws, f"scales {rows}x{cols}")
        assert_bytes_equal(host(codes), wc, f"codes {rows}x{cols}")


@pytest.mark.parametrize("rnd", [mx.MX_RNE, mx.MX_SR])
@pytest.mark.parametrize("e", [-127, -20, 0, 37, 125])
def test_every_bf16_value_under_a_fixed_scale(rnd, e):
    """All 65,536 bf16 patterns that fit under one block scale, 31 per block next to an anchor."""
    vals = O.bf16_bits_to_f32(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16))
    anchor = np.float32(np.ldexp(1.5, -126)) if e == -127 else np.float32(np.ldexp(1.875, e + 2))
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= anchor)]
    n = (len(vals) + 30) // 31 * 31
    vals = np.concatenate([vals, np.zeros(n - len(vals), np.float32)]).reshape(-1, 31)
    blocks = np.concatenate([np.full((vals.shape[0], 1), anchor, np.float32), vals], axis=1)
    bits = synth.f32_to_bf16_bits(blocks)
    assert np.array_equal(O.bf16_bits_to_f32(bits), blocks)
    codes, scales = mx.quantize(upload(bits, "bf16"), mx.MX_ROW, rnd, 77)
    wc, ws = O.quantize(blocks, O.ROW, rnd, 77)
    assert_bytes_equal(host(scales), ws, "scales")
    assert_bytes_equal(host(codes), wc, "codes")


@pytest.mark.parametrize("axis", [mx.MX_ROW, mx.MX_COL])
def test_sr_decisions_one_step_either_side_of_the_carry(axis):
    """Each value sits one 2^-22 step below or exactly at the carry point of its
    own random bits, in every interval of the grid, under random block scales:
    the GPU codes are the expected neighbours, as the oracle's are."""
    from tests.sr_cases import carry_boundary_case
    seed = 0xC0FFEE
    x, codes, scales = carry_boundary_case(160, 224, axis, seed, np.random.default_rng(8))
    c, s = mx.quantize(upload(x, "f32"), axis, mx.MX_SR, seed)
    assert_bytes_equal(host(s), scales, "scales")
    assert_bytes_equal(host(c), O.pack_codes(codes), "codes")


def test_random_f32_bit_patterns():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 0x7F800000, (256, 256), dtype=np.uint32)
    u |= rng.integers(0, 2, (256, 256), dtype=np.uint32) << 31
    x = u.view(np.float32)
    for rnd in (mx.MX_RNE, mx.MX_SR):
        for axis in (mx.MX_ROW, mx.MX_COL):
            codes, scales = mx.quantize(upload(x, "f32"), axis, rnd, 5)
            wc, ws = O.quantize(x, axis, rnd, 5)
            assert_bytes_equal(host(scales), ws, "scales")
            assert_bytes_equal(host(codes), wc, "codes")


def test_nonfinite_blocks_get_nan_scale_and_zero_codes():
    x = np.ones((64, 64), np.float32)
    x[0, 3] = np.nan
    x[1, 40] = np.inf
    x[33, 0] = -np.inf
    for axis in (mx.MX_ROW, mx.MX_COL):
        codes, scales = mx.quantize(upload(x, "f32"), axis, mx.MX_RNE)
        wc, ws = O.quantize(x, axis, O.RNE)
        assert_bytes_equal(host(scales), ws, "scales")
        assert_bytes_equal(host(codes), wc, "codes")
        assert (host(scales) == 255).sum() == 3


@pytest.mark.parametrize("rows,cols", [(32, 32), (288, 96), (544, 160)])
@pytest.mark.parametrize("rnd", [mx.MX_RNE, mx.MX_SR])
def test_requantize_matches_oracle(rows, cols, rnd):
    x = mixed_input(rows, cols, 7, "f32")
    c, s = O.quantize(x, O.ROW, O.RNE)
    co, so = mx.requantize(to_dev_u8(c), to_dev_u8(s), rows, cols, rnd, 991)
    wc, ws = O.requantize(c, s, rows, cols, rnd, 991)
    assert_bytes_equal(host(so), ws, "scales")
    assert_bytes_equal(host(co), wc, "codes")


def test_requantize_of_extreme_scales():
    # scale bytes 0 and 1 give values down to 2^-128 (float32 subnormals)
    rng = np.random.default_rng(8)
    rows, cols = 64, 64
    codes = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    c = O.pack_codes(codes)
    s = rng.choice(np.array([0, 1, 2, 250, 252], np.uint8), (rows, cols // 32))
    co, so = mx.requantize(to_dev_u8(c), to_dev_u8(s), rows, cols, mx.MX_SR, 3)
    wc, ws = O.requantize(c, s, rows, cols, O.SR, 3)
    assert_bytes_equal(host(so), ws, "scales")
    assert_bytes_equal(host(co), wc, "codes")


@pytest.mark.parametrize("rnd", [mx.MX_RNE, mx.MX_SR])
def test_requantize_of_nan_and_overflowing_scales(rnd):
    """Input scale bytes at the top of the E8M0 range: 0xFF decodes every value of
    its row block to NaN (the column blocks through that row take the NaN scale and
    zero codes, reading R4), and bytes 253 / 254 put the larger magnitudes past the
    float32 range (decoded as +-Inf: non-finite column blocks as well), beside
    ordinary bytes; rows past the first 32 keep finite scales."""
    rng = np.random.default_rng(21)
    rows, cols = 96, 128
    codes = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    c = O.pack_codes(codes)
    s = rng.choice(np.array([0, 1, 100, 127, 200, 252], np.uint8), (rows, cols // 32))
    s[3, 0] = 255
    s[40, 2] = 254
    s[41, 2] = 253
    s[70, 1] = 255
    co, so = mx.requantize(to_dev_u8(c), to_dev_u8(s), rows, cols, rnd, 17)
    with np.errstate(over="ignore", invalid="ignore"):
        wc, ws = O.requantize(c, s, rows, cols, rnd, 17)
    assert (ws == 255).any() and (ws < 255).any()
    assert_bytes_equal(host(so), ws, "scales")
    assert_bytes_equal(host(co), wc, "codes")


@pytest.mark.parametrize("rows,cols", [(64, 96), (288, 160)])
def test_quantize_dual_equals_two_quantizations(rows, cols):
    for dtype in ("f32", "bf16"):
        x = mixed_input(rows, cols, 9, dtype)
        d = upload(x, dtype)
        cr = torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV)
        sr = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
        cc = torch.empty((cols, rows // 2), dtype=torch.uint8, device=DEV)
        sc = torch.empty((cols, rows // 32), dtype=torch.uint8, device=DEV)
        mx.mx_quantize_dual(d, mx.dtype_code(d), rows, cols, mx.MX_SR, 13, 15, cr, sr, cc, sc)
        xin = oracle_input(x, dtype)
        w1 = O.quantize(xin, O.ROW, O.SR, 13)
        w2 = O.quantize(xin, O.COL, O.SR, 15)
        assert_bytes_equal(host(cr), w1[0], "row codes")
        assert_bytes_equal(host(sr), w1[1], "row scales")
        assert_bytes_equal(host(cc), w2[0], "col codes")
        assert_bytes_equal(host(sc), w2[1], "col scales")


@pytest.mark.parametrize("axis", [mx.MX_ROW, mx.MX_COL])
@pytest.mark.parametrize("had", [0, 1])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_dequantize_matches_oracle(axis, had, out):
    rows, cols = 96, 160
    rng = np.random.default_rng(12)
    outer, inner = (rows, cols) if axis == mx.MX_ROW else (cols, rows)
    codes = O.pack_codes(rng.integers(0, 16, (outer, inner)).astype(np.uint8))
    scales = rng.integers(100, 150, (outer, inner // 32)).astype(np.uint8)
    scales[0, 0] = 0
    mask = 0x0F0F1234
    got = host(mx.dequantize(to_dev_u8(codes), to_dev_u8(scales), rows, cols, axis, had, mask, out))
    want = O.dequantize(codes, scales, rows, cols, axis, bool(had), mask).astype(np.float32)
    if out == torch.bfloat16:
        want = synth.f32_to_bf16_bits(want)
    assert_bytes_equal(got.view(np.uint32) if out == torch.float32 else got,
                       want.view(np.uint32) if out == torch.float32 else want, "values")


def test_quantize_sweep_size_sampled_blocks():
    """8192 x 8192 bf16 Student-t(3) with 0.1% outliers x100: every variant of the
    sweep, checked on 4096 random blocks per variant."""
    cfg = synth.sweep_config()
    x = cfg["x"]
    rows, cols, mask = cfg["rows"], cfg["cols"], cfg["sign_mask"]
    d = upload(x, "bf16")
    rng = np.random.default_rng(0)
    xf = O.bf16_bits_to_f32(x)
    for axis in (mx.MX_ROW, mx.MX_COL):
        for rnd in (mx.MX_RNE, mx.MX_SR):
            for had in (0, 1):
                print(f"sweep axis={axis} round={rnd} had={had}", flush=True)
                codes, scales = mx.quantize(d, axis, rnd, 2, had, mask)
                hc, hs = host(codes), host(scales)
                outer, nb = hs.shape
                o = rng.integers(0, outer, 4096)
                b = rng.integers(0, nb, 4096)
                if axis == mx.MX_ROW:
                    v = np.stack([xf[oi, bi * 32:(bi + 1) * 32] for oi, bi in zip(o, b)])
                    idx = np.stack([oi * cols + bi * 32 + np.arange(32) for oi, bi in zip(o, b)])
                else:
                    v = np.stack([xf[bi * 32:(bi + 1) * 32, oi] for oi, bi in zip(o, b)])
                    idx = np.stack([(bi * 32 + np.arange(32)) * cols + oi for oi, bi in zip(o, b)])
                wc, ws = O.quantize_blocks(v, idx, rnd, 2, bool(had), mask)
                assert_bytes_equal(hs[o, b], ws, "sampled scales")
                got = np.stack([hc[oi, bi * 16:(bi + 1) * 16] for oi, bi in zip(o, b)])
                assert_bytes_equal(got, O.pack_codes(wc), "sampled codes")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rnd,had", [(mx.MX_RNE, 0), (mx.MX_SR, 0), (mx.MX_RNE, 1), (mx.MX_SR, 1)])
@pytest.mark.parametrize("rows0,rows1", [(37, 300), (0, 96), (64, 0), (1, 1)])
def test_quantize_pair_equals_two_quantizations(dtype, rnd, had, rows0, rows1):
    cols, mask = 224, 0x1357_9BDF
    x0 = mixed_input(max(rows0, 1), cols, 51, dtype)[:rows0]
    x1 = mixed_input(max(rows1, 1), cols, 52, dtype)[:rows1]
    d0, d1 = upload(x0, dtype), upload(x1, dtype)
    u8 = lambda *sh: torch.full(sh, 0x55, dtype=torch.uint8, device=DEV)
    c0, s0, c1, s1 = u8(rows0, cols // 2), u8(rows0, cols // 32), u8(rows1, cols // 2), u8(rows1, cols // 32)
    mx.mx_quantize_pair(d0, rows0, d1, rows1, cols, mx.dtype_code(d0), rnd, 11, 12, had, mask,
                        c0, s0, c1, s1)
    for d, rows, c, s, seed in ((d0, rows0, c0, s0, 11), (d1, rows1, c1, s1, 12)):
        if rows == 0:
            continue
        wc, ws = mx.quantize(d, mx.MX_ROW, rnd, seed, had, mask)
        assert torch.equal(c, wc) and torch.equal(s, ws), (rows, seed)


@pytest.mark.parametrize("rows0,rows1,cols", [(96, 544, 160), (0, 64, 96), (288, 0, 64), (32, 32, 32)])
@pytest.mark.parametrize("rnd", [mx.MX_RNE, mx.MX_SR])
def test_requantize_pair_equals_two_requantizations(rows0, rows1, cols, rnd):
    def packed(rows, seed):
        x = mixed_input(max(rows, 32), cols, seed, "f32")[:rows]
        return O.quantize(x, O.ROW, O.RNE) if rows else (np.zeros((0, cols // 2), np.uint8),
                                                         np.zeros((0, cols // 32), np.uint8))
    a, b = packed(rows0, 61), packed(rows1, 62)
    u8 = lambda *sh: torch.full(sh, 0x55, dtype=torch.uint8, device=DEV)
    outs = (u8(cols, rows0 // 2), u8(cols, rows0 // 32), u8(cols, rows1 // 2), u8(cols, rows1 // 32))
    ins = [to_dev_u8(z) for z in (*a, *b)]
    mx.mx_requantize_pair(ins[0], ins[1], rows0, ins[2], ins[3], rows1, cols, rnd, 21, 22, *outs)
    for (ci, si), rows, c, s, seed in (((ins[0], ins[1]), rows0, outs[0], outs[1], 21),
                                       ((ins[2], ins[3]), rows1, outs[2], outs[3], 22)):
        if rows == 0:
            continue
        wc, ws = u8(cols, rows // 2), u8(cols, rows // 32)
        mx.mx_requantize(ci, si, rows, cols, rnd, seed, wc, ws)
        assert torch.equal(c, wc) and torch.equal(s, ws), (rows, seed)


def test_quantize_is_deterministic():
    x = mixed_input(544, 200, 4, "bf16")
    d = upload(x, "bf16")
    a = [host(t) for t in mx.quantize(d, mx.MX_COL, mx.MX_SR, 1)]
    b = [host(t) for t in mx.quantize(d, mx.MX_COL, mx.MX_SR, 1)]
    assert all(np.array_equal(p, q) for p, q in zip(a, b))
