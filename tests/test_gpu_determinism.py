"""Results that must not depend on how the work is cut into launches, tiles or
windows, NaN scale blocks through the GEMM, and a de-oscillation window whose
state leaves the GPU half way and comes back."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_microscaling_quantization_amd import mx
from tests.gpu_util import DEV, assert_bytes_equal, assert_gemm_close, host, to_dev_f32, to_dev_u8

pytestmark = pytest.mark.gpu


def random_operand(rng, rows, K, lo=110, hi=140):
    codes = O.pack_codes(rng.integers(0, 16, (rows, K)).astype(np.uint8))
    scales = rng.integers(lo, hi, (rows, K // 32)).astype(np.uint8)
    return codes, scales


def gemm(a, b, M, N, K):
    c = torch.full((M, N), float("nan"), device=DEV)
    mx.mx_gemm(*a, *b, M, N, K, 1.0, c, N)
    return c


@pytest.mark.parametrize("K", [1024, 640])
def test_gemm_rows_do_not_depend_on_the_tile_path(K):
    """A 4096 x 8192 product takes 256 x 256 tiles (the ping-pong kernel, whose scale
    groups are shifted into place when K % 512 != 0); 256-row slices of it, launched
    alone, take 128 x 128 tiles.  Both sum every output over K in
    the same order (64-wide MFMA chunks in K order, no split), so the slices must
    equal the big product's rows bit for bit."""
    M, N = 4096, 8192
    rng = np.random.default_rng(K)
    a = tuple(to_dev_u8(t) for t in random_operand(rng, M, K))
    b = tuple(to_dev_u8(t) for t in random_operand(rng, N, K))
    print(f"determinism: gemm {M}x{N}x{K}", flush=True)
    big = gemm(a, b, M, N, K)
    for r0 in (0, 1792, M - 256):
        part = gemm((a[0][r0:r0 + 256], a[1][r0:r0 + 256]), b, 256, N, K)
        assert torch.equal(part.view(torch.int32), big[r0:r0 + 256].view(torch.int32)), r0


def test_row_quantizer_grid_stride_is_deterministic():
    """8192 x 20480 bf16 has 5.2 M row blocks, more windows than the row
    quantizer's grid (16,384 workgroups), so workgroups stride; each half alone
    fits the grid.  Nearest rounding does not depend on the element index, so the
    halves must reproduce the whole bit for bit; stochastic rounding is checked
    against the oracle on blocks of strided windows (block index >= 16384 * 256)."""
    rows, cols = 8192, 20480
    g = torch.Generator(device=DEV).manual_seed(5)
    x = torch.randn(rows, cols, device=DEV, dtype=torch.bfloat16, generator=g)
    print("determinism: row quantizer grid stride", flush=True)
    c, s = mx.quantize(x, mx.MX_ROW, mx.MX_RNE)
    for r0, r1 in ((0, rows // 2), (rows // 2, rows)):
        hc, hs = mx.quantize(x[r0:r1].contiguous(), mx.MX_ROW, mx.MX_RNE)
        assert torch.equal(hc, c[r0:r1]) and torch.equal(hs, s[r0:r1]), (r0, r1)
    seed = 0xDE7
    c, s = mx.quantize(x, mx.MX_ROW, mx.MX_SR, seed)
    rng = np.random.default_rng(3)
    nb = cols // 32
    blk = np.concatenate([rng.integers(16384 * 256, rows * nb, 1500), rng.integers(0, rows * nb, 500)])
    o, b = blk // nb, blk % nb
    ot, bt = torch.from_numpy(o).to(DEV), torch.from_numpy(b).to(DEV)
    ar = torch.arange(32, device=DEV)
    v = x[ot[:, None], bt[:, None] * 32 + ar[None, :]].float().cpu().numpy()
    idx = o[:, None] * cols + b[:, None] * 32 + np.arange(32)[None, :]
    wc, ws = O.quantize_blocks(v, idx, O.SR, seed)
    assert_bytes_equal(s[ot, bt].cpu().numpy(), ws, "SR scales of strided windows")
    got = c[ot[:, None], bt[:, None] * 16 + torch.arange(16, device=DEV)[None, :]].cpu().numpy()
    assert_bytes_equal(got, O.pack_codes(wc), "SR codes of strided windows")


def nan_operands(rng, M, N, K, a_rows, b_rows):
    """Random operands with scale byte 0xFF in one block of each listed row."""
    a = random_operand(rng, M, K)
    b = random_operand(rng, N, K)
    a[1][a_rows, rng.integers(0, K // 32, len(a_rows))] = 0xFF
    b[1][b_rows, rng.integers(0, K // 32, len(b_rows))] = 0xFF
    return a, b


def check_nan_rows(got, a, b, rows, N, K):
    want = O.gemm(a[0][rows], a[1][rows], *b, len(rows), N, K)
    nan = np.isnan(want)
    assert nan.any() and not nan.all()
    assert np.array_equal(np.isnan(got[rows]), nan), "NaN positions"
    ab = O.gemm_abs(a[0][rows], a[1][rows], *b, len(rows), N, K)
    fin = ~nan
    assert_gemm_close(got[rows][fin], want[fin], ab[fin], "finite outputs")


def test_gemm_nan_scale_blocks():
    """Scale byte 0xFF (the E8M0 NaN code, written by the quantizers for blocks
    holding NaN or Inf) makes the block's values NaN: every output whose
    contraction meets such a block is NaN, as in the oracle, and the others stay
    within the tolerance (128 x 128 tiles)."""
    rng = np.random.default_rng(31)
    M, N, K = 96, 80, 256
    a, b = nan_operands(rng, M, N, K, rng.integers(0, M, 5), rng.integers(0, N, 4))
    got = host(gemm(tuple(to_dev_u8(t) for t in a), tuple(to_dev_u8(t) for t in b), M, N, K))
    check_nan_rows(got, a, b, np.arange(M), N, K)


def test_gemm_nan_scale_blocks_large_tiles():
    """The same through the 256 x 256 ping-pong kernel (6144 x 6144 x 512), on 64
    sampled rows of which 16 carry a NaN scale block."""
    rng = np.random.default_rng(32)
    M, N, K = 6144, 6144, 512
    rows = np.sort(rng.choice(M, 64, replace=False))
    a, b = nan_operands(rng, M, N, K, rows[::4], rng.integers(0, N, 6))
    print(f"determinism: NaN scale blocks {M}x{N}x{K}", flush=True)
    got = host(gemm(tuple(to_dev_u8(t) for t in a), tuple(to_dev_u8(t) for t in b), M, N, K))
    check_nan_rows(got, a, b, rows, N, K)


def test_deosc_state_save_restore_on_the_gpu():
    """100 steps, the state (w, w_prev, d_w, d_q) copied to the host and into fresh
    device buffers, 100 more steps with the window ending at step 200: bit-identical
    to one uninterrupted 200-step window (the ALTO page's window length)."""
    rng = np.random.default_rng(9)
    w0 = (rng.standard_normal((64, 2880)) * 0.02).astype(np.float32)
    w0[1, 32:64] = 0.0
    rows, cols = w0.shape
    seed, steps, half = 4, 200, 100

    def window(split):
        w = to_dev_f32(w0)
        st = [torch.empty_like(w) for _ in range(3)]
        flags = torch.full((rows, cols), 7, dtype=torch.uint8, device=DEV)
        mx.mx_deosc_init(w, rows, cols, *st)
        for t in range(1, steps + 1):
            if split and t == half + 1:
                saved = [host(a).copy() for a in (w, *st)]
                w, *st = [to_dev_f32(a) for a in saved]
            mx.mx_synth_step(w, rows * cols, seed, t)
            mx.mx_deosc_step(w, rows, cols, *st, t == steps, 4.0, flags)
        return [host(w)] + [host(a) for a in st] + [host(flags)]

    print("determinism: de-oscillation save/restore", flush=True)
    straight, resumed = window(False), window(True)
    assert straight[-1].sum() > 0          # some weights were flagged and snapped
    for a, b, name in zip(straight, resumed, ["w", "w_prev", "d_w", "d_q", "flags"]):
        assert_bytes_equal(b.view(np.uint8), a.view(np.uint8), name)
