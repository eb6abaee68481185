"""Tensors past 2^31 elements: 64-bit indexing in the quantizers and the GEMM.

X is a [65600, 32768] bf16 tensor (2^31 + 2,097,152 elements, 4.3 GB) drawn on the
device; the row, column and fused dual stochastic quantizers and the double
quantization are checked on sampled 32-element blocks, always including blocks
whose element indices lie past 2^31 (where a 32-bit index would wrap, the
stochastic rounding bits and the output offsets would both go wrong).  A GEMM
with a [65536, 32800] fp32 output (also past 2^31 elements) is checked on its
first and last rows."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_microscaling_quantization_amd import mx
from tests.gpu_util import DEV, assert_bytes_equal, assert_gemm_close, host

pytestmark = pytest.mark.gpu

ROWS, COLS = 65600, 32768
SEED = 0x1234_5678_9ABC


@pytest.fixture(scope="module")
def big_x():
    g = torch.Generator(device=DEV).manual_seed(11)
    x = torch.randn(ROWS, COLS, device=DEV, dtype=torch.bfloat16, generator=g)
    assert x.numel() > 2**31
    yield x
    del x
    torch.cuda.empty_cache()


def sample_blocks(axis, n, rng):
    """(outer, block) pairs: random ones plus the last blocks of the tensor."""
    outer, nb = (ROWS, COLS // 32) if axis == mx.MX_ROW else (COLS, ROWS // 32)
    o = np.concatenate([rng.integers(0, outer, n), [outer - 1, outer - 1, outer - 2]])
    b = np.concatenate([rng.integers(0, nb, n), [nb - 1, nb - 2, nb - 1]])
    if axis == mx.MX_ROW:   # force some row blocks past element 2^31
        o[:8] = ROWS - 1 - np.arange(8)
    else:                   # column blocks in the last row blocks
        b[:8] = nb - 1 - np.arange(8) % 2
    return o, b


def block_values(x, axis, o, b):
    """float32 values and logical indices of the sampled blocks."""
    ar = torch.arange(32, device=DEV)
    ot = torch.from_numpy(o).to(DEV)
    bt = torch.from_numpy(b).to(DEV)
    if axis == mx.MX_ROW:
        r = ot[:, None].expand(-1, 32)
        c = bt[:, None] * 32 + ar[None, :]
    else:
        r = bt[:, None] * 32 + ar[None, :]
        c = ot[:, None].expand(-1, 32)
    v = x[r, c].float().cpu().numpy()
    idx = (r.to(torch.int64) * COLS + c).cpu().numpy()
    assert idx.max() >= 2**31
    return v, idx


def check_sampled(codes, scales, x, axis, rnd, seed, rng, n=2048):
    o, b = sample_blocks(axis, n, rng)
    v, idx = block_values(x, axis, o, b)
    wc, ws = O.quantize_blocks(v, idx, rnd, seed)
    ot, bt = torch.from_numpy(o).to(DEV), torch.from_numpy(b).to(DEV)
    got_s = scales[ot, bt].cpu().numpy()
    got_c = codes[ot[:, None], bt[:, None] * 16 + torch.arange(16, device=DEV)[None, :]].cpu().numpy()
    assert_bytes_equal(got_s, ws, f"sampled scales axis {axis}")
    assert_bytes_equal(got_c, O.pack_codes(wc), f"sampled codes axis {axis}")


@pytest.mark.parametrize("axis", [mx.MX_ROW, mx.MX_COL])
def test_quantize_past_2_31_elements(big_x, axis):
    print(f"large quantize axis={axis}", flush=True)
    codes, scales = mx.quantize(big_x, axis, mx.MX_SR, SEED)
    check_sampled(codes, scales, big_x, axis, O.SR, SEED, np.random.default_rng(axis))


def test_dual_and_double_quantization_past_2_31_elements(big_x):
    print("large dual + requantize", flush=True)
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=DEV)
    cr, sr, cc, sc = u8(ROWS, COLS // 2), u8(ROWS, COLS // 32), u8(COLS, ROWS // 2), u8(COLS, ROWS // 32)
    mx.mx_quantize_dual(big_x, mx.MX_BF16, ROWS, COLS, mx.MX_SR, SEED, SEED + 1, cr, sr, cc, sc)
    rng = np.random.default_rng(5)
    check_sampled(cr, sr, big_x, mx.MX_ROW, O.SR, SEED, rng)
    check_sampled(cc, sc, big_x, mx.MX_COL, O.SR, SEED + 1, rng)
    del cc, sc
    # double quantization of the row-quantized tensor: 32x1 SR over its exact values
    rq_c, rq_s = u8(COLS, ROWS // 2), u8(COLS, ROWS // 32)
    mx.mx_requantize(cr, sr, ROWS, COLS, mx.MX_SR, SEED + 2, rq_c, rq_s)
    o, b = sample_blocks(mx.MX_COL, 1024, rng)              # column o, row block b
    rows = b[:, None] * 32 + np.arange(32)[None, :]          # [n, 32] input rows
    rt = torch.from_numpy(rows).to(DEV)
    code_bytes = cr[rt, torch.from_numpy(o // 2).to(DEV)[:, None]].cpu().numpy().astype(np.int64)
    nib = np.where((o % 2)[:, None] == 1, code_bytes >> 4, code_bytes & 15)
    sbytes = sr[rt, torch.from_numpy(o // 32).to(DEV)[:, None]].cpu().numpy().astype(np.int64)
    # exact values of the row-quantized tensor at the sampled positions (finite scales)
    assert (sbytes < 255).all()
    vals = np.ldexp(O.E2M1_MAGNITUDES[nib & 7] * np.where(nib & 8, -1.0, 1.0), sbytes - 127)
    vals = vals.astype(np.float32)
    idx = rows.astype(np.int64) * COLS + o[:, None]
    wc, ws = O.quantize_blocks(vals, idx, O.SR, SEED + 2)
    ot, bt = torch.from_numpy(o).to(DEV), torch.from_numpy(b).to(DEV)
    assert_bytes_equal(rq_s[ot, bt].cpu().numpy(), ws, "requantized scales")
    got = rq_c[ot[:, None], bt[:, None] * 16 + torch.arange(16, device=DEV)[None, :]].cpu().numpy()
    assert_bytes_equal(got, O.pack_codes(wc), "requantized codes")


def test_gemm_output_past_2_31_elements():
    M, N, K = 65536, 32800, 128
    assert M * N > 2**31
    print("large gemm", flush=True)
    rng = np.random.default_rng(6)
    a = rng.standard_normal((M, K)).astype(np.float32)
    bm = rng.standard_normal((N, K)).astype(np.float32)
    aq = O.quantize(a, O.ROW, O.RNE)
    bq = O.quantize(bm, O.ROW, O.RNE)
    to = lambda z: torch.from_numpy(np.ascontiguousarray(z)).to(DEV)
    c = torch.empty((M, N), dtype=torch.float32, device=DEV)
    mx.mx_gemm(to(aq[0]), to(aq[1]), to(bq[0]), to(bq[1]), M, N, K, 1.0, c, N)
    for rws in (np.arange(4), np.arange(M - 4, M)):
        ra = (aq[0][rws], aq[1][rws])
        want = O.gemm(*ra, *bq, len(rws), N, K)
        ab = O.gemm_abs(*ra, *bq, len(rws), N, K)
        assert_gemm_close(c[torch.from_numpy(rws).to(DEV)].cpu().numpy(), want, ab, f"rows {rws[0]}..")
    del c
    torch.cuda.empty_cache()
