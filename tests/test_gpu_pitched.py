"""GPU checks of the scale-pitch entry points (mx_quantize_ld, mx_gemm_ld,
mx_gemm_grouped_ld) against their packed counterparts, which the other GPU tests
hold to the oracle: the same codes, the same scale bytes at their pitch (padding
bytes untouched), and bit-identical products whatever the padding holds."""
import numpy as np
import pytest
import torch

from mxfp4_microscaling_quantization_amd import mx
from tests.gpu_util import DEV, host, to_dev_u8, upload
from tests.test_gpu_gemm import random_operand
from tests.test_gpu_quant import mixed_input

pytestmark = pytest.mark.gpu


def pad16(v):
    return (v + 15) // 16 * 16


def pitched(scales: np.ndarray, ld: int, fill=0xFF) -> torch.Tensor:
    """[rows][nb] scales copied into rows ld bytes apart, the padding set to fill."""
    rows, nb = scales.shape
    out = np.full((rows, ld), fill, np.uint8)
    out[:, :nb] = scales
    return to_dev_u8(out)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("axis", [mx.MX_ROW, mx.MX_COL])
@pytest.mark.parametrize("rnd,had", [(mx.MX_RNE, 0), (mx.MX_SR, 0), (mx.MX_SR, 1)])
def test_quantize_ld_equals_packed(dtype, axis, rnd, had):
    rows, cols = 160, 2880                     # 90 blocks per row: pitch 96
    x = upload(mixed_input(rows, cols, 61, dtype), dtype)
    dt = mx.dtype_code(x)
    outer, inner = (rows, cols) if axis == mx.MX_ROW else (cols, rows)
    nb, ld = inner // 32, pad16(inner // 32) + 16
    c0 = torch.empty((outer, inner // 2), dtype=torch.uint8, device=DEV)
    s0 = torch.empty((outer, nb), dtype=torch.uint8, device=DEV)
    mx.mx_quantize(x, dt, rows, cols, axis, rnd, 7, had, 0x1234567, c0, s0)
    c1 = torch.full_like(c0, 0x5A)
    s1 = torch.full((outer, ld), 0x5A, dtype=torch.uint8, device=DEV)
    mx.mx_quantize_ld(x, dt, rows, cols, axis, rnd, 7, had, 0x1234567, c1, s1, ld)
    assert torch.equal(c0, c1)
    assert torch.equal(s0, s1[:, :nb])
    assert bool((s1[:, nb:] == 0x5A).all()), "padding bytes written"


@pytest.mark.parametrize("M,N,K", [(333, 129, 2880),    # small tiles, 2-byte -> group loads
                                   (6144, 6144, 2880),  # 256 x 256 tiles, eight waves
                                   (500, 300, 4096)])   # already packed-aligned K
def test_gemm_ld_equals_packed(M, N, K):
    rng = np.random.default_rng(M + K)
    a = random_operand(rng, M, K)
    b = random_operand(rng, N, K)
    ldc = (N + 3) // 4 * 4
    c0 = torch.empty((M, ldc), dtype=torch.float32, device=DEV)
    mx.mx_gemm(to_dev_u8(a[0]), to_dev_u8(a[1]), to_dev_u8(b[0]), to_dev_u8(b[1]), M, N, K, 1.0,
               c0, ldc)
    lda, ldb = pad16(K // 32), pad16(K // 32) + 32
    c1 = torch.empty_like(c0)
    mx.mx_gemm_ld(to_dev_u8(a[0]), pitched(a[1], lda), lda, to_dev_u8(b[0]), pitched(b[1], ldb),
                  ldb, M, N, K, 1.0, c1, ldc)
    assert torch.equal(c0[:, :N], c1[:, :N])


def test_gemm_grouped_ld_equals_packed():
    rng = np.random.default_rng(71)
    offs = [0, 0, 300, 777, 777, 1500, 2100]   # empty and ragged groups
    E, N, K = len(offs) - 1, 384, 2880
    R = offs[-1]
    a = random_operand(rng, R, K)
    b = random_operand(rng, E * N, K)
    c0 = torch.empty((R, N), dtype=torch.float32, device=DEV)
    mx.mx_gemm_grouped(to_dev_u8(a[0]), to_dev_u8(a[1]), to_dev_u8(b[0]), to_dev_u8(b[1]), offs, E,
                       N, K, 1.0, c0)
    ld = pad16(K // 32)
    c1 = torch.empty_like(c0)
    mx.mx_gemm_grouped_ld(to_dev_u8(a[0]), pitched(a[1], ld), ld, to_dev_u8(b[0]),
                          pitched(b[1], ld), ld, offs, E, N, K, 1.0, c1)
    assert torch.equal(c0, c1)
