"""CPU-only checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

from mxfp4_microscaling_quantization_amd import mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PRODUCT_HEADER = os.path.join(ROOT, "include", "mx.h")
SYNTH_HEADER = os.path.join(ROOT, "include", "mx_synth.h")


def declared_functions(header):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text))


@pytest.fixture(scope="module")
def L():
    return mx.lib()


def test_every_declared_symbol_is_exported_and_bound(L):
    names = declared_functions(PRODUCT_HEADER)
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert names == set(mx.SIGNATURES), names ^ set(mx.SIGNATURES)


def test_workload_generator_lives_outside_the_product_library(L):
    """mx_synth.h's generator is exported by libmx355_synth.so only: the product
    library carries nothing but the method."""
    S = mx.synth_lib()
    names = declared_functions(SYNTH_HEADER)
    assert names == set(mx.SYNTH_SIGNATURES), names ^ set(mx.SYNTH_SIGNATURES)
    for n in names:
        assert hasattr(S, n), n
        assert not hasattr(L, n), n


def test_status_strings(L):
    for s in range(7):
        assert L.mx_status_string(s).decode().startswith(
            ["MX_OK", "MX_ERR_NULL", "MX_ERR_SHAPE", "MX_ERR_ALIGN", "MX_ERR_ENUM",
             "MX_ERR_WORKSPACE", "MX_ERR_HIP"][s])
    assert "unknown" in L.mx_status_string(99).decode()


BAD = 0x1001       # non-null, misaligned: validation must reject it without dereferencing
GOOD = 0x10000     # non-null, aligned: only reached by calls that fail validation first


def test_quantize_validation(L):
    q = L.mx_quantize
    assert q(None, 0, 32, 32, 0, 0, 0, 0, 0, None, None, None) == mx.MX_ERR_NULL
    assert q(GOOD, 2, 32, 32, 0, 0, 0, 0, 0, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert q(GOOD, 0, 32, 32, 2, 0, 0, 0, 0, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert q(GOOD, 0, 32, 32, 0, 2, 0, 0, 0, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert q(GOOD, 0, 32, 32, 0, 0, 0, 3, 0, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert q(GOOD, 0, 32, 31, 0, 0, 0, 0, 0, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert q(GOOD, 0, 31, 32, 1, 0, 0, 0, 0, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert q(GOOD, 0, 32, 12, 1, 0, 0, 0, 0, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert q(GOOD, 0, -32, 32, 0, 0, 0, 0, 0, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert q(BAD, 0, 32, 32, 0, 0, 0, 0, 0, GOOD, GOOD, None) == mx.MX_ERR_ALIGN
    assert q(GOOD, 0, 32, 32, 0, 0, 0, 0, 0, BAD, GOOD, None) == mx.MX_ERR_ALIGN
    # empty tensors are a no-op, even with NULL pointers
    assert q(None, 0, 0, 32, 0, 0, 0, 0, 0, None, None, None) == mx.MX_OK
    assert q(None, 1, 64, 0, 1, 1, 0, 0, 0, None, None, None) == mx.MX_OK


def test_other_quantizer_validation(L):
    assert L.mx_quantize_dual(GOOD, 0, 32, 48, 0, 0, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert L.mx_quantize_dual(GOOD, 0, 32, 32, 0, 0, 0, GOOD, None, GOOD, GOOD, None) == mx.MX_ERR_NULL
    assert L.mx_requantize(GOOD, GOOD, 32, 40, 1, 0, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert L.mx_requantize(GOOD, GOOD, 32, 32, 5, 0, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert L.mx_requantize(GOOD, GOOD, 32, 32, 1, 0, BAD, GOOD, None) == mx.MX_ERR_ALIGN
    assert L.mx_dequantize(GOOD, GOOD, 32, 32, 0, 0, 0, GOOD, 7, None) == mx.MX_ERR_ENUM
    assert L.mx_dequantize(GOOD, GOOD, 30, 32, 1, 0, 0, GOOD, 0, None) == mx.MX_ERR_SHAPE
    assert L.mx_dequantize(GOOD, None, 32, 32, 0, 0, 0, GOOD, 0, None) == mx.MX_ERR_NULL


def test_pair_entry_points_validation(L):
    qp, rp = L.mx_quantize_pair, L.mx_requantize_pair
    # x0, rows0, x1, rows1, cols, dtype, round, seed0, seed1, had, mask, c0, s0, c1, s1, stream
    assert qp(GOOD, 32, GOOD, 64, 48, 0, 0, 0, 0, 0, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert qp(GOOD, -32, GOOD, 64, 64, 0, 0, 0, 0, 0, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert qp(GOOD, 32, GOOD, 64, 64, 3, 0, 0, 0, 0, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert qp(GOOD, 32, GOOD, 64, 64, 0, 2, 0, 0, 0, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert qp(GOOD, 32, GOOD, 64, 64, 0, 0, 0, 0, 2, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert qp(GOOD, 32, None, 64, 64, 0, 0, 0, 0, 0, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_NULL
    assert qp(GOOD, 32, GOOD, 64, 64, 0, 0, 0, 0, 0, 0, BAD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_ALIGN
    # a tensor with no rows is skipped and may be NULL; both empty is a no-op
    assert qp(None, 0, None, 0, 64, 0, 0, 0, 0, 0, 0, None, None, None, None, None) == mx.MX_OK
    # codes_in0, scales_in0, rows0, codes_in1, scales_in1, rows1, cols, round, seed0, seed1, outs, stream
    assert rp(GOOD, GOOD, 32, GOOD, GOOD, 48, 64, 1, 0, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert rp(GOOD, GOOD, 32, GOOD, GOOD, 64, 40, 1, 0, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert rp(GOOD, GOOD, 32, GOOD, GOOD, 64, 64, 4, 0, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert rp(GOOD, GOOD, 32, GOOD, None, 64, 64, 1, 0, 0, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_NULL
    assert rp(GOOD, GOOD, 32, GOOD, GOOD, 64, 64, 1, 0, 0, GOOD, GOOD, BAD, GOOD, None) == mx.MX_ERR_ALIGN
    assert rp(None, None, 0, None, None, 0, 64, 1, 0, 0, None, None, None, None, None) == mx.MX_OK


def test_gemm_validation(L):
    g = L.mx_gemm
    assert g(GOOD, GOOD, GOOD, GOOD, 4, 4, 48, 1.0, GOOD, 4, None) == mx.MX_ERR_SHAPE   # K % 32
    assert g(GOOD, GOOD, GOOD, GOOD, 4, 8, 64, 1.0, GOOD, 4, None) == mx.MX_ERR_SHAPE   # ldc < N
    assert g(GOOD, GOOD, GOOD, GOOD, 4, 6, 64, 1.0, GOOD, 6, None) == mx.MX_ERR_SHAPE   # ldc % 4
    assert g(GOOD, None, GOOD, GOOD, 4, 4, 64, 1.0, GOOD, 4, None) == mx.MX_ERR_NULL
    assert g(GOOD, GOOD, GOOD, GOOD, 4, 4, 64, 1.0, BAD, 4, None) == mx.MX_ERR_ALIGN
    assert g(GOOD, GOOD, GOOD, GOOD, 4, 4, 1 << 31, 1.0, GOOD, 4, None) == mx.MX_ERR_SHAPE  # K > 2^31 - 1
    assert g(None, None, None, None, 0, 4, 64, 1.0, None, 4, None) == mx.MX_OK


def test_grouped_gemm_validation(L):
    offs = (ctypes.c_int64 * 4)(0, 10, 5, 20)             # decreasing offsets
    gg = L.mx_gemm_grouped
    assert gg(GOOD, GOOD, GOOD, GOOD, ctypes.addressof(offs), 3, 8, 64, 1.0, GOOD, None) == mx.MX_ERR_SHAPE
    ok = (ctypes.c_int64 * 3)(0, 10, 20)
    assert gg(GOOD, GOOD, GOOD, GOOD, ctypes.addressof(ok), 0, 8, 64, 1.0, GOOD, None) == mx.MX_ERR_SHAPE
    assert gg(GOOD, GOOD, GOOD, GOOD, ctypes.addressof(ok), 2, 6, 64, 1.0, GOOD, None) == mx.MX_ERR_SHAPE
    assert gg(GOOD, GOOD, GOOD, GOOD, None, 2, 8, 64, 1.0, GOOD, None) == mx.MX_ERR_NULL
    assert gg(GOOD, GOOD, GOOD, GOOD, ctypes.addressof(ok), 2, 8, 1 << 31, 1.0, GOOD, None) == mx.MX_ERR_SHAPE
    big = (ctypes.c_int64 * 200)(*range(200))
    assert gg(GOOD, GOOD, GOOD, GOOD, ctypes.addressof(big), 199, 8, 64, 1.0, GOOD, None) == mx.MX_ERR_SHAPE


def test_pitched_entry_points_validation(L):
    """The scale-pitch variants reject a pitch below the blocks per row, then
    validate like their packed counterparts."""
    q = L.mx_quantize_ld
    assert q(GOOD, mx.MX_F32, 64, 128, mx.MX_ROW, 0, 0, 0, 0, GOOD, GOOD, 3, None) == mx.MX_ERR_SHAPE
    assert q(GOOD, mx.MX_F32, 64, 128, mx.MX_COL, 0, 0, 0, 0, GOOD, GOOD, 1, None) == mx.MX_ERR_SHAPE
    assert q(GOOD, mx.MX_F32, 64, 100, mx.MX_ROW, 0, 0, 0, 0, GOOD, GOOD, 16, None) == mx.MX_ERR_SHAPE
    assert q(GOOD, 7, 64, 128, mx.MX_ROW, 0, 0, 0, 0, GOOD, GOOD, 16, None) == mx.MX_ERR_ENUM
    assert q(GOOD, mx.MX_F32, 64, 128, mx.MX_ROW, 0, 0, 0, 0, None, GOOD, 16, None) == mx.MX_ERR_NULL
    assert q(BAD, mx.MX_F32, 64, 128, mx.MX_ROW, 0, 0, 0, 0, GOOD, GOOD, 16, None) == mx.MX_ERR_ALIGN
    assert q(None, mx.MX_F32, 0, 128, mx.MX_ROW, 0, 0, 0, 0, None, None, 16, None) == mx.MX_OK
    g = L.mx_gemm_ld
    assert g(GOOD, GOOD, 1, GOOD, GOOD, 2, 4, 4, 64, 1.0, GOOD, 4, None) == mx.MX_ERR_SHAPE  # a_scale_ld < K/32
    assert g(GOOD, GOOD, 2, GOOD, GOOD, 1, 4, 4, 64, 1.0, GOOD, 4, None) == mx.MX_ERR_SHAPE  # b_scale_ld < K/32
    assert g(GOOD, GOOD, 16, GOOD, GOOD, 16, 4, 4, 48, 1.0, GOOD, 4, None) == mx.MX_ERR_SHAPE
    assert g(GOOD, None, 16, GOOD, GOOD, 16, 4, 4, 64, 1.0, GOOD, 4, None) == mx.MX_ERR_NULL
    assert g(GOOD, GOOD, 16, GOOD, GOOD, 16, 4, 4, 64, 1.0, BAD, 4, None) == mx.MX_ERR_ALIGN
    ok = (ctypes.c_int64 * 3)(0, 10, 20)
    gg = L.mx_gemm_grouped_ld
    assert gg(GOOD, GOOD, 1, GOOD, GOOD, 16, ctypes.addressof(ok), 2, 8, 64, 1.0, GOOD, None) == mx.MX_ERR_SHAPE
    assert gg(GOOD, GOOD, 16, GOOD, GOOD, 16, None, 2, 8, 64, 1.0, GOOD, None) == mx.MX_ERR_NULL
    bad = (ctypes.c_int64 * 3)(0, 10, 5)
    assert gg(GOOD, GOOD, 16, GOOD, GOOD, 16, ctypes.addressof(bad), 2, 8, 64, 1.0, GOOD, None) == mx.MX_ERR_SHAPE


def test_linear_validation_and_workspace_size(L):
    need = L.mx_linear_bwd_workspace_size(8192, 14336, 4096)
    packed = 0.53125
    assert need >= int(packed * 2 * (8192 * 14336 + 4096 * 14336 / 2 + 4096 * 8192 / 2) * 0.99)
    assert need % 256 == 0
    assert L.mx_linear_bwd_workspace_size(-1, 2, 3) == 0
    assert L.mx_linear_fwd(GOOD, GOOD, 0, 64, 64, 48, GOOD, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert L.mx_linear_fwd(GOOD, GOOD, 3, 64, 64, 64, GOOD, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    # dimensions past the GEMM's 32-bit contraction bound fail before any launch
    assert L.mx_linear_fwd(GOOD, GOOD, 0, 64, 64, 1 << 31, GOOD, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    big = [GOOD, 0, 1 << 31, 64, 64, GOOD, GOOD, GOOD, GOOD, 0, GOOD, GOOD]
    assert L.mx_linear_bwd(*big, GOOD, 1 << 30, None) == mx.MX_ERR_SHAPE
    offs = (ctypes.c_int64 * 2)(0, 64)
    assert L.mx_grouped_linear_bwd(GOOD, 0, ctypes.addressof(offs), 1, 1 << 31, 64, GOOD, GOOD,
                                   GOOD, GOOD, 0, GOOD, GOOD, GOOD, 1 << 30, None) == mx.MX_ERR_SHAPE
    args = [GOOD, 0, 64, 64, 64, GOOD, GOOD, GOOD, GOOD, 0, GOOD, GOOD]
    small = L.mx_linear_bwd_workspace_size(64, 64, 64) - 16
    assert L.mx_linear_bwd(*args, GOOD, small, None) == mx.MX_ERR_WORKSPACE
    assert L.mx_linear_bwd(*args, None, 1 << 30, None) == mx.MX_ERR_WORKSPACE
    assert L.mx_linear_bwd(*args, BAD, 1 << 30, None) == mx.MX_ERR_ALIGN
    # empty contractions: only the zero-filled output is required (validated
    # before the fill kernel; a NULL operand is fine)
    assert L.mx_linear_fwd(None, None, 0, 64, 64, 0, None, None, None, None, None, None) == mx.MX_ERR_NULL
    assert L.mx_linear_fwd(None, None, 0, 64, 64, 0, BAD, None, None, None, None, None) == mx.MX_ERR_ALIGN
    assert L.mx_linear_fwd(None, None, 0, 0, 64, 0, None, None, None, None, None, None) == mx.MX_OK
    assert L.mx_linear_bwd(None, 0, 0, 64, 64, None, None, None, None, 0, None, None, None, 0,
                           None) == mx.MX_ERR_NULL                     # dW required when N > 0
    assert L.mx_linear_bwd(None, 0, 0, 64, 64, None, None, None, None, 0, None, BAD, None, 0,
                           None) == mx.MX_ERR_ALIGN
    assert L.mx_linear_bwd(None, 0, 64, 0, 64, None, None, None, None, 0, None, None, None, 0,
                           None) == mx.MX_ERR_NULL                     # dX required when M > 0
    assert L.mx_linear_bwd(None, 0, 64, 64, 0, None, None, None, None, 0, None, None, None, 0,
                           None) == mx.MX_OK                           # K == 0: nothing to write
    assert L.mx_linear_bwd(None, 0, 0, 0, 64, None, None, None, None, 0, None, None, None, 0,
                           None) == mx.MX_OK


def test_rotated_entry_points_validation(L):
    d = L.mx_quantize_dual_rht
    assert d(GOOD, 2, 32, 32, 1, 1, 2, 5, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert d(GOOD, 1, 32, 40, 1, 1, 2, 5, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert d(GOOD, 1, 32, 32, 1, 1, 2, 5, GOOD, None, GOOD, GOOD, None) == mx.MX_ERR_NULL
    assert d(BAD, 1, 32, 32, 1, 1, 2, 5, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_ALIGN
    r = L.mx_requantize_rht
    assert r(GOOD, GOOD, 32, 48, 1, 1, 5, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert r(GOOD, GOOD, 32, 32, 3, 1, 5, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert r(GOOD, None, 32, 32, 1, 1, 5, GOOD, GOOD, None) == mx.MX_ERR_NULL
    assert r(GOOD, GOOD, 32, 32, 1, 1, 5, BAD, GOOD, None) == mx.MX_ERR_ALIGN
    f = L.mx_linear_fwd_rht
    assert f(GOOD, GOOD, 1, 32, 32, 40, 5, GOOD, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert f(GOOD, GOOD, 7, 32, 32, 32, 5, GOOD, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert f(GOOD, None, 1, 32, 32, 32, 5, GOOD, GOOD, GOOD, GOOD, GOOD, None) == mx.MX_ERR_NULL
    b = L.mx_linear_bwd_rht
    need = L.mx_linear_bwd_workspace_size(32, 32, 32)
    assert b(GOOD, 1, 32, 32, 32, GOOD, GOOD, GOOD, GOOD, 1, 5, GOOD, GOOD, GOOD, need - 1,
             None) == mx.MX_ERR_WORKSPACE
    assert b(GOOD, 1, 32, 32, 40, GOOD, GOOD, GOOD, GOOD, 1, 5, GOOD, GOOD, GOOD, need,
             None) == mx.MX_ERR_SHAPE
    assert b(GOOD, 1, 32, 32, 32, GOOD, GOOD, GOOD, GOOD, 1, 5, GOOD, None, GOOD, need,
             None) == mx.MX_ERR_NULL


def test_segment_entry_points_validation(L):
    import ctypes
    offs = (ctypes.c_int64 * 4)(0, 37, 37, 100)
    bad = (ctypes.c_int64 * 4)(0, 37, 30, 100)       # decreasing
    a, b = ctypes.addressof(offs), ctypes.addressof(bad)
    assert L.mx_segments_padded_rows(a, 3) == 256
    assert L.mx_segments_padded_rows(b, 3) == -1
    q = L.mx_quantize_segments
    assert q(GOOD, 1, 100, 60, a, 3, 1, 5, GOOD, GOOD, None) == mx.MX_ERR_SHAPE   # cols % 8
    assert q(GOOD, 1, 100, 64, b, 3, 1, 5, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert q(GOOD, 1, 99, 64, a, 3, 1, 5, GOOD, GOOD, None) == mx.MX_ERR_SHAPE    # offs[end] != rows
    assert q(GOOD, 1, 100, 64, a, 3, 1, 5, GOOD, None, None) == mx.MX_ERR_NULL
    assert q(GOOD, 1, 100, 64, a, 3, 1, 5, BAD, GOOD, None) == mx.MX_ERR_ALIGN
    r = L.mx_requantize_segments
    assert r(GOOD, GOOD, 100, 48, a, 3, 1, 5, GOOD, GOOD, None) == mx.MX_ERR_SHAPE  # cols % 32
    assert r(GOOD, GOOD, 100, 64, a, 3, 4, 5, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert r(GOOD, GOOD, 100, 64, a, 3, 1, 5, GOOD, None, None) == mx.MX_ERR_NULL
    g = L.mx_grouped_linear_bwd
    need = L.mx_grouped_linear_bwd_workspace_size(a, 3, 64, 96)
    assert need > 0 and L.mx_grouped_linear_bwd_workspace_size(b, 3, 64, 96) == 0
    args = (GOOD, GOOD, GOOD, GOOD, 7, GOOD, GOOD, GOOD)
    assert g(GOOD, 1, a, 3, 64, 96, *args, need - 1, None) == mx.MX_ERR_WORKSPACE
    assert g(GOOD, 1, a, 3, 64, 80, *args, need, None) == mx.MX_ERR_SHAPE
    assert g(GOOD, 1, b, 3, 64, 96, *args, need, None) == mx.MX_ERR_SHAPE
    assert g(GOOD, 5, a, 3, 64, 96, *args, need, None) == mx.MX_ERR_ENUM
    assert g(GOOD, 1, a, 3, 64, 96, GOOD, GOOD, GOOD, GOOD, 7, GOOD, None, GOOD, need,
             None) == mx.MX_ERR_NULL


def test_deosc_validation(L):
    assert L.mx_deosc_step(GOOD, 4, 40, GOOD, GOOD, GOOD, 0, 4.0, None, None) == mx.MX_ERR_SHAPE
    assert L.mx_deosc_step(GOOD, 4, 32, GOOD, GOOD, GOOD, 1, 4.0, None, None) == mx.MX_ERR_NULL
    assert L.mx_deosc_step(GOOD, 4, 32, GOOD, GOOD, GOOD, 2, 4.0, GOOD, None) == mx.MX_ERR_ENUM
    assert L.mx_deosc_step(GOOD, 4, 32, BAD, GOOD, GOOD, 0, 4.0, None, None) == mx.MX_ERR_ALIGN
    assert L.mx_deosc_init(GOOD, 4, 32, GOOD, None, GOOD, None) == mx.MX_ERR_NULL
    q = L.mx_deosc_step_quantize
    assert q(GOOD, 4, 40, GOOD, GOOD, GOOD, 0, 4.0, None, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert q(GOOD, 4, 32, GOOD, GOOD, GOOD, 0, 4.0, None, None, GOOD, None) == mx.MX_ERR_NULL
    assert q(GOOD, 4, 32, GOOD, GOOD, GOOD, 1, 4.0, None, GOOD, GOOD, None) == mx.MX_ERR_NULL
    assert q(GOOD, 4, 32, GOOD, GOOD, GOOD, 3, 4.0, GOOD, GOOD, GOOD, None) == mx.MX_ERR_ENUM
    assert q(GOOD, 4, 32, GOOD, GOOD, GOOD, 0, 4.0, None, BAD, GOOD, None) == mx.MX_ERR_ALIGN
    assert q(GOOD, 0, 32, None, None, None, 0, 4.0, None, None, None, None) == mx.MX_OK
    e = L.mx_qema_step
    assert e(GOOD, GOOD, 4, 48, 0.998, GOOD, GOOD, None) == mx.MX_ERR_SHAPE
    assert e(GOOD, None, 4, 32, 0.998, GOOD, GOOD, None) == mx.MX_ERR_NULL
    assert e(GOOD, GOOD, 4, 32, 0.998, GOOD, None, None) == mx.MX_ERR_NULL
    assert e(BAD, GOOD, 4, 32, 0.998, GOOD, GOOD, None) == mx.MX_ERR_ALIGN
    assert e(None, None, 4, 0, 0.998, None, None, None) == mx.MX_OK
    S = mx.synth_lib()
    assert S.mx_synth_step(GOOD, 1 << 41, 0, 1, None) == mx.MX_ERR_SHAPE
    assert S.mx_synth_step(BAD, 16, 0, 1, None) == mx.MX_ERR_ALIGN


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mx, "_lib", None)
    monkeypatch.setattr(mx, "LIB_PATH", tmp_path / "missing.so")
    with pytest.raises(RuntimeError, match="missing"):
        mx.lib()


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "mxfp4_microscaling_quantization_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f
