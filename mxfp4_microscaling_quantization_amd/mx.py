"""ctypes binding of libmx355.so (include/mx.h) and of the workload generator
libmx355_synth.so (include/mx_synth.h).

Argument marshalling only: every step of the hot path runs in the HIP library.
The functions named like the C entry points take torch tensors (device memory)
and the current torch stream; they raise MxError on a non-zero status.  The
library is loaded on first use and a missing build raises immediately -- there
is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import torch

MX_OK, MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_ENUM, MX_ERR_WORKSPACE, MX_ERR_HIP = range(7)
MX_F32, MX_BF16 = 0, 1
MX_ROW, MX_COL = 0, 1
MX_RNE, MX_SR = 0, 1
MX_MAX_GROUPS = 128

LIB_PATH = Path(__file__).resolve().parent / "libmx355.so"
SYNTH_LIB_PATH = Path(__file__).resolve().parent / "libmx355_synth.so"

_c_void_p, _i64, _u64, _u32, _i32, _f32, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                                  ctypes.c_uint32, ctypes.c_int, ctypes.c_float,
                                                  ctypes.c_size_t)
_P = _c_void_p
SIGNATURES = {
    "mx_status_string": ([_i32], ctypes.c_char_p),
    "mx_quantize": ([_P, _i32, _i64, _i64, _i32, _i32, _u64, _i32, _u32, _P, _P, _P], _i32),
    "mx_quantize_ld": ([_P, _i32, _i64, _i64, _i32, _i32, _u64, _i32, _u32, _P, _P, _i64, _P], _i32),
    "mx_quantize_dual": ([_P, _i32, _i64, _i64, _i32, _u64, _u64, _P, _P, _P, _P, _P], _i32),
    "mx_requantize": ([_P, _P, _i64, _i64, _i32, _u64, _P, _P, _P], _i32),
    "mx_quantize_pair": ([_P, _i64, _P, _i64, _i64, _i32, _i32, _u64, _u64, _i32, _u32,
                          _P, _P, _P, _P, _P], _i32),
    "mx_requantize_pair": ([_P, _P, _i64, _P, _P, _i64, _i64, _i32, _u64, _u64,
                            _P, _P, _P, _P, _P], _i32),
    "mx_quantize_dual_rht": ([_P, _i32, _i64, _i64, _i32, _u64, _u64, _u32, _P, _P, _P, _P, _P], _i32),
    "mx_requantize_rht": ([_P, _P, _i64, _i64, _i32, _u64, _u32, _P, _P, _P], _i32),
    "mx_segments_padded_rows": ([_P, _i64], _i64),
    "mx_quantize_segments": ([_P, _i32, _i64, _i64, _P, _i64, _i32, _u64, _P, _P, _P], _i32),
    "mx_requantize_segments": ([_P, _P, _i64, _i64, _P, _i64, _i32, _u64, _P, _P, _P], _i32),
    "mx_dequantize": ([_P, _P, _i64, _i64, _i32, _i32, _u32, _P, _i32, _P], _i32),
    "mx_gemm": ([_P, _P, _P, _P, _i64, _i64, _i64, _f32, _P, _i64, _P], _i32),
    "mx_gemm_grouped": ([_P, _P, _P, _P, _P, _i64, _i64, _i64, _f32, _P, _P], _i32),
    "mx_gemm_ld": ([_P, _P, _i64, _P, _P, _i64, _i64, _i64, _i64, _f32, _P, _i64, _P], _i32),
    "mx_gemm_grouped_ld": ([_P, _P, _i64, _P, _P, _i64, _P, _i64, _i64, _i64, _f32, _P, _P], _i32),
    "mx_linear_fwd": ([_P, _P, _i32, _i64, _i64, _i64, _P, _P, _P, _P, _P, _P], _i32),
    "mx_linear_bwd_workspace_size": ([_i64, _i64, _i64], _sz),
    "mx_linear_bwd": ([_P, _i32, _i64, _i64, _i64, _P, _P, _P, _P, _u64, _P, _P, _P, _sz, _P], _i32),
    "mx_linear_bwd_noalloc": ([_P, _i32, _i64, _i64, _i64, _P, _P, _P, _P, _u64, _P, _P, _P], _i32),
    "mx_linear_bwd_noalloc_max_workspace": ([], _sz),
    "mx_grouped_linear_bwd_workspace_size": ([_P, _i64, _i64, _i64], _sz),
    "mx_grouped_linear_bwd": ([_P, _i32, _P, _i64, _i64, _i64, _P, _P, _P, _P, _u64, _P, _P, _P, _sz,
                               _P], _i32),
    "mx_linear_fwd_rht": ([_P, _P, _i32, _i64, _i64, _i64, _u32, _P, _P, _P, _P, _P, _P], _i32),
    "mx_linear_bwd_rht": ([_P, _i32, _i64, _i64, _i64, _P, _P, _P, _P, _u64, _u32, _P, _P, _P, _sz,
                           _P], _i32),
    "mx_deosc_init": ([_P, _i64, _i64, _P, _P, _P, _P], _i32),
    "mx_deosc_step": ([_P, _i64, _i64, _P, _P, _P, _i32, _f32, _P, _P], _i32),
    "mx_deosc_step_quantize": ([_P, _i64, _i64, _P, _P, _P, _i32, _f32, _P, _P, _P, _P], _i32),
    "mx_qema_step": ([_P, _P, _i64, _i64, _f32, _P, _P, _P], _i32),
}
SYNTH_SIGNATURES = {
    "mx_synth_step": ([_P, _i64, _u64, _i64, _P], _i32),
}

_lib = None
_synth_lib = None


class MxError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} -> {status_string(status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mxfp4_microscaling_quantization_amd.build`")
        handle = ctypes.CDLL(str(LIB_PATH))
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def synth_lib() -> ctypes.CDLL:
    """The workload generator's library (the synthetic optimizer steps); raises if
    it has not been built."""
    global _synth_lib
    if _synth_lib is None:
        if not SYNTH_LIB_PATH.exists():
            raise RuntimeError(f"{SYNTH_LIB_PATH} is missing: build it with "
                               "`python -m mxfp4_microscaling_quantization_amd.build`")
        handle = ctypes.CDLL(str(SYNTH_LIB_PATH))
        for name, (args, res) in SYNTH_SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _synth_lib = handle
    return _synth_lib


def status_string(status: int) -> str:
    return lib().mx_status_string(int(status)).decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(name: str, status: int) -> None:
    if status != MX_OK:
        raise MxError(name, status)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MX_F32
    if t.dtype == torch.bfloat16:
        return MX_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ C-named entry points
def mx_quantize(x, dtype, rows, cols, axis, round, seed, hadamard, sign_mask, codes, scales,
                stream=None):
    _check("mx_quantize", lib().mx_quantize(_ptr(x), dtype, rows, cols, axis, round, seed,
                                            hadamard, sign_mask, _ptr(codes), _ptr(scales),
                                            _stream(stream)))


def mx_quantize_ld(x, dtype, rows, cols, axis, round, seed, hadamard, sign_mask, codes, scales,
                   scale_ld, stream=None):
    _check("mx_quantize_ld", lib().mx_quantize_ld(_ptr(x), dtype, rows, cols, axis, round, seed,
                                                  hadamard, sign_mask, _ptr(codes), _ptr(scales),
                                                  scale_ld, _stream(stream)))


def mx_quantize_dual(x, dtype, rows, cols, round, seed_row, seed_col, codes_row, scales_row,
                     codes_col, scales_col, stream=None):
    _check("mx_quantize_dual", lib().mx_quantize_dual(
        _ptr(x), dtype, rows, cols, round, seed_row, seed_col, _ptr(codes_row), _ptr(scales_row),
        _ptr(codes_col), _ptr(scales_col), _stream(stream)))


def mx_quantize_dual_rht(x, dtype, rows, cols, round, seed_row, seed_col, sign_mask, codes_row,
                         scales_row, codes_col, scales_col, stream=None):
    _check("mx_quantize_dual_rht", lib().mx_quantize_dual_rht(
        _ptr(x), dtype, rows, cols, round, seed_row, seed_col, sign_mask, _ptr(codes_row),
        _ptr(scales_row), _ptr(codes_col), _ptr(scales_col), _stream(stream)))


def mx_requantize_rht(codes_in, scales_in, rows, cols, round, seed, sign_mask, codes_out,
                      scales_out, stream=None):
    _check("mx_requantize_rht", lib().mx_requantize_rht(
        _ptr(codes_in), _ptr(scales_in), rows, cols, round, seed, sign_mask, _ptr(codes_out),
        _ptr(scales_out), _stream(stream)))


def mx_requantize(codes_in, scales_in, rows, cols, round, seed, codes_out, scales_out, stream=None):
    _check("mx_requantize", lib().mx_requantize(_ptr(codes_in), _ptr(scales_in), rows, cols, round,
                                                seed, _ptr(codes_out), _ptr(scales_out),
                                                _stream(stream)))


def mx_quantize_pair(x0, rows0, x1, rows1, cols, dtype, round, seed0, seed1, hadamard, sign_mask,
                     codes0, scales0, codes1, scales1, stream=None):
    _check("mx_quantize_pair", lib().mx_quantize_pair(
        _ptr(x0), rows0, _ptr(x1), rows1, cols, dtype, round, seed0, seed1, hadamard, sign_mask,
        _ptr(codes0), _ptr(scales0), _ptr(codes1), _ptr(scales1), _stream(stream)))


def mx_requantize_pair(codes_in0, scales_in0, rows0, codes_in1, scales_in1, rows1, cols, round,
                       seed0, seed1, codes_out0, scales_out0, codes_out1, scales_out1,
                       stream=None):
    _check("mx_requantize_pair", lib().mx_requantize_pair(
        _ptr(codes_in0), _ptr(scales_in0), rows0, _ptr(codes_in1), _ptr(scales_in1), rows1, cols,
        round, seed0, seed1, _ptr(codes_out0), _ptr(scales_out0), _ptr(codes_out1),
        _ptr(scales_out1), _stream(stream)))


def mx_dequantize(codes, scales, rows, cols, axis, hadamard, sign_mask, out, out_dtype,
                  stream=None):
    _check("mx_dequantize", lib().mx_dequantize(_ptr(codes), _ptr(scales), rows, cols, axis,
                                                hadamard, sign_mask, _ptr(out), out_dtype,
                                                _stream(stream)))


def mx_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, alpha, c, ldc, stream=None):
    _check("mx_gemm", lib().mx_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales),
                                    M, N, K, alpha, _ptr(c), ldc, _stream(stream)))


def mx_gemm_ld(a_codes, a_scales, a_scale_ld, b_codes, b_scales, b_scale_ld, M, N, K, alpha, c,
               ldc, stream=None):
    _check("mx_gemm_ld", lib().mx_gemm_ld(_ptr(a_codes), _ptr(a_scales), a_scale_ld,
                                          _ptr(b_codes), _ptr(b_scales), b_scale_ld, M, N, K,
                                          alpha, _ptr(c), ldc, _stream(stream)))


def _offsets(offs):
    """Host int64 array of the offsets (kept alive by the caller's reference)."""
    return (ctypes.c_int64 * len(offs))(*[int(o) for o in offs])


def mx_segments_padded_rows(offs, groups) -> int:
    arr = _offsets(offs)
    return int(lib().mx_segments_padded_rows(ctypes.addressof(arr), groups))


def mx_quantize_segments(x, dtype, rows, cols, offs, groups, round, seed, codes, scales,
                         stream=None):
    arr = _offsets(offs)
    _check("mx_quantize_segments", lib().mx_quantize_segments(
        _ptr(x), dtype, rows, cols, ctypes.addressof(arr), groups, round, seed, _ptr(codes),
        _ptr(scales), _stream(stream)))


def mx_requantize_segments(codes_in, scales_in, rows, cols, offs, groups, round, seed, codes_out,
                           scales_out, stream=None):
    arr = _offsets(offs)
    _check("mx_requantize_segments", lib().mx_requantize_segments(
        _ptr(codes_in), _ptr(scales_in), rows, cols, ctypes.addressof(arr), groups, round, seed,
        _ptr(codes_out), _ptr(scales_out), _stream(stream)))


def mx_grouped_linear_bwd_workspace_size(offs, groups, N, K) -> int:
    arr = _offsets(offs)
    return int(lib().mx_grouped_linear_bwd_workspace_size(ctypes.addressof(arr), groups, N, K))


def mx_grouped_linear_bwd(dy, dtype, offs, groups, N, K, xq_codes, xq_scales, wq_codes, wq_scales,
                          seed, dx, dw, workspace, workspace_bytes, stream=None):
    arr = _offsets(offs)
    _check("mx_grouped_linear_bwd", lib().mx_grouped_linear_bwd(
        _ptr(dy), dtype, ctypes.addressof(arr), groups, N, K, _ptr(xq_codes), _ptr(xq_scales),
        _ptr(wq_codes), _ptr(wq_scales), seed, _ptr(dx), _ptr(dw), _ptr(workspace),
        workspace_bytes, _stream(stream)))


def mx_gemm_grouped(a_codes, a_scales, b_codes, b_scales, offs, groups, N, K, alpha, c,
                    stream=None):
    arr = _offsets(offs)
    _check("mx_gemm_grouped", lib().mx_gemm_grouped(
        _ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), ctypes.addressof(arr),
        groups, N, K, alpha, _ptr(c), _stream(stream)))


def mx_gemm_grouped_ld(a_codes, a_scales, a_scale_ld, b_codes, b_scales, b_scale_ld, offs, groups,
                       N, K, alpha, c, stream=None):
    arr = _offsets(offs)
    _check("mx_gemm_grouped_ld", lib().mx_gemm_grouped_ld(
        _ptr(a_codes), _ptr(a_scales), a_scale_ld, _ptr(b_codes), _ptr(b_scales), b_scale_ld,
        ctypes.addressof(arr), groups, N, K, alpha, _ptr(c), _stream(stream)))


def mx_linear_fwd(x, w, dtype, M, N, K, y, xq_codes, xq_scales, wq_codes, wq_scales, stream=None):
    _check("mx_linear_fwd", lib().mx_linear_fwd(_ptr(x), _ptr(w), dtype, M, N, K, _ptr(y),
                                                _ptr(xq_codes), _ptr(xq_scales), _ptr(wq_codes),
                                                _ptr(wq_scales), _stream(stream)))


def mx_linear_fwd_rht(x, w, dtype, M, N, K, sign_mask, y, xq_codes, xq_scales, wq_codes,
                      wq_scales, stream=None):
    _check("mx_linear_fwd_rht", lib().mx_linear_fwd_rht(
        _ptr(x), _ptr(w), dtype, M, N, K, sign_mask, _ptr(y), _ptr(xq_codes), _ptr(xq_scales),
        _ptr(wq_codes), _ptr(wq_scales), _stream(stream)))


def mx_linear_bwd_workspace_size(M, N, K) -> int:
    return int(lib().mx_linear_bwd_workspace_size(M, N, K))


def mx_linear_bwd(dy, dtype, M, N, K, xq_codes, xq_scales, wq_codes, wq_scales, seed, dx, dw,
                  workspace, workspace_bytes, stream=None):
    _check("mx_linear_bwd", lib().mx_linear_bwd(
        _ptr(dy), dtype, M, N, K, _ptr(xq_codes), _ptr(xq_scales), _ptr(wq_codes),
        _ptr(wq_scales), seed, _ptr(dx), _ptr(dw), _ptr(workspace), workspace_bytes,
        _stream(stream)))


def mx_linear_bwd_noalloc(dy, dtype, M, N, K, xq_codes, xq_scales, wq_codes, wq_scales, seed, dx,
                          dw, stream=None):
    _check("mx_linear_bwd_noalloc", lib().mx_linear_bwd_noalloc(
        _ptr(dy), dtype, M, N, K, _ptr(xq_codes), _ptr(xq_scales), _ptr(wq_codes),
        _ptr(wq_scales), seed, _ptr(dx), _ptr(dw), _stream(stream)))


def mx_linear_bwd_noalloc_max_workspace():
    return int(lib().mx_linear_bwd_noalloc_max_workspace())


def mx_linear_bwd_rht(dy, dtype, M, N, K, xq_codes, xq_scales, wq_codes, wq_scales, seed,
                      sign_mask, dx, dw, workspace, workspace_bytes, stream=None):
    _check("mx_linear_bwd_rht", lib().mx_linear_bwd_rht(
        _ptr(dy), dtype, M, N, K, _ptr(xq_codes), _ptr(xq_scales), _ptr(wq_codes),
        _ptr(wq_scales), seed, sign_mask, _ptr(dx), _ptr(dw), _ptr(workspace), workspace_bytes,
        _stream(stream)))


def mx_deosc_init(w, rows, cols, w_prev, d_w, d_q, stream=None):
    _check("mx_deosc_init", lib().mx_deosc_init(_ptr(w), rows, cols, _ptr(w_prev), _ptr(d_w),
                                                _ptr(d_q), _stream(stream)))


def mx_deosc_step(w, rows, cols, w_prev, d_w, d_q, end_of_window, threshold, flags, stream=None):
    _check("mx_deosc_step", lib().mx_deosc_step(_ptr(w), rows, cols, _ptr(w_prev), _ptr(d_w),
                                                _ptr(d_q), int(end_of_window), threshold,
                                                _ptr(flags), _stream(stream)))


def mx_deosc_step_quantize(w, rows, cols, w_prev, d_w, d_q, end_of_window, threshold, flags,
                           wq_codes, wq_scales, stream=None):
    _check("mx_deosc_step_quantize",
           lib().mx_deosc_step_quantize(_ptr(w), rows, cols, _ptr(w_prev), _ptr(d_w), _ptr(d_q),
                                        int(end_of_window), threshold, _ptr(flags),
                                        _ptr(wq_codes), _ptr(wq_scales), _stream(stream)))


def mx_qema_step(w, ema, rows, cols, beta, wq_codes, wq_scales, stream=None):
    _check("mx_qema_step", lib().mx_qema_step(_ptr(w), _ptr(ema), rows, cols, beta,
                                              _ptr(wq_codes), _ptr(wq_scales), _stream(stream)))


def mx_synth_step(w, n, seed, step, stream=None):
    _check("mx_synth_step", synth_lib().mx_synth_step(_ptr(w), n, seed, step, _stream(stream)))


# ------------------------------------------------------------------ tensor conveniences
def _u8(shape, device):
    return torch.empty(shape, dtype=torch.uint8, device=device)


def quantize(x: torch.Tensor, axis=MX_ROW, round=MX_RNE, seed=0, hadamard=False, sign_mask=0,
             stream=None):
    """Packed (codes, scales) of a 2-D float32/bf16 device tensor."""
    rows, cols = x.shape
    outer, inner = (rows, cols) if axis == MX_ROW else (cols, rows)
    codes = _u8((outer, inner // 2), x.device)
    scales = _u8((outer, inner // 32), x.device)
    mx_quantize(x, dtype_code(x), rows, cols, axis, round, seed, int(bool(hadamard)), sign_mask,
                codes, scales, stream)
    return codes, scales


def dequantize(codes, scales, rows, cols, axis=MX_ROW, hadamard=False, sign_mask=0,
               out_dtype=torch.float32, stream=None):
    out = torch.empty((rows, cols), dtype=out_dtype, device=codes.device)
    mx_dequantize(codes, scales, rows, cols, axis, int(bool(hadamard)), sign_mask, out,
                  dtype_code(out), stream)
    return out


def requantize(codes, scales, rows, cols, round=MX_SR, seed=0, stream=None):
    co = _u8((cols, rows // 2), codes.device)
    so = _u8((cols, rows // 32), codes.device)
    mx_requantize(codes, scales, rows, cols, round, seed, co, so, stream)
    return co, so


def gemm(a, b, M, N, K, alpha=1.0, stream=None):
    c = torch.empty((M, N), dtype=torch.float32, device=a[0].device)
    mx_gemm(a[0], a[1], b[0], b[1], M, N, K, alpha, c, N, stream)
    return c


def linear_fwd(x: torch.Tensor, w: torch.Tensor, stream=None):
    M, K = x.shape
    N = w.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    xq = (_u8((M, K // 2), x.device), _u8((M, K // 32), x.device))
    wq = (_u8((N, K // 2), x.device), _u8((N, K // 32), x.device))
    mx_linear_fwd(x, w, dtype_code(x), M, N, K, y, xq[0], xq[1], wq[0], wq[1], stream)
    return y, xq, wq


def linear_fwd_rht(x: torch.Tensor, w: torch.Tensor, sign_mask: int, stream=None):
    M, K = x.shape
    N = w.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    xq = (_u8((M, K // 2), x.device), _u8((M, K // 32), x.device))
    wq = (_u8((N, K // 2), x.device), _u8((N, K // 32), x.device))
    mx_linear_fwd_rht(x, w, dtype_code(x), M, N, K, sign_mask, y, xq[0], xq[1], wq[0], wq[1],
                      stream)
    return y, xq, wq


def linear_bwd_rht(dy: torch.Tensor, xq, wq, M, N, K, seed, sign_mask, workspace=None,
                   stream=None):
    need = mx_linear_bwd_workspace_size(M, N, K)
    if workspace is None:
        workspace = _u8((need,), dy.device)
    dx = torch.empty((M, K), dtype=torch.float32, device=dy.device)
    dw = torch.empty((N, K), dtype=torch.float32, device=dy.device)
    mx_linear_bwd_rht(dy, dtype_code(dy), M, N, K, xq[0], xq[1], wq[0], wq[1], seed, sign_mask,
                      dx, dw, workspace, workspace.numel(), stream)
    return dx, dw


def grouped_linear_bwd(dy: torch.Tensor, xq, wq, offs, N, K, seed, workspace=None, stream=None):
    """dX [R, K] and dW [groups, N, K] of a grouped layer (offs: host offsets)."""
    G = len(offs) - 1
    R = int(offs[-1])
    need = mx_grouped_linear_bwd_workspace_size(offs, G, N, K)
    if workspace is None:
        workspace = _u8((need,), wq[0].device)
    dx = torch.empty((R, K), dtype=torch.float32, device=wq[0].device)
    dw = torch.empty((G, N, K), dtype=torch.float32, device=wq[0].device)
    mx_grouped_linear_bwd(dy, dtype_code(dy), offs, G, N, K, xq[0], xq[1], wq[0], wq[1], seed, dx,
                          dw, workspace, workspace.numel(), stream)
    return dx, dw


def linear_bwd(dy: torch.Tensor, xq, wq, M, N, K, seed, workspace=None, stream=None):
    need = mx_linear_bwd_workspace_size(M, N, K)
    if workspace is None:
        workspace = _u8((need,), dy.device)
    dx = torch.empty((M, K), dtype=torch.float32, device=dy.device)
    dw = torch.empty((N, K), dtype=torch.float32, device=dy.device)
    mx_linear_bwd(dy, dtype_code(dy), M, N, K, xq[0], xq[1], wq[0], wq[1], seed, dx, dw,
                  workspace, workspace.numel(), stream)
    return dx, dw
