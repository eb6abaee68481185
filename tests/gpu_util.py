"""Helpers for the GPU parity tests: device upload/download and comparisons."""
import numpy as np
import torch

import oracle as O

DEV = torch.device("cuda:0")


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    b = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(b).to(DEV).view(torch.bfloat16)


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def oracle_input(x: np.ndarray, dtype: str) -> np.ndarray:
    """The float32 values the oracle sees for a host array of the given storage type."""
    return O.bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


def upload(x: np.ndarray, dtype: str) -> torch.Tensor:
    return to_dev_bf16(x) if dtype == "bf16" else to_dev_f32(x)


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        first = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {first}: "
                             f"got {got[first]}, want {want[first]}")


def gemm_tolerance(abs_sum: np.ndarray) -> np.ndarray:
    """|C_gpu - C_oracle| <= 1e-5 * sum_k |a_k b_k|, with a floor at the smallest
    float32 normal for products of extreme scales (they can underflow float32)."""
    return 1e-5 * abs_sum + 2.0 ** -126


def assert_gemm_close(got: np.ndarray, want: np.ndarray, abs_sum: np.ndarray, what: str):
    err = np.abs(got.astype(np.float64) - want)
    tol = gemm_tolerance(abs_sum)
    if not np.all(err <= tol):
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(f"{what}: max err/tol {float((err / tol)[i]):.3g} at {i}: "
                             f"got {got[i]!r}, want {want[i]!r}, sum|ab| {abs_sum[i]!r}")
