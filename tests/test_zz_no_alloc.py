"""The no-allocation backward entry point, mx_linear_bwd_noalloc, against
mx_linear_bwd with a caller workspace: the same kernels on the same inputs, so
dX and dW must agree bit for bit.  Two calls in a row on the library's one
scratch array, the second with a smaller layer (the array keeps the first
call's contents), and a layer whose workspace exceeds the array is rejected
before anything runs."""
import numpy as np
import pytest
import torch

from mxfp4_microscaling_quantization_amd import mx, synth
from tests.gpu_util import DEV, host

pytestmark = pytest.mark.gpu


def layer_inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    dy = synth.f32_to_bf16_bits((rng.standard_normal((M, N)) * 1e-3).astype(np.float32))
    dev = lambda b: torch.from_numpy(b.view(np.int16)).to(DEV).view(torch.bfloat16)
    return dev(x), dev(w), dev(dy)


def both_ways(M, N, K, seed):
    x, w, dy = layer_inputs(M, N, K, seed)
    _, xq, wq = mx.linear_fwd(x, w)
    want_dx, want_dw = mx.linear_bwd(dy, xq, wq, M, N, K, seed)
    dx = torch.full((M, K), float("nan"), device=DEV)
    dw = torch.full((N, K), float("nan"), device=DEV)
    print(f"mx_linear_bwd_noalloc M={M} N={N} K={K} seed={seed}", flush=True)
    mx.mx_linear_bwd_noalloc(dy, mx.MX_BF16, M, N, K, *xq, *wq, seed, dx, dw)
    return host(dx), host(dw), host(want_dx), host(want_dw)


def test_noalloc_backward_equals_workspace_backward_twice():
    assert mx.mx_linear_bwd_noalloc_max_workspace() == 64 << 20
    # DeiT-S fc1 at full size (split-K partial sums in the scratch array), then a
    # smaller layer that reuses the array's first bytes
    for M, N, K, seed in ((12608, 1536, 384, 1), (1024, 512, 256, 7)):
        assert mx.mx_linear_bwd_workspace_size(M, N, K) <= mx.mx_linear_bwd_noalloc_max_workspace()
        dx, dw, want_dx, want_dw = both_ways(M, N, K, seed)
        assert np.array_equal(dx.view(np.uint32), want_dx.view(np.uint32)), (M, N, K, "dx")
        assert np.array_equal(dw.view(np.uint32), want_dw.view(np.uint32)), (M, N, K, "dw")


def test_noalloc_backward_rejects_layers_beyond_the_scratch_array():
    M, N, K = 8192, 14336, 4096          # 166 MiB of workspace
    assert mx.mx_linear_bwd_workspace_size(M, N, K) > mx.mx_linear_bwd_noalloc_max_workspace()
    dx = torch.empty((16,), device=DEV)
    with pytest.raises(mx.MxError) as e:
        mx.mx_linear_bwd_noalloc(dx, mx.MX_BF16, M, N, K, dx, dx, dx, dx, 1, dx, dx)
    assert e.value.status == mx.MX_ERR_WORKSPACE
