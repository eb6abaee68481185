"""Seeded synthetic inputs for the MXFP4 hot path (no MXFP4 arithmetic here).

This module only draws tensors: it is shared by the tests, the benchmark and the
oracle-side checks, and it does not quantize, round to E2M1 or multiply
matrices.  Every generator uses numpy's Generator(PCG64(seed)).  bf16 tensors
are returned as uint16 bit patterns (float32 rounded to nearest-even bf16).

The shapes stand in for the layers the pages train: a DeiT-S MLP fc1 layer
(64 images x 197 tokens, d = 384 -> 1536), a Llama-3-8B MLP up-projection
(4096 -> 14336, 8192 tokens) and a 32-expert, top-4 MoE feed-forward block with
hidden size 2880 ("ALTO MXFP4 training -- Weight de-oscillation", the news
paragraph on GPT-OSS-20B MoE).  No dataset or trained weight is used.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "rng_for",
    "tiny_config", "deit_config", "sweep_config", "llama_config", "moe_config",
    "moe_routing", "moe_master_weights", "deosc_delta_f32", "DEOSC_STEP_SCALE_BITS",
]


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape, std=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _scale_random_entries(rng, x: np.ndarray, fraction: float, factor: float) -> int:
    """Multiply round(fraction * size) distinct entries (sign kept) by `factor`."""
    flat = x.reshape(-1)
    k = int(round(fraction * flat.size))
    if k:
        pos = rng.choice(flat.size, size=k, replace=False)
        flat[pos] *= np.float32(factor)
    return k


def tiny_config(seed: int = 0, n: int = 256):
    """X, W float32 [n, n] ~ N(0, 1), X drawn first, from one generator."""
    rng = rng_for(seed)
    x = _normal(rng, (n, n))
    w = _normal(rng, (n, n))
    return {"x": x, "w": w, "M": n, "N": n, "K": n}


def deit_config(seed: int = 1, M: int = 12608, K: int = 384, N: int = 1536):
    """DeiT-S fc1: X bf16 [M, K] N(0,1) with 0.5% of entries x20; W bf16 [N, K]
    N(0, 0.02); dY bf16 [M, N] N(0, 1e-3)."""
    rng = rng_for(seed)
    x = _normal(rng, (M, K))
    _scale_random_entries(rng, x, 0.005, 20.0)
    w = _normal(rng, (N, K), 0.02)
    dy = _normal(rng, (M, N), 1e-3)
    return {"x": f32_to_bf16_bits(x), "w": f32_to_bf16_bits(w), "dy": f32_to_bf16_bits(dy),
            "M": M, "N": N, "K": K}


def sweep_config(seed: int = 2, rows: int = 8192, cols: int = 8192):
    """Quantizer sweep input: bf16 [rows, cols] Student-t(3), 0.1% of entries x100."""
    rng = rng_for(seed)
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32)
    _scale_random_entries(rng, x, 0.001, 100.0)
    sign_mask = int(_splitmix64_scalar(seed, 0) & 0xFFFFFFFF)
    return {"x": f32_to_bf16_bits(x), "rows": rows, "cols": cols, "sign_mask": sign_mask}


def llama_config(seed: int = 3, M: int = 8192, K: int = 4096, N: int = 14336,
                 outlier_fraction: float = 0.01, outlier_factor: float = 30.0):
    """Llama-3-8B MLP up-projection: X bf16 [M, K] N(0,1) whose outlier channels
    (1% of K, chosen once) are x30; W bf16 [N, K] N(0, 0.02); dY bf16 [M, N] N(0, 1e-3)."""
    rng = rng_for(seed)
    x = _normal(rng, (M, K))
    n_out = int(round(outlier_fraction * K))
    cols = rng.choice(K, size=n_out, replace=False)
    x[:, cols] *= np.float32(outlier_factor)
    w = _normal(rng, (N, K), 0.02)
    dy = _normal(rng, (M, N), 1e-3)
    return {"x": f32_to_bf16_bits(x), "w": f32_to_bf16_bits(w), "dy": f32_to_bf16_bits(dy),
            "M": M, "N": N, "K": K, "outlier_cols": np.sort(cols)}


def moe_routing(seed: int = 4, tokens: int = 16384, experts: int = 32, top_k: int = 4):
    """Uniform-random gate logits -> softmax -> top-k experts per token.

    Returns (row_token [tokens*top_k] int64, offs [experts+1] int64): routed rows
    are expert-major and, within an expert, in increasing token order.
    """
    rng = rng_for(seed)
    logits = rng.random((tokens, experts))
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    top = np.argsort(-p, axis=1, kind="stable")[:, :top_k]
    sel = np.zeros((tokens, experts), dtype=bool)
    sel[np.arange(tokens)[:, None], top] = True
    counts = sel.sum(axis=0)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    row_token = np.concatenate([np.nonzero(sel[:, e])[0] for e in range(experts)]).astype(np.int64)
    return row_token, offs, rng


def moe_config(seed: int = 4, tokens: int = 16384, experts: int = 32, hidden: int = 2880,
               ffn: int = 5760, top_k: int = 4, with_weights: bool = True):
    """MoE block: routed up-projection input (gathered tokens) and down-projection
    input, bf16 N(0,1); fp32 master weights N(0, 0.02), up [E, ffn, hidden] and
    down [E, hidden, hidden], stored as one [E*ffn + E*hidden, hidden] buffer."""
    row_token, offs, rng = moe_routing(seed, tokens, experts, top_k)
    tok = _normal(rng, (tokens, hidden))
    x_up = f32_to_bf16_bits(tok)[row_token]
    x_down = f32_to_bf16_bits(_normal(rng, (offs[-1], hidden)))
    out = {"x_up": x_up, "x_down": x_down, "offs": offs, "row_token": row_token,
           "E": experts, "hidden": hidden, "ffn": ffn}
    if with_weights:
        out["w_master"] = moe_master_weights(rng, experts, hidden, ffn)
    return out


def moe_master_weights(rng, experts: int, hidden: int, ffn: int) -> np.ndarray:
    rows = experts * ffn + experts * hidden
    w = np.empty((rows, hidden), dtype=np.float32)
    chunk = 8192
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        w[r0:r1] = _normal(rng, (r1 - r0, hidden), 0.02)
    return w


# ---------------------------------------------------------------- synthetic optimizer steps
# The de-oscillation workload moves the fp32 master weights by synthetic
# AdamW-like steps of standard deviation 1e-4.  They must be reproducible on
# both sides without a transcendental function, so a step is an Irwin-Hall(4)
# sum of four 24-bit uniforms from SplitMix64 (Steele, Lea & Flood, OOPSLA 2014)
# keyed by (step, k, element index):
#   u_k = SplitMix64(seed, (step << 42) | (k << 40) | idx) >> 40
#   dw  = f32(f32(u_0 + u_1 + u_2 + u_3 - 2^25) * c),  c = f32(sqrt(3) * 1e-4 * 2^-24)
#   w   = f32(w + dw)
DEOSC_STEP_SCALE_BITS = int(np.float32(math.sqrt(3.0) * 1e-4 * 2.0 ** -24).view(np.uint32))


def _splitmix64_scalar(seed: int, idx: int) -> int:
    m = (1 << 64) - 1
    z = (seed + (idx + 1) * 0x9E3779B97F4A7C15) & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def _splitmix64_vec(seed: int, ctr: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (ctr.astype(np.uint64) + np.uint64(1)) * np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def deosc_delta_f32(seed: int, step: int, idx: np.ndarray) -> np.ndarray:
    """Synthetic update dw (float32) for the given flat element indices at `step`."""
    idx = np.asarray(idx, dtype=np.uint64)
    acc = np.zeros(idx.shape, dtype=np.int64)
    for k in range(4):
        ctr = (np.uint64(step) << np.uint64(42)) | (np.uint64(k) << np.uint64(40)) | idx
        acc += (_splitmix64_vec(seed, ctr) >> np.uint64(40)).astype(np.int64)
    centred = (acc - (1 << 25)).astype(np.int32).astype(np.float32)
    c = np.array([DEOSC_STEP_SCALE_BITS], dtype=np.uint32).view(np.float32)[0]
    return (centred * c).astype(np.float32)
