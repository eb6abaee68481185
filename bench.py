"""Benchmark of the MXFP4 training hot path on one MI355X.

Step = one MXFP4 linear forward + backward of the Llama-3-8B MLP up-projection
(M = 8192 tokens, K = 4096, N = 14336, bf16 activations with 1% outlier
channels x30, weights N(0, 0.02), dY N(0, 1e-3)):

  quantize X and W (1x32 RNE, one launch), GEMM Y = Q(X) Q(W)^T,
  dual-quantize dY (1x32 SR + 32x1 SR), requantize Q(W) and Q(X) (32x1 SR,
  one launch), GEMM dX, GEMM dW

-- the kernels mx_linear_fwd / mx_linear_bwd launch, issued one entry point at
a time on one stream.  Before the warm-up steps the bench checks the composed
step against the library's linear entry points (bit for bit) and then runs
REPEAT_CHECK_STEPS steps whose outputs must equal the first step's (bit for
bit); both checks are reported in the line.  value = 6 M N K / step time (TFLOP/s), the steps timed
back to back with events at the two ends of the timed region only (an event
record between kernels stops the next one from starting while the previous one
drains).  The GEMM's launch duration for its roofline comes from a second pass
of the same steps with an event pair around every GEMM launch.  The line also
carries the dominant kernel's roofline (the GEMM, vs the dense FP4 MFMA peak), the oracle's CPU
throughput on a bounded sample, and the other rows of the path measured on
their own workloads: the DeiT-S fc1 layer (12608 x 384 -> 1536) through
mx_linear_fwd / mx_linear_bwd, eager and as a replayed HIP graph; the rotated
layer; the quantizer sweep on 8192^2 bf16; the MoE grouped GEMM and backward
and the de-oscillation and Q-EMA passes on the 32-expert master weights.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np


PEAK_HBM_GBPS = 8000.0
PEAK_FP4_TFLOPS = 10100.0
# HBM bytes per GEMM launch (mean of the fwd, dX and dW launches of the step),
# from rocprofv3 FETCH_SIZE / WRITE_SIZE runs scaled by a 1 GiB copy, valid for
# the GEMM code with this sha256 only (of gemm.hip and gemm_schedule.h with
# comments and blank lines removed; the per-launch table is kept with the
# committed profiles).
GEMM_TRAFFIC = {"sha256": "687e8c008e3ce774e742d19db32d4d205615827319d7c2c8b9f0215985b11acd",
                 "bytes_per_launch": 668365929}
GEMM_SOURCES = ("gemm.hip", "gemm_schedule.h")

# VALU work per element of the stochastic-rounding kernels, valid for the
# quantizer code with this sha256 only (quant.hip and mx_device.h, comments and
# blank lines removed): `lane_ops` = SQ_INSTS_VALU x 64 lanes / elements from a
# rocprofv3 counter run on the 8192^2 bf16 sweep; `counts` = the multi-cycle
# instructions in the kernel's assembly, `elems` = elements one lane converts per
# pass over that code.  Each such instruction occupies its SIMD VALU_COST times
# as long as a simple one (measured by tests/valu_rate_probe.hip), so it adds
# VALU_COST - 1 lane-op equivalents.
QUANT_VALU = {"sha256": "ccc96e99b6ec45bbf2099332e37b8308361e08a3d94e89033a51b0627dc3cd6e",
               "per_elem": {
    "row_sr": {"kernel": "k_quant_row<bf16, SR>", "lane_ops": 15.56, "elems": 32,
               "counts": {"v_mul_lo_u32": 65, "v_mad_u64_u32": 33, "v_lshrrev_b64": 32,
                          "v_cvt_scalef32_sr_pk_fp4_f32": 32}},
    "col_sr": {"kernel": "k_quant_tile<bf16, SR>", "lane_ops": 14.34, "elems": 64,
               "counts": {"v_mul_lo_u32": 140, "v_mad_u64_u32": 73, "v_lshrrev_b64": 64,
                          "v_cvt_scalef32_sr_pk_fp4_f32": 64}},
    "dual_sr": {"kernel": "k_quant_tile<bf16, SR, row + column>", "lane_ops": 30.56, "elems": 64,
                "quantizations": 2,
                "counts": {"v_mul_lo_u32": 272, "v_mad_u64_u32": 163, "v_lshrrev_b64": 137,
                           "v_cvt_scalef32_sr_pk_fp4_f32": 128}},
    "requant_sr": {"kernel": "k_requant<SR>", "lane_ops": 14.68, "elems": 128,
                   "counts": {"v_mul_lo_u32": 272, "v_mad_u64_u32": 208, "v_lshrrev_b64": 130,
                              "v_cvt_scalef32_sr_pk_fp4_f32": 128}},
}}
# SIMD cycles per wave64 instruction relative to v_add_u32 (2 cycles), at four
# waves per SIMD.
VALU_COST = {"v_mul_lo_u32": 1.67, "v_mad_u64_u32": 2.03, "v_lshrrev_b64": 1.64,
             "v_cvt_scalef32_sr_pk_fp4_f32": 4.74}
# Time one SR decision per element costs on an 8192^2 tensor with no memory
# traffic (the library's SplitMix64 words + two stochastic conversions per element
# pair, in registers; tests/valu_rate_probe.hip): the floor of every stochastic
# quantization of such a tensor.
SR_PAIR_FLOOR_US = 23.4
# steps of the determinism check that runs before the warm-up steps
REPEAT_CHECK_STEPS = 25
QUANT_SOURCES = ("quant.hip", "mx_device.h")
# 256 CUs x 4 SIMDs x 32 lanes per clock (one wave64 instruction every 2 cycles)
# x 2.4 GHz
PEAK_VALU_LANE_OPS = 78.6e12


def weighted_lane_ops(c):
    """Lane-op equivalents per element: VALU lane-ops plus the extra SIMD time of
    the multi-cycle instructions."""
    extra = sum(n / c["elems"] * (VALU_COST[k] - 1.0) for k, n in c["counts"].items())
    return c["lane_ops"] + extra


def code_sha256(paths):
    """sha256 of C++ sources with // comments and blank lines removed, so that
    only code changes (not documentation edits) change it."""
    import hashlib
    import re
    lines = []
    for path in paths:
        for line in open(path, encoding="utf-8").read().splitlines():
            line = re.sub(r"//.*$", "", line).rstrip()
            if line.strip():
                lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def csrc(*names):
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                     "mxfp4_microscaling_quantization_amd", "csrc")
    return [os.path.join(d, n) for n in names]


def gemm_traffic():
    try:
        h = code_sha256(csrc(*GEMM_SOURCES))
    except OSError:
        return None
    return GEMM_TRAFFIC["bytes_per_launch"] if h == GEMM_TRAFFIC["sha256"] else None


def alu_roofline(sweep):
    """ALU roofline of the stochastic-rounding kernels on the 8192^2 sweep:
    weighted lane-op equivalents per element x elements / kernel time against the
    78.6 T lane-op/s VALU peak (`frac`), and the plain VALU issue fraction
    (`issue_frac`, lane-ops only); null when the quantizer code changed since the
    counts were taken."""
    try:
        if code_sha256(csrc(*QUANT_SOURCES)) != QUANT_VALU["sha256"]:
            return None
    except OSError:
        return None
    n = 8192 * 8192
    out = {}
    for key, c in QUANT_VALU["per_elem"].items():
        if key not in sweep:
            continue
        t = sweep[key]["us"] * 1e-6
        w = weighted_lane_ops(c)
        out[key] = {"kernel": c["kernel"], "bound": "alu", "unit": "T lane-op/s",
                    "achieved": round(w * n / t / 1e12, 2), "peak": PEAK_VALU_LANE_OPS / 1e12,
                    "frac": round(w * n / t / PEAK_VALU_LANE_OPS, 4),
                    "issue_frac": round(c["lane_ops"] * n / t / PEAK_VALU_LANE_OPS, 4),
                    "lane_ops_per_elem": c["lane_ops"], "weighted_per_elem": round(w, 2),
                    "sr_floor_us": SR_PAIR_FLOOR_US * c.get("quantizations", 1),
                    "hbm_frac": round(sweep[key]["frac_hbm"], 4)}
    return out


METRIC = "MXFP4 quantize GB/s + MXFP4 linear fwd+bwd TFLOP/s (%roofline), 1 MI355X"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-parts", action="store_true", help="skip the quantizer sweep / MoE rows")
    p.add_argument("--only", default=None, help="run one part only: linear|deit|rht|sweep|moe|deosc")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (known HBM bytes) for counter scaling")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """Per-kernel event pairs recorded on the launch stream; durations read at the end."""

    def __init__(self, torch, stream):
        self.torch, self.stream, self.pairs = torch, stream, {}

    def run(self, name, fn):
        t = self.torch
        a = t.cuda.Event(enable_timing=True)
        b = t.cuda.Event(enable_timing=True)
        a.record(self.stream)
        fn()
        b.record(self.stream)
        self.pairs.setdefault(name, []).append((a, b))

    def mean_ms(self, name):
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs[name]]))

    def count(self, name):
        return len(self.pairs.get(name, []))


def bf16_dev(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def linear_attainable_ms(M, N, K):
    """Attainable time of one linear fwd+bwd with bf16 inputs: the sum over its
    six kernels of max(flops / FP4 peak, algorithmic bytes / HBM peak)."""
    fl = 2.0 * M * N * K
    pk = 0.53125  # packed bytes per element (codes + scales)
    kernels = [  # (flops, algorithmic bytes)
        (0, (M + N) * K * (2 + pk)),                       # quantize X and W
        (fl, (M + N) * K * pk + 4 * M * N),                 # Y = Q(X) Q(W)^T
        (0, M * N * (2 + 2 * pk)),                          # dual quantize dY
        (0, (N + M) * K * 2 * pk),                          # double quantize W and X
        (fl, (M + K) * N * pk + 4 * M * K),                 # dX = Q3 [M,N] . Q4 [K,N]^T
        (fl, (N + K) * M * pk + 4 * N * K),                 # dW = Q5 [N,M] . Q6 [K,M]^T
    ]
    return sum(max(a / (PEAK_FP4_TFLOPS * 1e12), c / (PEAK_HBM_GBPS * 1e9))
               for a, c in kernels) * 1e3


# ---------------------------------------------------------------- linear fwd + bwd (the step)
def bench_linear(torch, mx, synth, dev, steps, warmup, seed=3):
    cfg = synth.llama_config()
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    x = bf16_dev(torch, cfg["x"], dev)
    w = bf16_dev(torch, cfg["w"], dev)
    dy = bf16_dev(torch, cfg["dy"], dev)
    del cfg
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    y, dx, dw = f32(M, N), f32(M, K), f32(N, K)
    xq, wq = (u8(M, K // 2), u8(M, K // 32)), (u8(N, K // 2), u8(N, K // 32))
    q3, q5 = (u8(M, N // 2), u8(M, N // 32)), (u8(N, M // 2), u8(N, M // 32))
    q4, q6 = (u8(K, N // 2), u8(K, N // 32)), (u8(K, M // 2), u8(K, M // 32))
    st = torch.cuda.current_stream()
    T = Timer(torch, st)
    BF = mx.MX_BF16

    def step(timer, timed=("gemm",)):
        """One linear fwd+bwd.  Only the kernels named in `timed` get event pairs
        (timer None: none).  An event record between two kernels keeps the second
        from starting while the first drains its last tiles (~20 us a record), so
        the step's own timed region has none."""
        def run(name, fn):
            (timer.run(name, fn) if timer is not None and name in timed else fn())
        run("quant_xw", lambda: mx.mx_quantize_pair(x, M, w, N, K, BF, mx.MX_RNE, 0, 0, 0, 0,
                                                   *xq, *wq, st))
        run("gemm", lambda: mx.mx_gemm(*xq, *wq, M, N, K, 1.0, y, N, st))
        run("dual_dy", lambda: mx.mx_quantize_dual(dy, BF, M, N, mx.MX_SR, seed + 3, seed + 5,
                                                  *q3, *q5, st))
        run("requant_wx", lambda: mx.mx_requantize_pair(*wq, N, *xq, M, K, mx.MX_SR, seed + 4,
                                                       seed + 6, *q4, *q6, st))
        run("gemm", lambda: mx.mx_gemm(*q3, *q4, M, K, N, 1.0, dx, K, st))
        run("gemm", lambda: mx.mx_gemm(*q5, *q6, N, K, M, 1.0, dw, K, st))

    # the composed step equals the library's own linear entry points, bit for bit
    # (checked first: the host-side comparison idles the GPU, whose clock then
    # needs the warm-up steps to come back up before the timed region)
    step(None)
    y2, xq2, wq2 = mx.linear_fwd(x, w)
    dx2, dw2 = mx.linear_bwd(dy, xq2, wq2, M, N, K, seed)
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in ((y, y2), (dx, dx2), (dw, dw2)))
    del y2, xq2, wq2, dx2, dw2
    # determinism over repeated steps: REPEAT_CHECK_STEPS more steps back to back
    # must reproduce the first step's outputs bit for bit (stochastic rounding is
    # keyed by seed and index, the GEMMs sum in a fixed order).  The device stays
    # busy through this check, so after the host-side setup above its clock has
    # left its idle state before the warm-up steps begin.
    first = [t.clone() for t in (y, dx, dw, *q3, *q4, *q5, *q6)]
    for _ in range(REPEAT_CHECK_STEPS):
        step(None)
    torch.cuda.synchronize()
    repeat_same = all(torch.equal(a, b) for a, b in zip(first, (y, dx, dw, *q3, *q4, *q5, *q6)))
    del first
    torch.cuda.synchronize()
    for _ in range(warmup):
        step(None)

    # the timed region: `steps` steps back to back, events at its two ends only
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(st)
    for _ in range(steps):
        step(None)
    end.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / steps
    flops = 6.0 * M * N * K
    # the GEMM launch duration for the roofline: a second live pass of `steps`
    # steps with an event pair around every GEMM launch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        step(T)
    e1.record(st)
    torch.cuda.synchronize()
    ms_step_events = e0.elapsed_time(e1) / steps
    # per-kernel breakdown of the quantizers: a separate pass with every kernel timed
    B = Timer(torch, st)
    for _ in range(5):
        step(B, timed=("quant_xw", "dual_dy", "requant_wx", "gemm"))
    torch.cuda.synchronize()
    kern = {k: B.mean_ms(k) for k in B.pairs}
    kern["gemm"] = T.mean_ms("gemm")  # the GEMM launches of the second pass
    gemm_ms = kern["gemm"]
    gemm_tf = 2.0 * M * N * K / (gemm_ms * 1e-3) / 1e12
    bytes_q = {
        "quant_xw": (M + N) * K * (2 + 0.53125), "dual_dy": M * N * (2 + 2 * 0.53125),
        "requant_wx": (N + M) * K * 2 * 0.53125,
    }
    quant = {k: {"us": kern[k] * 1e3, "GBps": bytes_q[k] / (kern[k] * 1e-3) / 1e9,
                 "frac_hbm": bytes_q[k] / (kern[k] * 1e-3) / 1e9 / PEAK_HBM_GBPS} for k in bytes_q}
    return {
        "M": M, "N": N, "K": K, "ms_per_step": ms_step, "wall_s": wall,
        "ms_per_step_with_gemm_events": ms_step_events,
        "tflops": flops / (ms_step * 1e-3) / 1e12, "attainable_ms": linear_attainable_ms(M, N, K),
        "frac_attainable": linear_attainable_ms(M, N, K) / ms_step,
        "gemm_ms": gemm_ms, "gemm_tflops": gemm_tf,
        "gemm_launches": T.count("gemm"), "kernels_us": {k: v * 1e3 for k, v in kern.items()},
        "quantizers": quant, "matches_linear_entry_points": bool(same),
        "repeat_steps_identical": bool(repeat_same), "repeat_check_steps": REPEAT_CHECK_STEPS,
    }


# ---------------------------------------------------------------- rotated linear layer
def bench_linear_rht(torch, mx, synth, dev, steps=10, seed=3, mask=0x9E3779B9):
    """The Llama up-projection through the random-sign Hadamard layer
    (mx_linear_fwd_rht + mx_linear_bwd_rht): after 5 untimed layers, the layer
    timed as `steps` fwd+bwd calls back to back (events at the ends only), then
    forward and backward apart with an event pair around each call."""
    cfg = synth.llama_config()
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    x = bf16_dev(torch, cfg["x"], dev)
    w = bf16_dev(torch, cfg["w"], dev)
    dy = bf16_dev(torch, cfg["dy"], dev)
    del cfg
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    y, dx, dw = (torch.empty(s, dtype=torch.float32, device=dev) for s in ((M, N), (M, K), (N, K)))
    xq, wq = (u8(M, K // 2), u8(M, K // 32)), (u8(N, K // 2), u8(N, K // 32))
    ws = u8(mx.mx_linear_bwd_workspace_size(M, N, K))
    st = torch.cuda.current_stream()
    BF = mx.MX_BF16
    fwd = lambda: mx.mx_linear_fwd_rht(x, w, BF, M, N, K, mask, y, *xq, *wq, st)
    bwd = lambda: mx.mx_linear_bwd_rht(dy, BF, M, N, K, *xq, *wq, seed, mask, dx, dw, ws,
                                       ws.numel(), st)
    for _ in range(5):
        fwd()
        bwd()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        fwd()
        bwd()
    e1.record(st)
    torch.cuda.synchronize()
    layer = e0.elapsed_time(e1) / steps
    T = Timer(torch, st)
    for _ in range(steps):
        T.run("fwd", fwd)
        T.run("bwd", bwd)
    torch.cuda.synchronize()
    f, b = T.mean_ms("fwd"), T.mean_ms("bwd")
    fl = 2.0 * M * N * K
    return {"fwd_us": f * 1e3, "bwd_us": b * 1e3, "fwd_bwd_ms": layer,
            "TFLOPs": 3 * fl / (layer * 1e-3) / 1e12, "sign_mask": mask}


# ---------------------------------------------------------------- DeiT-S fc1 layer
def bench_linear_deit(torch, mx, synth, dev, steps=50, seed=1):
    """The DeiT-S MLP fc1 layer (M = 12608 tokens, K = 384, N = 1536) through the
    library's own entry points mx_linear_fwd + mx_linear_bwd.  Its six kernels
    take tens of microseconds each, so eager launches from Python leave the GPU
    idle between them; the layer is also captured once in a HIP graph and
    replayed (every replay checked bit for bit against the eager outputs before
    the timed replays).  The GEMMs are bound by their fp32 output writes
    (K = 384): the attainable time is the sum over the six kernels of
    max(flops / FP4 peak, algorithmic bytes / HBM peak)."""
    cfg = synth.deit_config()
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    x = bf16_dev(torch, cfg["x"], dev)
    w = bf16_dev(torch, cfg["w"], dev)
    dy = bf16_dev(torch, cfg["dy"], dev)
    del cfg
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    y, dx, dw = (torch.empty(s, dtype=torch.float32, device=dev) for s in ((M, N), (M, K), (N, K)))
    xq, wq = (u8(M, K // 2), u8(M, K // 32)), (u8(N, K // 2), u8(N, K // 32))
    ws = u8(mx.mx_linear_bwd_workspace_size(M, N, K))
    BF = mx.MX_BF16

    def layer(st):
        mx.mx_linear_fwd(x, w, BF, M, N, K, y, *xq, *wq, st)
        mx.mx_linear_bwd(dy, BF, M, N, K, *xq, *wq, seed, dx, dw, ws, ws.numel(), st)

    st = torch.cuda.current_stream()
    for _ in range(3):
        layer(st)
    torch.cuda.synchronize()
    want = [t.clone() for t in (y, dx, dw, *xq, *wq)]

    def eager_ms():
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(steps):
            layer(st)
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    eager = eager_ms()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(torch.cuda.current_stream())
    torch.cuda.synchronize()
    replays_equal = True
    for _ in range(3):  # eager fills between replays, every replay checked
        for t in (y, dx, dw, *xq, *wq):
            t.fill_(0x5A if t.dtype == torch.uint8 else float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replays_equal &= all(torch.equal(a, b) for a, b in zip((y, dx, dw, *xq, *wq), want))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(steps):
        g.replay()
    b.record(st)
    torch.cuda.synchronize()
    graph = a.elapsed_time(b) / steps
    del g
    fl = 2.0 * M * N * K
    ideal_ms = linear_attainable_ms(M, N, K)
    return {"M": M, "N": N, "K": K, "eager_ms": eager, "graph_ms": graph,
            "graph_replays_equal_eager": bool(replays_equal),
            "TFLOPs_graph": 3 * fl / (graph * 1e-3) / 1e12,
            "TFLOPs_eager": 3 * fl / (eager * 1e-3) / 1e12, "attainable_ms": ideal_ms,
            "frac_attainable_graph": ideal_ms / graph}


# ---------------------------------------------------------------- quantizer sweep
def bench_sweep(torch, mx, synth, dev, iters=20):
    cfg = synth.sweep_config()
    rows, cols, mask = cfg["rows"], cfg["cols"], cfg["sign_mask"]
    # 4 input buffers (4 x 134 MB > the 256 MB Infinity Cache) used in rotation
    xs = [bf16_dev(torch, cfg["x"], dev) for _ in range(4)]
    del cfg
    n = rows * cols
    st = torch.cuda.current_stream()
    out = {}
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    for axis, an in ((mx.MX_ROW, "row"), (mx.MX_COL, "col")):
        outer, inner = (rows, cols) if axis == mx.MX_ROW else (cols, rows)
        c, s = u8(outer, inner // 2), u8(outer, inner // 32)
        for rnd, rn in ((mx.MX_RNE, "rne"), (mx.MX_SR, "sr")):
            for had in (0, 1):
                T = Timer(torch, st)
                for i in range(iters + 3):
                    fn = lambda: mx.mx_quantize(xs[i % 4], mx.MX_BF16, rows, cols, axis, rnd, 2, had,
                                                mask, c, s, st)
                    (T.run("q", fn) if i >= 3 else fn())
                torch.cuda.synchronize()
                ms = T.mean_ms("q")
                gbps = n * 2.53125 / (ms * 1e-3) / 1e9
                out[f"{an}_{rn}{'_had' if had else ''}"] = {"us": ms * 1e3, "GBps": gbps,
                                                             "frac_hbm": gbps / PEAK_HBM_GBPS}
    # double quantization and the fused dual quantizer on the same tensor
    c, s = mx.quantize(xs[0])
    co, so = u8(cols, rows // 2), u8(cols, rows // 32)
    T = Timer(torch, st)
    for i in range(iters):
        T.run("r", lambda: mx.mx_requantize(c, s, rows, cols, mx.MX_SR, 2, co, so, st))
    cr, sr_ = u8(rows, cols // 2), u8(rows, cols // 32)
    for i in range(iters):
        T.run("d", lambda: mx.mx_quantize_dual(xs[i % 4], mx.MX_BF16, rows, cols, mx.MX_SR, 5, 3,
                                               cr, sr_, co, so, st))
    torch.cuda.synchronize()
    for key, name, bpe in (("r", "requant_sr", 1.0625), ("d", "dual_sr", 3.0625)):
        ms = T.mean_ms(key)
        gbps = n * bpe / (ms * 1e-3) / 1e9
        out[name] = {"us": ms * 1e3, "GBps": gbps, "frac_hbm": gbps / PEAK_HBM_GBPS}
    return out


# ---------------------------------------------------------------- MoE + de-oscillation
def bench_moe(torch, mx, synth, dev, iters=10, deosc_steps=20):
    cfg = synth.moe_config()
    E, H, F, offs = cfg["E"], cfg["hidden"], cfg["ffn"], cfg["offs"]
    w = torch.from_numpy(cfg["w_master"]).to(dev)
    x_up = bf16_dev(torch, cfg["x_up"], dev)
    x_dn = bf16_dev(torch, cfg["x_down"], dev)
    del cfg
    rows, cols = w.shape
    st = torch.cuda.current_stream()
    wq = mx.quantize(w)
    xq_up, xq_dn = mx.quantize(x_up), mx.quantize(x_dn)
    # the forward's operands also with their scale rows padded to 16 bytes
    # (H = 2880: 90 scale bytes per row, 96 apart), the layout a caller picks so
    # that the grouped product loads four K-steps' scales of a row at once
    ld = (H // 32 + 15) // 16 * 16

    def quantize_ld(x):
        c = torch.empty((x.shape[0], H // 2), dtype=torch.uint8, device=dev)
        s_ = torch.empty((x.shape[0], ld), dtype=torch.uint8, device=dev)
        mx.mx_quantize_ld(x, mx.dtype_code(x), x.shape[0], H, mx.MX_ROW, mx.MX_RNE, 0, 0, 0, c, s_,
                          ld, st)
        return c, s_

    wl, xl_up, xl_dn = quantize_ld(w), quantize_ld(x_up), quantize_ld(x_dn)
    c_up = torch.empty((int(offs[-1]), F), dtype=torch.float32, device=dev)
    c_dn = torch.empty((int(offs[-1]), H), dtype=torch.float32, device=dev)
    T = Timer(torch, st)
    runs = {
        "up_packed": lambda: mx.mx_gemm_grouped(*xq_up, wq[0][:E * F], wq[1][:E * F], offs, E, F, H,
                                                1.0, c_up, st),
        "down_packed": lambda: mx.mx_gemm_grouped(*xq_dn, wq[0][E * F:], wq[1][E * F:], offs, E, H,
                                                  H, 1.0, c_dn, st),
        "up": lambda: mx.mx_gemm_grouped_ld(xl_up[0], xl_up[1], ld, wl[0][:E * F], wl[1][:E * F], ld,
                                            offs, E, F, H, 1.0, c_up, st),
        "down": lambda: mx.mx_gemm_grouped_ld(xl_dn[0], xl_dn[1], ld, wl[0][E * F:], wl[1][E * F:],
                                              ld, offs, E, H, H, 1.0, c_dn, st),
    }
    for i in range(iters + 2):
        for key, fn in runs.items():
            (T.run(key, fn) if i >= 2 else fn())
    torch.cuda.synchronize()
    R = int(offs[-1])
    res = {}
    for key in runs:
        n_out = F if key.startswith("up") else H
        ms = T.mean_ms(key)
        res[f"grouped_{key}"] = {"us": ms * 1e3,
                                 "TFLOPs": 2.0 * R * n_out * H / (ms * 1e-3) / 1e12,
                                 "frac_fp4_peak": 2.0 * R * n_out * H / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS}
    del wl, xl_up, xl_dn
    # grouped backward (dX and every expert's dW): dY N(0, 1e-3) bf16 drawn on the
    # device with a fixed seed; 4 R N K flops (dX and dW each 2 R N K)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    for key, xq_g, wq_g, n_out in (("down", xq_dn, (wq[0][E * F:], wq[1][E * F:]), H),
                                   ("up", xq_up, (wq[0][:E * F], wq[1][:E * F]), F)):
        dy = (torch.randn((R, n_out), generator=gen, device=dev) * 1e-3).to(torch.bfloat16)
        dx_g = torch.empty((R, H), dtype=torch.float32, device=dev)
        dw_g = torch.empty((E, n_out, H), dtype=torch.float32, device=dev)
        wsz = mx.mx_grouped_linear_bwd_workspace_size(offs, E, n_out, H)
        ws_g = torch.empty(wsz, dtype=torch.uint8, device=dev)
        run = lambda: mx.mx_grouped_linear_bwd(dy, mx.MX_BF16, offs, E, n_out, H, *xq_g, *wq_g, 4,
                                               dx_g, dw_g, ws_g, wsz, st)
        run()
        T = Timer(torch, st)
        for _ in range(5):
            T.run("b", run)
        torch.cuda.synchronize()
        ms = T.mean_ms("b")
        fl = 4.0 * R * n_out * H
        res[f"grouped_bwd_{key}"] = {"us": ms * 1e3, "TFLOPs": fl / (ms * 1e-3) / 1e12,
                                     "frac_fp4_peak": fl / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS}
        del dy, dx_g, dw_g, ws_g
    del c_up, c_dn, xq_up, xq_dn, x_up, x_dn, wq
    # de-oscillation: 796M fp32 master weights, synthetic optimizer step between passes
    wp, dw_, dq_ = (torch.empty_like(w) for _ in range(3))
    flags = torch.empty(w.shape, dtype=torch.uint8, device=dev)
    mx.mx_deosc_init(w, rows, cols, wp, dw_, dq_, st)
    T = Timer(torch, st)
    for t in range(1, deosc_steps + 1):
        mx.mx_synth_step(w, rows * cols, 4, t, st)
        end = t == deosc_steps
        T.run("end" if end else "step",
              lambda: mx.mx_deosc_step(w, rows, cols, wp, dw_, dq_, end, 4.0, flags, st))
    torch.cuda.synchronize()
    n = rows * cols
    ms = T.mean_ms("step")
    res["deosc_step"] = {"us": ms * 1e3, "GBps": 28.0 * n / (ms * 1e-3) / 1e9,
                         "frac_hbm": 28.0 * n / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    ms_end = T.mean_ms("end")
    res["deosc_window_end"] = {"us": ms_end * 1e3, "GBps": 33.0 * n / (ms_end * 1e-3) / 1e9}
    # the same pass emitting the next forward's Q_D(W) (+0.53125 B/elem), against the
    # two-pass alternative (de-oscillation, then a 4.53125 B/elem weight quantization)
    wc = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    T = Timer(torch, st)
    for t in range(deosc_steps + 1, deosc_steps + 11):
        mx.mx_synth_step(w, rows * cols, 4, t, st)
        T.run("fused", lambda: mx.mx_deosc_step_quantize(w, rows, cols, wp, dw_, dq_, False, 4.0,
                                                         flags, wc, ws, st))
        T.run("quant", lambda: mx.mx_quantize(w, mx.MX_F32, rows, cols, mx.MX_ROW, mx.MX_RNE, 0, 0, 0,
                                              wc, ws, st))
    torch.cuda.synchronize()
    ms_f, ms_q = T.mean_ms("fused"), T.mean_ms("quant")
    res["deosc_step_quantize"] = {"us": ms_f * 1e3, "GBps": 28.53125 * n / (ms_f * 1e-3) / 1e9,
                                  "frac_hbm": 28.53125 * n / (ms_f * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                  "two_pass_us": (ms + ms_q) * 1e3}
    # Q-EMA: read w and the EMA, write the EMA and its Q_D (12.53125 B/elem)
    ema = w.clone()
    T = Timer(torch, st)
    for t in range(10):
        T.run("qema", lambda: mx.mx_qema_step(w, ema, rows, cols, 0.998, wc, ws, st))
    torch.cuda.synchronize()
    ms_e = T.mean_ms("qema")
    res["qema_step"] = {"us": ms_e * 1e3, "GBps": 12.53125 * n / (ms_e * 1e-3) / 1e9,
                        "frac_hbm": 12.53125 * n / (ms_e * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    return res


# ---------------------------------------------------------------- CPU oracle baseline
def cpu_baseline(synth):
    """The oracle's linear fwd + bwd on a bounded slice of the same workload
    (first 2048 tokens, first 4096 output features, full K = 4096).  The GEMM
    oracle (float64 numpy.matmul on the exact dequantized operands) runs on
    every host core BLAS will use; the quantizer oracle is plain single-threaded
    NumPy.  `cores` is the BLAS thread count in the timed region and
    `host_cpu_count` what os.cpu_count() reports."""
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits

    cfg = synth.llama_config()
    Ms, Ns, K = 2048, 4096, cfg["K"]
    x = O.bf16_bits_to_f32(cfg["x"][:Ms])
    w = O.bf16_bits_to_f32(cfg["w"][:Ns])
    dy = O.bf16_bits_to_f32(cfg["dy"][:Ms, :Ns])
    del cfg
    ncpu = os.cpu_count() or 1
    with threadpool_limits(limits=ncpu, user_api="blas"):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
        t0 = time.perf_counter()
        _, xq, wq = O.linear_fwd(x, w)
        O.linear_bwd(dy, xq, wq, Ms, Ns, K, 3)
        dt = time.perf_counter() - t0
    flops = 6.0 * Ms * Ns * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "host_cpu_count": ncpu, "kind": "oracle", "seconds": dt,
            "sample": f"linear fwd+bwd on X[:{Ms}], W[:{Ns}], dY[:{Ms},:{Ns}] (K={K}) of the "
                      f"Llama up-projection workload; GEMM oracle float64 numpy.matmul on "
                      f"{int(threads)} BLAS threads, quantizer oracle single-threaded NumPy"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU: this build has no multi-GPU path "
              "(the sharding plan is described in the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch

    from mxfp4_microscaling_quantization_amd import mx, synth

    mx.lib()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 28  # 2^28 float32 = 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": 4 * n, "copies": 3}))
        return
    parts = {}
    lin = None
    if args.only in (None, "linear"):
        log("linear fwd+bwd (Llama-3-8B up-projection)")
        lin = bench_linear(torch, mx, synth, dev, args.steps, args.warmup)
        torch.cuda.empty_cache()
    if not args.no_parts and args.only in (None, "deit"):
        log("DeiT-S fc1 linear fwd+bwd")
        parts["linear_deit_s_fc1"] = bench_linear_deit(torch, mx, synth, dev)
        torch.cuda.empty_cache()
    if not args.no_parts and args.only in (None, "rht"):
        log("rotated linear fwd+bwd (Llama-3-8B up-projection)")
        parts["linear_rht_llama_up_proj"] = bench_linear_rht(torch, mx, synth, dev)
        torch.cuda.empty_cache()
    if not args.no_parts and args.only in (None, "sweep"):
        log("quantizer sweep 8192x8192 bf16")
        parts["quantizer_sweep_8192sq_bf16"] = bench_sweep(torch, mx, synth, dev)
        torch.cuda.empty_cache()
    if not args.no_parts and args.only in (None, "moe", "deosc"):
        log("MoE grouped GEMM + de-oscillation")
        parts["moe_32x2880"] = bench_moe(torch, mx, synth, dev)
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline and args.only in (None, "linear"):
        log("CPU oracle baseline")
        cpu = cpu_baseline(synth)
    if lin is None:
        print(json.dumps({"parts": parts}))
        return
    parts["linear_kernels"] = {"kernels_us": lin["kernels_us"], "quantizers": lin["quantizers"],
                               "gemm_launches_timed": lin["gemm_launches"],
                               "step_attainable_ms": lin["attainable_ms"],
                               "step_frac_attainable": lin["frac_attainable"],
                               "ms_per_step_with_gemm_events": lin["ms_per_step_with_gemm_events"],
                               "matches_linear_entry_points": lin["matches_linear_entry_points"],
                               "repeat_steps_identical": lin["repeat_steps_identical"],
                               "repeat_check_steps": lin["repeat_check_steps"]}
    ach = lin["gemm_tflops"]
    line = {
        "metric": METRIC,
        "value": round(lin["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(lin["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "llama3-8b-mlp-up-proj-linear-fwd-bwd", "M": lin["M"],
                   "N": lin["N"], "K": lin["K"], "input_dtype": "bf16",
                   "parallelism": "single-gpu"},
        "roofline": {"kernel": "k_gemm_pp (MXFP4 GEMM, 256x256 tiles, 2MNK per launch)",
                     "bound": "mfma",
                     "achieved": round(ach, 2), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_FP4_TFLOPS, 4), "traffic": gemm_traffic()},
        "cpu_baseline": cpu,
        "quantize_GBps": {k: round(v["GBps"], 1) for k, v in
                          parts.get("quantizer_sweep_8192sq_bf16", {}).items()},
        "alu_roofline": alu_roofline(parts.get("quantizer_sweep_8192sq_bf16", {})),
        "parts": parts,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
