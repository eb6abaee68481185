"""CPU checks of bench.py's command line: the multi-GPU refusal happens before
anything touches a GPU, and the defaults match the one-GPU contract."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line for a run that did not happen


def test_defaults_are_one_gpu_and_a_short_run():
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse()
    finally:
        sys.argv = old
    assert a.gpus == 1 and 1 <= a.steps <= 50 and 0 <= a.warmup <= 50


def test_attainable_time_of_the_deit_layer():
    """Sum over the six kernels of max(flops / 10.1 PFLOP/s, bytes / 8 TB/s), written out
    for M, N, K = 12608, 1536, 384 (every kernel is bandwidth-bound at this shape)."""
    sys.path.insert(0, ROOT)
    import bench
    M, N, K = 12608, 1536, 384
    pk = 17 / 32  # packed bytes per element: half a code byte + 1/32 scale byte
    bytes_ = [(M + N) * K * (2 + pk),            # quantize X and W
              (M + N) * K * pk + 4 * M * N,      # Y
              M * N * (2 + 2 * pk),              # dual quantization of dY
              (N + M) * K * 2 * pk,              # double quantization of W and X
              (M + K) * N * pk + 4 * M * K,      # dX = Q3 [M, N] . Q4 [K, N]^T
              (N + K) * M * pk + 4 * N * K]      # dW = Q5 [N, M] . Q6 [K, M]^T
    flops = 2.0 * M * N * K
    for b, f in zip(bytes_, [0, flops, 0, 0, flops, flops]):
        assert b / 8e12 >= f / 10.1e15      # bandwidth-bound
    want_ms = sum(bytes_) / 8e12 * 1e3
    assert abs(bench.linear_attainable_ms(M, N, K) - want_ms) < 1e-12


def test_code_hash_ignores_comments_only(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f() {\n  return 1;  // one\n}\n")
    b.write_text("// header\n\nint f() {\n  return 1;\n}\n\n")
    c.write_text("int f() {\n  return 2;\n}\n")
    assert bench.code_sha256([a]) == bench.code_sha256([b])
    assert bench.code_sha256([a]) != bench.code_sha256([c])
    assert bench.code_sha256([a, c]) != bench.code_sha256([c, a])


def test_alu_roofline_weights_multi_cycle_instructions():
    """Weighted lane-op equivalents per element are the VALU lane-ops plus, for
    each multi-cycle instruction, its count per element times its extra cost;
    the figure is withheld when the quantizer code no longer matches the counted
    one."""
    sys.path.insert(0, ROOT)
    import bench
    c = {"lane_ops": 10.0, "elems": 32, "counts": {"v_mul_lo_u32": 64, "v_cvt_scalef32_sr_pk_fp4_f32": 16}}
    want = 10.0 + 2 * (bench.VALU_COST["v_mul_lo_u32"] - 1) + 0.5 * (
        bench.VALU_COST["v_cvt_scalef32_sr_pk_fp4_f32"] - 1)
    assert abs(bench.weighted_lane_ops(c) - want) < 1e-12
    sweep = {k: {"us": 100.0, "frac_hbm": 0.5} for k in bench.QUANT_VALU["per_elem"]}
    got = bench.alu_roofline(sweep)
    if bench.code_sha256(bench.csrc(*bench.QUANT_SOURCES)) != bench.QUANT_VALU["sha256"]:
        assert got is None
        return
    for k, c in bench.QUANT_VALU["per_elem"].items():
        w = bench.weighted_lane_ops(c) * 8192 * 8192 / 100e-6
        assert abs(got[k]["achieved"] - w / 1e12) < 0.01
        assert abs(got[k]["frac"] - w / 78.6e12) < 1e-4
        assert got[k]["issue_frac"] < got[k]["frac"]
