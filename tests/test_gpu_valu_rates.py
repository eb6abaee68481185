"""VALU issue rates on the GPU against what the ALU roofline assumes: simple
32-bit operations issue one wave64 instruction per SIMD every 2 cycles (256 CUs
x 4 SIMDs x 32 lanes x 2.4 GHz = 78.6 T lane-op/s), and the multi-cycle
instructions of the stochastic quantizers cost the multiples bench.py weights
them by."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "_build", "valu_rate_probe")

pytestmark = pytest.mark.gpu


def probe_rows():
    if not os.path.exists(PROBE):
        pytest.skip("valu_rate_probe not built (build() compiles it)")
    print("valu rates: probe", flush=True)
    res = subprocess.run([PROBE], capture_output=True, text=True, timeout=90)
    assert res.returncode == 0, res.stderr
    rows = [json.loads(line) for line in res.stdout.splitlines() if line.startswith("{")]
    head = rows[0]
    rates = {(r["instr"], r["waves_per_simd"]): r for r in rows[1:] if "instr" in r}
    seqs = {r["sequence"]: r for r in rows[1:] if "sequence" in r}
    return head, rates, seqs


def test_simple_ops_issue_every_two_cycles_and_weights_match():
    sys.path.insert(0, ROOT)
    import bench
    head, rates, seqs = probe_rows()
    assert head["arch"].startswith("gfx950") and head["cus"] == 256, head
    simple = rates[("v_add_u32", 4)]["cycles_per_instr"]
    for name in ("v_add_u32", "v_xor_b32"):
        cpi = rates[(name, 4)]["cycles_per_instr"]
        assert 1.8 <= cpi <= 2.3, (name, cpi)
    for name, cost in bench.VALU_COST.items():
        got = rates[(name, 4)]["cycles_per_instr"] / simple
        assert abs(got - cost) <= 0.2 * cost, (name, got, cost)


def test_sr_pair_sequence_costs_more_than_its_parts_alone():
    """The stochastic-rounding pair (SplitMix64 words, two conversions, merge) runs
    slower than either part alone, and the figure bench.py quotes as the SR floor
    of an 8192^2 tensor is within 25 % of the measured one."""
    sys.path.insert(0, ROOT)
    import bench
    _, _, seqs = probe_rows()
    pair = seqs["sr_pair"]["us_per_8192sq_elements"]
    assert pair > seqs["splitmix64_words"]["us_per_8192sq_elements"]
    assert pair > seqs["cvt_sr_pair"]["us_per_8192sq_elements"]
    assert abs(pair - bench.SR_PAIR_FLOOR_US) <= 0.25 * bench.SR_PAIR_FLOOR_US, pair
