"""Sustained rate of the block-scaled FP4 MFMA with register operands
(tests/mfma_rate_probe.hip): the ceiling of the MXFP4 GEMM on this chip under
the data it multiplies.  The checks are sanity bounds: no mode beats the nominal
10.1 PFLOP/s, the clocks are plausible, and random operands, which toggle the
multipliers, never run faster than all-zero ones."""
import json
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "_build", "mfma_rate_probe")

pytestmark = pytest.mark.gpu


def test_mfma_rate_probe_modes():
    if not os.path.exists(PROBE):
        pytest.skip("mfma_rate_probe not built (build() compiles it)")
    print("mfma rates: probe", flush=True)
    res = subprocess.run([PROBE], capture_output=True, text=True, timeout=90)
    assert res.returncode == 0, res.stderr
    rows = [json.loads(line) for line in res.stdout.splitlines() if line.startswith("{")]
    head = rows[0]
    assert head["arch"].startswith("gfx950") and head["cus"] == 256, head
    modes = {r["mode"]: r for r in rows[1:]}
    assert set(modes) == {"zero", "fixed", "rotating", "rotating_scales"}
    for name, r in modes.items():
        print(name, r)
        assert 0 < r["tflops"] <= 10100 * 1.02, r
        assert 0.5 < r["clock_ghz"] < 2.6, r
    assert modes["rotating"]["tflops"] <= modes["zero"]["tflops"] * 1.02
