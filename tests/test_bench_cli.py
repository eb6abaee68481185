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
    assert a.gpus == 1 and 1 <= a.steps <= 50 and 0 <= a.warmup <= 10
