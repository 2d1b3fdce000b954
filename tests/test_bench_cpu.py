"""Host-side checks of bench.py's contract (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, timeout=300)


@pytest.mark.parametrize("n", ["2", "8"])
def test_bench_refuses_more_than_one_gpu(n):
    r = _run("--gpus", n)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_modes_are_listed():
    r = _run("--help")
    assert r.returncode == 0
    for mode in ("throughput", "latency", "materialize", "vjp"):
        assert mode in r.stdout


def test_committed_traffic_records_name_their_kernel_and_command():
    # Each counter record carries the kernel it measured, the command that made
    # it and a source hash; bench.py reports its bytes only while the hash
    # matches the current sources of that kernel.
    prof = os.path.join(ROOT, "profiles")
    recs = [f for f in os.listdir(prof) if f.startswith("traffic_") and f.endswith(".json")]
    assert recs
    for f in recs:
        rec = json.load(open(os.path.join(prof, f)))
        for key in ("kernel", "kernel_hash", "command", "bytes_per_launch", "scale_read", "scale_write"):
            assert key in rec, (f, key)
        assert rec["bytes_per_launch"] > 0
