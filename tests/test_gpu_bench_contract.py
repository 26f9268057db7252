"""bench.py prints one JSON line with the fields its consumers read.

Runs the benchmark on the small workload in a child process (a few seconds)
and checks the line: metric and unit, n_gpus 1, the step counts asked for,
a positive value consistent with ms_per_step, the roofline object of the
attention kernel and the CPU-baseline object. ``--gpus 2`` must refuse.
"""

import json
import os
import subprocess
import sys

import pytest

from _parity import note

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=240)
    return r.returncode, r.stdout.strip().splitlines()


def test_bench_json_line():
    note("bench.py contract (tiny workload)")
    rc, lines = run_bench("--workload", "tiny", "--steps", "3", "--warmup", "1", "--cpu-budget", "1")
    assert rc == 0, lines
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    assert d["metric"].startswith("STA fwd ms/call + effective TFLOP/s")
    assert d["unit"] == "TFLOP/s" and d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "tiny" and d["vs_baseline"] is None
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - d["effective_flop_per_call"] / (d["ms_per_step"] * 1e-3) / 1e12) \
        <= 1e-6 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] > 2500
    assert 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert "traffic" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]


def test_bench_refuses_more_gpus():
    note("bench.py --gpus 2")
    rc, lines = run_bench("--gpus", "2")
    assert rc != 0
    assert "one GPU" in lines[-1]
