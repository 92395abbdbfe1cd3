"""GPU: bench.py's output line, from a short run on the 512-token binned f32
batch (the small workload, so the run takes seconds).

The line must be one JSON object with the metric, a positive throughput on one
GPU, the workload named in ``config``, and a ``roofline`` object whose
fraction is its achieved rate over MI355X's 8 TB/s, per-kernel durations in
the back-to-back steps and with the caches flushed, torch's streaming rates,
and the combine backward outside the step; the CPU legs are skipped here
(tests/test_host.py covers them on the CPU).
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line():
    cmd = [sys.executable, "bench.py", "--workload", "1", "--steps", "20", "--warmup", "3", "--no-cpu"]
    print("[bench line] " + " ".join(cmd[1:]), flush=True)
    out = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=100)
    print(out.stderr[-2000:], flush=True)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [ln for ln in out.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, out.stdout
    rec = json.loads(lines[0])
    assert rec["n_gpus"] == 1 and rec["steps"] == 20 and rec["warmup"] == 3
    assert rec["unit"] == "GB/s" and rec["value"] > 0 and rec["higher_is_better"] is True
    assert rec["dtype"] == "f32" and rec["data"] == "synthetic"
    assert rec["config"]["workload"] == "binned-f32-T512-H250-E8-K2-C128"
    assert rec["ms_per_step"] > 0
    roof = rec["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert rec["cpu_baseline"] is None and rec["cpu_baseline_threads"] is None
    for op in ("route_prep", "gather", "combine", "wgrad"):
        assert rec["kernels"][op]["avg_us"] > 0, op
        assert rec["kernels_flushed"][op]["avg_us"] > 0, op
    assert rec["flush_bytes"] >= 1 << 30
    # torch's own streaming kernels as reference rates, and the out-of-step
    # calls timed back to back and cache-flushed
    assert set(rec["streaming_GBps"]) == {"copy", "write", "read", "add"}
    assert all(v > 0 for v in rec["streaming_GBps"].values())
    cb = rec["outside_step"]["combine_backward"]
    assert cb["avg_us"] > 0 and cb["avg_us_flushed"] > 0 and cb["bytes"] > 0
