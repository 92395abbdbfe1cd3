"""GPU: the routing path driven from plain C, with no Python in the process.

tests/c/gpu_path.c allocates device memory with the HIP runtime, calls
peg_route_prep, peg_gather_binned / peg_gather_padded, peg_scatter_combine
and peg_wgrad through include/peg.h, and compares every output with the C
oracle on the same seeded batch (index outputs and the gathered tensor bit
for bit, the combine and wgrad within the tolerance of tests/gpu_util.py).
The binary is built by __graft_entry__.build().
"""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "gpu_path")


def test_c_driver_matches_oracle():
    assert os.access(EXE, os.X_OK), "tests/c/gpu_path is not built (run __graft_entry__.build())"
    print("[c driver] tests/c/gpu_path: binned, padded, padded-tiled", flush=True)
    out = subprocess.run([EXE], capture_output=True, text=True, timeout=100)
    print(out.stdout, out.stderr, flush=True)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "gpu_path ok"
