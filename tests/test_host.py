"""CPU: host-side behaviour of the product path and the benchmark.

* the product package never imports or loads the oracle (it is test
  infrastructure), and the HIP sources include nothing of it;
* a missing library fails loudly (no CPU fallback);
* bench.py refuses more than one GPU with a message and exit status 2;
* its one-thread and all-cores CPU-oracle legs report whole steps.
"""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "padded_expert_gather_amd")


def _sources():
    for d, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                yield os.path.join(d, f)


def test_product_path_does_not_use_the_oracle():
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle|#include\s+\"[^\"]*oracle)|libpeg_oracle|pego_", re.M)
    for path in _sources():
        with open(path) as f:
            text = f.read()
        assert not pat.search(text), f"{path} refers to the oracle"


def test_missing_library_raises():
    code = ("import padded_expert_gather_amd as peg\n"
            "try:\n"
            "    peg.library()\n"
            "except OSError:\n"
            "    print('raised')\n")
    env = dict(os.environ, PEG_LIBRARY="/nonexistent/libpeg.so")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert out.stdout.strip() == "raised", out.stdout + out.stderr


def test_bench_refuses_several_gpus():
    out = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 2
    assert "one GPU" in out.stderr


def test_bench_cpu_oracle_legs():
    """The one-thread and multi-thread oracle legs of bench.py on the
    512-token batch: both report whole steps, the threaded one with its thread
    count, and both the host's CPU count, the CPUs allowed and the model."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W
    wl = W.config(1, 0)
    one = bench.cpu_baseline(wl, W, 0.2, 1000)
    two = bench.cpu_baseline_threads(wl, W, 0.2, 1000, 2)
    for leg, cores in ((one, 1), (two, 2)):
        assert leg["kind"] == "oracle" and leg["unit"] == "GB/s"
        assert leg["cores"] == cores and leg["value"] > 0
        assert leg["host_cpus"] >= 1 and 1 <= leg["allowed_cpus"] <= leg["host_cpus"]
        assert "cpu_model" in leg
    assert "16" in two["thread_cap"]
    assert 1 <= bench.cpu_threads() <= 16
