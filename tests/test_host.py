"""CPU: host-side behaviour of the product path and the benchmark.

* the product package never imports or loads the oracle (it is test
  infrastructure), and the HIP sources include nothing of it;
* a missing library fails loudly (no CPU fallback);
* bench.py refuses more than one GPU with a message and exit status 2.
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
