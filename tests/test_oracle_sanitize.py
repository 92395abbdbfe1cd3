"""CPU: the oracle's C source, built with the address and undefined-behaviour
sanitizers into a small C driver, runs every oracle function on small inputs
(empty, one token, ragged) without a sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    flags = ["-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]
    subprocess.run(["gcc", *flags, "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "peg_oracle.c"),
                    os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"), "-o", str(exe), "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert out.returncode == 0, out.stderr[-4000:]
    assert "oracle sanitize ok" in out.stdout
