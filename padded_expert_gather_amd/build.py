"""Build ``libpeg.so`` (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into ``padded_expert_gather_amd/libpeg.so``. Symbols are hidden except the
``peg_*`` entry points that ``include/peg.h`` declares.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpeg.so")

ARCH = os.environ.get("PEG_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # packed fp32 instructions stay off (plain float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src, objdir, extra):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False, extra_flags=(), out=LIB):
    """Compile every HIP source (always) and link the library (default
    libpeg.so). ``extra_flags`` may set the tuning macros (-DPEG_...) for a
    variant build written to ``out``. Returns the library path."""
    objdir = OBJDIR if out == LIB else out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir, list(extra_flags)), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(out)
    return out


def is_stale():
    """True if libpeg.so is missing or older than a source or header."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + glob.glob(os.path.join(CSRC, "*.hpp")) + [os.path.join(INCLUDE, "peg.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    build(verbose=True)
