"""CPU: the C-ABI library loads, exports every entry point of include/peg.h,
and its host-side argument checks return the documented status codes.

No call here passes its argument checks, so no kernel is launched and no GPU
is needed (every case fails before the first HIP call).
"""
import ctypes
import os
import re

import pytest

import padded_expert_gather_amd as peg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "peg.h")

OK, NULL_ARG, BAD_SHAPE, BAD_DTYPE, WORKSPACE, LAUNCH, ALIGNMENT, SCRATCH_LIMIT = 0, 1, 2, 3, 4, 5, 6, 7


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(peg_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return peg.library()


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert len(names) == 17
    for name in names:
        assert hasattr(lib, name), name


def test_version_status_and_workspace(lib):
    assert lib.peg_abi_version() >> 16 == 1
    for s in range(8):
        assert lib.peg_status_string(s) != b"unknown status"
    assert lib.peg_status_string(99) == b"unknown status"
    assert lib.peg_workspace_bytes(-1, 2, 8) == 0
    assert lib.peg_workspace_bytes(10, 0, 8) == 0
    assert lib.peg_workspace_bytes(10, 2, 2000) == 0
    # route_prep tiles of 1024 ids at E <= 512: 65536 ids -> 64 tiles * 256 experts * 4 B
    assert lib.peg_workspace_bytes(8192, 8, 256) >= 64 * 256 * 4
    # slot-row rebuild needs T*K int32
    assert lib.peg_workspace_bytes(4096, 2, 8) >= 4096 * 2 * 4
    assert lib.peg_workspace_bytes(0, 1, 1) == 256


def _p(v):
    return ctypes.c_void_p(v)


FAKE = 0x10000  # never dereferenced: every call below fails its host checks first


def test_route_prep_checks(lib):
    f = lib.peg_route_prep
    base = dict(top=_p(FAKE), T=4, K=2, E=4, layout=0, C=2, m=0, idx=_p(FAKE), bid=_p(FAKE), tpe=None,
                bins=_p(FAKE), pb=None, sr=None, ws=_p(FAKE), wsb=1 << 20, s=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["top"], a["T"], a["K"], a["E"], a["layout"], a["C"], a["m"], a["idx"], a["bid"], a["tpe"],
                 a["bins"], a["pb"], a["sr"], a["ws"], a["wsb"], a["s"])

    assert call(layout=7) == BAD_DTYPE
    assert call(T=-1) == BAD_SHAPE
    assert call(K=0) == BAD_SHAPE
    assert call(E=0) == BAD_SHAPE
    assert call(E=1025) == BAD_SHAPE
    assert call(T=1 << 30, K=4) == BAD_SHAPE          # T*K >= 2^31
    assert call(C=0) == BAD_SHAPE                      # binned needs capacity >= 1
    assert call(layout=1, pb=_p(FAKE), m=0) == BAD_SHAPE  # padded needs m >= 1
    assert call(top=None) == NULL_ARG
    assert call(bins=None) == NULL_ARG
    assert call(idx=None) == NULL_ARG
    assert call(layout=1, m=4, pb=None) == NULL_ARG    # padded layout needs padded_bins
    assert call(ws=None) == WORKSPACE
    assert call(wsb=8) == WORKSPACE


def test_route_prep_noalloc_checks(lib):
    """The allocation-free routing preparation: the checks of route_prep, and
    sizes past its static scratch refused before any HIP call."""
    f = lib.peg_route_prep_noalloc
    base = dict(top=_p(FAKE), T=4, K=2, E=4, layout=0, C=2, m=0, idx=_p(FAKE), bid=_p(FAKE), tpe=None,
                bins=_p(FAKE), pb=None, sr=None, s=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["top"], a["T"], a["K"], a["E"], a["layout"], a["C"], a["m"], a["idx"], a["bid"], a["tpe"],
                 a["bins"], a["pb"], a["sr"], a["s"])

    assert call(layout=7) == BAD_DTYPE
    assert call(T=-1) == BAD_SHAPE
    assert call(E=1025) == BAD_SHAPE
    assert call(C=0) == BAD_SHAPE
    assert call(top=None) == NULL_ARG
    assert call(layout=1, m=4, pb=None) == NULL_ARG
    # E = 1024 tiles hold 512 assignments: 131,073 of them need 257 tiles of
    # 1024 counts (1,052,672 bytes), past the 1 MiB scratch
    assert call(T=131073, K=1, E=1024, C=200) == SCRATCH_LIMIT
    assert call(T=(1 << 19) + 128, K=8, E=64, C=200) == SCRATCH_LIMIT  # 4097 tiles of 1024 x 64 counts


def test_gather_checks(lib):
    g = lib.peg_gather_binned

    def binned(x=_p(FAKE), dt=1, T=4, H=8, K=2, E=4, C=2, idx=_p(FAKE), bid=_p(FAKE), bins=_p(FAKE), sr=_p(FAKE),
               out=_p(FAKE), ws=_p(FAKE), wsb=1 << 20):
        return g(x, dt, T, H, K, E, C, idx, bid, bins, sr, out, ws, wsb, None)

    assert binned(dt=5) == BAD_DTYPE
    assert binned(H=0) == BAD_SHAPE
    assert binned(C=0) == BAD_SHAPE
    assert binned(E=2000) == BAD_SHAPE
    assert binned(x=None) == NULL_ARG
    assert binned(out=None) == NULL_ARG
    assert binned(bins=None) == NULL_ARG
    assert binned(sr=None, idx=None) == NULL_ARG          # rebuild needs the sorted arrays
    assert binned(x=_p(FAKE + 1)) == ALIGNMENT             # bf16 rows need 2-byte alignment
    assert binned(dt=0, out=_p(FAKE + 2)) == ALIGNMENT     # f32 rows need 4-byte alignment
    assert binned(sr=None, ws=None) == WORKSPACE
    assert binned(sr=None, wsb=4) == WORKSPACE

    p = lib.peg_gather_padded

    def padded(pb=_p(FAKE), out_rows=16, sr=_p(FAKE)):
        return p(_p(FAKE), 1, 4, 8, 2, 4, _p(FAKE), _p(FAKE), _p(FAKE), pb, sr, _p(FAKE), out_rows, None, _p(FAKE),
                 1 << 20, None)

    assert padded(pb=None) == NULL_ARG
    assert padded(out_rows=-1) == BAD_SHAPE


def test_combine_wgrad_checks(lib):
    c = lib.peg_scatter_combine

    def comb(y=_p(FAKE), dt=1, layout=0, T=4, H=8, K=2, E=4, C=2, pb=None, sr=_p(FAKE), w=None, out=_p(FAKE)):
        return c(y, dt, layout, T, H, K, E, C, _p(FAKE), _p(FAKE), _p(FAKE), pb, sr, w, out, _p(FAKE), 1 << 20, None)

    assert comb(dt=3) == BAD_DTYPE
    assert comb(layout=2) == BAD_DTYPE
    assert comb(C=0) == BAD_SHAPE
    assert comb(layout=1, pb=None) == NULL_ARG
    assert comb(y=None) == NULL_ARG
    assert comb(out=None) == NULL_ARG
    assert comb(w=_p(FAKE + 2)) == ALIGNMENT

    wg = lib.peg_wgrad

    def wgr(y=_p(FAKE), g=_p(FAKE), dt=1, T=4, H=8, out=_p(FAKE)):
        return wg(y, g, dt, 0, T, H, 2, 4, 2, _p(FAKE), _p(FAKE), _p(FAKE), None, _p(FAKE), out, _p(FAKE), 1 << 20,
                  None)

    assert wgr(g=None) == NULL_ARG
    assert wgr(out=None) == NULL_ARG
    assert wgr(H=-3) == BAD_SHAPE
    assert wgr(g=_p(FAKE + 1)) == ALIGNMENT


def test_router_topk_checks(lib):
    f = lib.peg_router_topk

    def call(lg=_p(FAKE), dt=0, T=4, E=8, K=2, gating=0, norm=1, top=_p(FAKE), w=_p(FAKE)):
        return f(lg, dt, T, E, K, gating, norm, top, w, None)

    assert call(dt=7) == BAD_DTYPE
    assert call(gating=2) == BAD_DTYPE
    assert call(T=-1) == BAD_SHAPE
    assert call(E=0) == BAD_SHAPE
    assert call(E=1025, K=2) == BAD_SHAPE
    assert call(K=0) == BAD_SHAPE
    assert call(K=9) == BAD_SHAPE                      # K > E
    assert call(T=1 << 28, E=16) == BAD_SHAPE          # T*E >= 2^31
    assert call(lg=None) == NULL_ARG
    assert call(top=None) == NULL_ARG
    assert call(w=None) == NULL_ARG
    assert call(lg=_p(FAKE + 2)) == ALIGNMENT          # f32 scores need 4-byte alignment
    assert call(dt=1, lg=_p(FAKE + 1)) == ALIGNMENT
    assert call(w=_p(FAKE + 2)) == ALIGNMENT
    assert call(T=0, lg=None, top=None, w=None) == OK   # nothing to do, nothing enqueued


def test_route_prep_logits_checks(lib):
    f = lib.peg_route_prep_logits

    def call(lg=_p(FAKE), dt=0, T=4, E=8, K=2, gating=0, layout=0, C=2, m=0, top=_p(FAKE), w=_p(FAKE),
             idx=_p(FAKE), bins=_p(FAKE), pb=None, ws=_p(FAKE), wsb=1 << 20):
        return f(lg, dt, T, E, K, gating, 1, layout, C, m, top, w, idx, _p(FAKE), None, bins, pb, None, ws, wsb,
                 None)

    assert call(dt=5) == BAD_DTYPE
    assert call(gating=3) == BAD_DTYPE
    assert call(layout=4) == BAD_DTYPE
    assert call(K=9) == BAD_SHAPE
    assert call(C=0) == BAD_SHAPE                      # binned needs capacity >= 1
    assert call(layout=1, pb=_p(FAKE), m=0) == BAD_SHAPE
    assert call(layout=1, m=4, pb=None) == NULL_ARG
    assert call(idx=None) == NULL_ARG
    assert call(bins=None) == NULL_ARG
    assert call(top=None) == NULL_ARG
    assert call(ws=None) == WORKSPACE
    assert call(wsb=8) == WORKSPACE
    assert call(w=_p(FAKE + 1)) == ALIGNMENT


def test_windows_and_gather_rows_checks(lib):
    f = lib.peg_route_prep_windows

    def win(T=4, K=2, E=4, base=_p(FAKE), limit=_p(FAKE), idx=_p(FAKE), bins=_p(FAKE), sr=_p(FAKE), ws=_p(FAKE),
            wsb=1 << 20):
        return f(_p(FAKE), T, K, E, base, limit, idx, _p(FAKE), None, bins, sr, ws, wsb, None)

    assert win(E=0) == BAD_SHAPE
    assert win(K=0) == BAD_SHAPE
    assert win(base=None) == NULL_ARG
    assert win(limit=None) == NULL_ARG
    assert win(sr=None) == NULL_ARG
    assert win(bins=None) == NULL_ARG
    assert win(ws=None) == WORKSPACE
    assert win(wsb=16) == WORKSPACE
    g = lib.peg_gather_rows

    def gr(x=_p(FAKE), dt=1, T=4, H=8, K=2, sr=_p(FAKE), out=_p(FAKE), rows=16):
        return g(x, dt, T, H, K, sr, out, rows, None, None)

    assert gr(dt=4) == BAD_DTYPE
    assert gr(H=0) == BAD_SHAPE
    assert gr(rows=-1) == BAD_SHAPE
    assert gr(sr=None) == NULL_ARG
    assert gr(x=_p(FAKE + 1)) == ALIGNMENT
    assert gr(T=0, x=None, sr=None) == OK


def test_compaction_and_validate_checks(lib):
    f = lib.peg_routing_map_compact
    assert f(_p(FAKE), 9, _p(FAKE), 4, 8, 2, _p(FAKE), _p(FAKE), None) == BAD_DTYPE
    assert f(_p(FAKE), 0, _p(FAKE), 4, 8, 9, _p(FAKE), _p(FAKE), None) == BAD_SHAPE   # topk > E
    assert f(_p(FAKE), 0, _p(FAKE), 4, 8, 0, _p(FAKE), _p(FAKE), None) == BAD_SHAPE
    assert f(None, 0, _p(FAKE), 4, 8, 2, _p(FAKE), _p(FAKE), None) == NULL_ARG
    b = lib.peg_routing_map_compact_backward
    assert b(_p(FAKE), _p(FAKE), 4, 0, 2, _p(FAKE), None) == BAD_SHAPE
    assert b(None, _p(FAKE), 4, 8, 2, _p(FAKE), None) == NULL_ARG
    v = lib.peg_validate_routing
    assert v(_p(FAKE), _p(FAKE), _p(FAKE), None, 4, 2, 4, 9, _p(FAKE), _p(FAKE), 1 << 20, None) == BAD_SHAPE
    assert v(_p(FAKE), _p(FAKE), None, None, 4, 2, 4, -1, _p(FAKE), _p(FAKE), 1 << 20, None) == NULL_ARG
    assert v(_p(FAKE), _p(FAKE), _p(FAKE), None, 4, 2, 4, -1, _p(FAKE), None, 0, None) == WORKSPACE


def test_oversized_launches_refused(lib):
    """A launch past 2^32 - 1 threads (a HIP dispatch counts threads in 32
    bits) is refused with BAD_SHAPE before anything is enqueued."""
    g = lib.peg_gather_rows
    assert g(_p(FAKE), 1, 40_000_000, 8, 1, _p(FAKE), _p(FAKE), 16, None, None) == BAD_SHAPE
    b = lib.peg_gather_binned
    assert b(_p(FAKE), 1, 40_000_000, 8, 1, 4, 2, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), 1 << 20,
             None) == BAD_SHAPE
    c = lib.peg_scatter_combine
    assert c(_p(FAKE), 1, 0, 20_000_000, 8, 1, 4, 2, _p(FAKE), _p(FAKE), _p(FAKE), None, _p(FAKE), None, _p(FAKE),
             _p(FAKE), 1 << 20, None) == BAD_SHAPE
    w = lib.peg_wgrad
    assert w(_p(FAKE), _p(FAKE), 1, 0, 80_000_000, 8, 2, 4, 2, _p(FAKE), _p(FAKE), _p(FAKE), None, _p(FAKE),
             _p(FAKE), _p(FAKE), 1 << 20, None) == BAD_SHAPE
    cb = lib.peg_combine_backward  # K = 2 (one pass) and K = 4 (dy gather, then wgrad)
    for K in (2, 4):
        assert cb(_p(FAKE), _p(FAKE), None, 1, 0, 80_000_000 // K * 2, 8, K, 4, 2, _p(FAKE), _p(FAKE), _p(FAKE),
                  None, _p(FAKE), _p(FAKE), 8, _p(FAKE), _p(FAKE), 1 << 20, None) == BAD_SHAPE, K
    r = lib.peg_router_topk
    assert r(_p(FAKE), 0, 1 << 29, 2, 1, 0, 1, _p(FAKE), _p(FAKE), None) == BAD_SHAPE
    f = lib.peg_routing_map_compact
    assert f(_p(FAKE), 0, _p(FAKE), (1 << 31) - 1, 1, 1, _p(FAKE), _p(FAKE), None) == BAD_SHAPE
    fb = lib.peg_routing_map_compact_backward
    assert fb(_p(FAKE), _p(FAKE), (1 << 31) - 1, 1, 1, _p(FAKE), None) == BAD_SHAPE


def test_python_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        peg.route_prep(torch.zeros((4, 2), dtype=torch.int32), 4, capacity=2)


def test_plain_c_consumer(tmp_path):
    """The header compiles as strict C99 and the library links from C."""
    import subprocess
    src = os.path.join(ROOT, "tests", "c", "abi_check.c")
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(peg.LIB_PATH)
    lib = os.path.basename(peg.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    src, "-o", str(exe), "-L", libdir, "-l:" + lib, "-Wl,-rpath," + libdir], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert "abi_check ok" in out.stdout



def test_c_gpu_driver_compiles():
    """tests/c/gpu_path.c (the plain C driver of the GPU path, run by the GPU
    tests) builds against the header, the oracle and the HIP runtime; it is
    only compiled here, not run."""
    import __graft_entry__ as entry
    from oracle import build as oracle_build
    oracle_build.ensure_built()
    assert os.access(entry.build_c_driver(), os.X_OK)
