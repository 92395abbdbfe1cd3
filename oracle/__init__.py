"""CPU oracle of the MoE token-routing data path (numpy front end).

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU library never does, and
this package never imports the GPU library. All arithmetic lives in
``peg_oracle.c`` (plain scalar C, double precision); this module only
marshals numpy arrays.

Element types: ``F32`` arrays are ``np.float32``; ``BF16`` and ``F16`` arrays
are raw 16-bit patterns held in ``np.uint16``.

Page references are given per function (title, section):
  [BIN] "Build Triton-Ascend Binned MoE Routing"
  [PAD] "Build Triton-Ascend Padded MoE Routing"
  [MOK] "core.transformer.moe.megakernel.mok.route_adapter"
"""
import ctypes
from ctypes import c_double, c_float, c_int32, c_int64, c_uint8, c_uint16, c_uint32, c_void_p, POINTER

import numpy as np

from . import build as _build

F32, BF16, F16 = 0, 1, 2
BINNED, PADDED = 0, 1

_lib = None


def load_library(path):
    """Open an oracle shared library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i32p, i64p, f32p, f64p = POINTER(c_int32), POINTER(c_int64), POINTER(c_float), POINTER(c_double)
    lib.pego_round_bf16.argtypes = [c_double]
    lib.pego_round_bf16.restype = c_uint16
    lib.pego_round_f16.argtypes = [c_double]
    lib.pego_round_f16.restype = c_uint16
    lib.pego_load.argtypes = [c_void_p, c_int32, c_int64]
    lib.pego_load.restype = c_double
    lib.pego_route_prep.argtypes = [i32p, c_int64, c_int32, c_int32, c_int32, i32p, i32p, i32p, i32p, i32p]
    lib.pego_route_prep.restype = c_int64
    lib.pego_assignment_rows.argtypes = [c_int64, c_int32, c_int32, c_int32, c_int32, i32p, i32p, i32p, i32p, i32p]
    lib.pego_assignment_rows.restype = c_int32
    lib.pego_gather.argtypes = [c_void_p, c_int64, c_int64, c_int32, c_int32, c_int32, c_int32, i32p, i32p,
                                i32p, i32p, c_int64, i64p, c_int64, c_void_p]
    lib.pego_gather.restype = c_int32
    lib.pego_scatter_combine.argtypes = [c_void_p, c_int32, c_int64, c_int64, c_int64, c_int32, c_int32,
                                         c_int32, c_int32, i32p, i32p, i32p, i32p, f32p, i64p, c_int64,
                                         c_void_p, f64p]
    lib.pego_scatter_combine.restype = c_int32
    lib.pego_wgrad.argtypes = [c_void_p, c_void_p, c_int32, c_int64, c_int64, c_int64, c_int32, c_int32,
                               c_int32, c_int32, i32p, i32p, i32p, i32p, i64p, c_int64, f32p, f64p]
    lib.pego_wgrad.restype = c_int32
    lib.pego_combine_backward_dy.argtypes = [c_void_p, c_int32, c_int64, c_int64, c_int32, c_int32, c_int32, c_int32,
                                             i32p, i32p, i32p, i32p, f32p, c_int64, i64p, c_int64, c_void_p]
    lib.pego_combine_backward_dy.restype = c_int32
    lib.pego_routing_map_compact.argtypes = [c_void_p, c_int32, POINTER(c_uint8), c_int64, c_int32, c_int32,
                                             f32p, i32p]
    lib.pego_routing_map_compact.restype = c_int32
    lib.pego_routing_map_compact_backward.argtypes = [f32p, i32p, c_int64, c_int32, c_int32, f32p]
    lib.pego_routing_map_compact_backward.restype = c_int32
    lib.pego_assignment_rows_windows.argtypes = [c_int64, c_int32, c_int32, i32p, i32p, i32p, i32p, i32p, i32p]
    lib.pego_assignment_rows_windows.restype = c_int32
    lib.pego_router_topk.argtypes = [c_void_p, c_int32, c_int64, c_int32, c_int32, c_int32, c_int32, i32p, f32p]
    lib.pego_router_topk.restype = c_int32
    lib.pego_validate_routing.argtypes = [i32p, i32p, i32p, i32p, c_int64, c_int32, c_int32, c_int64]
    lib.pego_validate_routing.restype = c_uint32
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = load_library(_build.ensure_built())
    return _lib


def _p(arr, ctype):
    if arr is None:
        return None
    return arr.ctypes.data_as(POINTER(ctype))


def _vp(arr):
    return None if arr is None else c_void_p(arr.ctypes.data)


def _c(arr, dtype):
    return None if arr is None else np.ascontiguousarray(arr, dtype=dtype)


def _np_dtype(dtype):
    return np.float32 if dtype == F32 else np.uint16


def round_bf16(v):
    """bfloat16 bits of the double ``v``, rounded to nearest even."""
    return int(_load().pego_round_bf16(float(v)))


def round_f16(v):
    """binary16 bits of the double ``v``, rounded to nearest even."""
    return int(_load().pego_round_f16(float(v)))


def to_double(arr, dtype):
    """Exact widening of an element array to float64 (elementwise oracle load)."""
    lib = _load()
    a = np.ascontiguousarray(arr)
    flat = a.reshape(-1)
    out = np.empty(flat.shape[0], dtype=np.float64)
    for i in range(flat.shape[0]):
        out[i] = lib.pego_load(_vp(flat), dtype, i)
    return out.reshape(a.shape)


class Routing:
    """Result of :func:`route_prep` (host arrays)."""

    def __init__(self, T, K, E, indices, bin_ids, tokens_per_expert, bins, padded_bins, n, pad_multiple):
        self.T, self.K, self.E = T, K, E
        self.indices, self.bin_ids = indices, bin_ids
        self.tokens_per_expert, self.bins, self.padded_bins = tokens_per_expert, bins, padded_bins
        self.n = n
        self.pad_multiple = pad_multiple


def route_prep(top_experts, E, pad_multiple=None):
    """[PAD] Workflow steps 1-3 / [BIN] Workflow steps 1-2 (stable sort by expert,
    inclusive bins, padded bins). ``top_experts`` is [T, K] int32, -1 = no route."""
    top = _c(top_experts, np.int32)
    T, K = top.shape
    total = T * K
    indices = np.empty(total, np.int32)
    bin_ids = np.empty(total, np.int32)
    tpe = np.empty(E, np.int32)
    bins = np.empty(E, np.int32)
    padded = np.empty(E, np.int32) if pad_multiple is not None else None
    n = _load().pego_route_prep(_p(top, c_int32), T, K, E, pad_multiple or 0, _p(indices, c_int32),
                                _p(bin_ids, c_int32), _p(tpe, c_int32), _p(bins, c_int32), _p(padded, c_int32))
    if n < 0:
        raise ValueError("oracle route_prep refused its arguments")
    return Routing(T, K, E, indices, bin_ids, tpe, bins, padded, int(n), pad_multiple)


def expert_rows(r, layout, capacity=None):
    """Rows of the expert tensor: E*C (binned) or padded_bins[E-1] (padded)."""
    if layout == BINNED:
        return r.E * capacity
    return int(r.padded_bins[-1]) if r.E > 0 else 0


def assignment_rows(r, layout, capacity=None):
    """Expert-tensor row of every assignment id, -1 = unrouted or dropped."""
    out = np.empty(r.T * r.K, np.int32)
    rc = _load().pego_assignment_rows(r.T, r.K, r.E, layout, capacity or 0, _p(r.indices, c_int32),
                                      _p(r.bin_ids, c_int32), _p(r.bins, c_int32), _p(r.padded_bins, c_int32),
                                      _p(out, c_int32))
    if rc != 0:
        raise ValueError("oracle assignment_rows refused its arguments")
    return out


def assignment_rows_windows(r, row_base, row_limit):
    """Row of every assignment when expert e owns rows [row_base[e],
    row_limit[e]) (-1: no route, or past the window)."""
    total = r.T * r.K
    out = np.empty(total, np.int32)
    base = _c(row_base, np.int32)
    limit = _c(row_limit, np.int32)
    rc = _load().pego_assignment_rows_windows(r.T, r.K, r.E, _p(r.indices, c_int32), _p(r.bin_ids, c_int32),
                                              _p(r.bins, c_int32), _p(base, c_int32), _p(limit, c_int32),
                                              _p(out, c_int32))
    if rc != 0:
        raise ValueError("oracle assignment_rows_windows refused its arguments")
    return out


def gather(x, r, layout, capacity=None, rows=None, R=None):
    """[BIN] Workflow step 3 + Ascend Guardrails / [PAD] Workflow steps 4-5:
    zero expert tensor, kept positions copy token indices[i] // K (bits).
    ``rows``: optional list of expert-tensor rows to return (a sample)."""
    x = np.ascontiguousarray(x)
    T = x.shape[0]
    row_bytes = x.shape[1] * x.itemsize  # numpy reports stride 0 for an empty batch
    H = x.shape[1]
    if R is None:
        R = expert_rows(r, layout, capacity)
    rows_arr = _c(rows, np.int64)
    count = R if rows_arr is None else rows_arr.shape[0]
    out = np.empty((count, H), dtype=x.dtype)
    rc = _load().pego_gather(_vp(x), T, row_bytes, r.K, r.E, layout, capacity or 0, _p(r.indices, c_int32),
                             _p(r.bin_ids, c_int32), _p(r.bins, c_int32), _p(r.padded_bins, c_int32), R,
                             _p(rows_arr, c_int64), 0 if rows_arr is None else count, _vp(out))
    if rc != 0:
        raise ValueError("oracle gather refused its arguments")
    return out


def scatter_combine(y, dtype, r, layout, capacity=None, weights=None, tokens=None, with_scale=False):
    """[BIN] Workflow step 5 / [PAD] Workflow step 6: weighted top-k combine in
    double, rounded once to ``dtype``. Returns out (and the error scale)."""
    y = np.ascontiguousarray(y)
    R, H = y.shape
    w = _c(weights, np.float32)
    tok = _c(tokens, np.int64)
    count = r.T if tok is None else tok.shape[0]
    out = np.empty((count, H), dtype=_np_dtype(dtype))
    scale = np.empty((count, H), np.float64) if with_scale else None
    rc = _load().pego_scatter_combine(_vp(y), dtype, R, r.T, H, r.K, r.E, layout, capacity or 0,
                                      _p(r.indices, c_int32), _p(r.bin_ids, c_int32), _p(r.bins, c_int32),
                                      _p(r.padded_bins, c_int32), _p(w, c_float), _p(tok, c_int64),
                                      0 if tok is None else count, _vp(out), _p(scale, c_double))
    if rc != 0:
        raise ValueError("oracle scatter_combine refused its arguments")
    return (out, scale) if with_scale else out


def wgrad(y, grad, dtype, r, layout, capacity=None, tokens=None, with_scale=False):
    """[BIN] Workflow step 6 / [PAD] Workflow step 6: per kept assignment,
    dot(expert row, grad[token]) in double, rounded to float32. Shape [count, K]."""
    y = np.ascontiguousarray(y)
    grad = np.ascontiguousarray(grad)
    R, H = y.shape
    tok = _c(tokens, np.int64)
    count = r.T if tok is None else tok.shape[0]
    out = np.empty((count, r.K), np.float32)
    scale = np.empty((count, r.K), np.float64) if with_scale else None
    rc = _load().pego_wgrad(_vp(y), _vp(grad), dtype, R, r.T, H, r.K, r.E, layout, capacity or 0,
                            _p(r.indices, c_int32), _p(r.bin_ids, c_int32), _p(r.bins, c_int32),
                            _p(r.padded_bins, c_int32), _p(tok, c_int64), 0 if tok is None else count,
                            _p(out, c_float), _p(scale, c_double))
    if rc != 0:
        raise ValueError("oracle wgrad refused its arguments")
    return (out, scale) if with_scale else out


def combine_backward_dy(dout, dtype, r, layout, capacity=None, weights=None, rows=None, R=None):
    """Gradient of the combine with respect to the expert tensor: kept row of
    assignment a gets w[a] * dout[a // K] (raw copy without weights), other
    rows 0. ``rows``: optional sample of expert-tensor rows."""
    dout = np.ascontiguousarray(dout)
    T, H = dout.shape
    if R is None:
        R = expert_rows(r, layout, capacity)
    w = _c(weights, np.float32)
    rows_arr = _c(rows, np.int64)
    count = R if rows_arr is None else rows_arr.shape[0]
    out = np.empty((count, H), dtype=dout.dtype)
    rc = _load().pego_combine_backward_dy(_vp(dout), dtype, T, H, r.K, r.E, layout, capacity or 0,
                                          _p(r.indices, c_int32), _p(r.bin_ids, c_int32), _p(r.bins, c_int32),
                                          _p(r.padded_bins, c_int32), _p(w, c_float), R, _p(rows_arr, c_int64),
                                          0 if rows_arr is None else count, _vp(out))
    if rc != 0:
        raise ValueError("oracle combine_backward_dy refused its arguments")
    return out


def routing_map_compact(probs, probs_dtype, routing_map, topk):
    """[MOK] routing_map_to_mok_inputs: returns (probs_out f32 [T, topk],
    route_experts int32 [T, topk]) in increasing expert order, -1 / 0 padded."""
    probs = np.ascontiguousarray(probs)
    rmap = np.ascontiguousarray(routing_map).astype(np.uint8, copy=False)
    T, E = rmap.shape
    pout = np.empty((T, topk), np.float32)
    idx = np.empty((T, topk), np.int32)
    rc = _load().pego_routing_map_compact(_vp(probs), probs_dtype, _p(rmap, c_uint8), T, E, topk,
                                          _p(pout, c_float), _p(idx, c_int32))
    if rc != 0:
        raise ValueError("oracle routing_map_compact refused its arguments")
    return pout, idx


def routing_map_compact_backward(grad_probs_out, route_experts, E):
    """[MOK] RoutingMapToIndices backward: dense [T, E] f32 router gradient."""
    g = _c(grad_probs_out, np.float32)
    idx = _c(route_experts, np.int32)
    T, topk = idx.shape
    out = np.empty((T, E), np.float32)
    rc = _load().pego_routing_map_compact_backward(_p(g, c_float), _p(idx, c_int32), T, E, topk,
                                                   _p(out, c_float))
    if rc != 0:
        raise ValueError("oracle routing_map_compact_backward refused its arguments")
    return out


SOFTMAX, SIGMOID = 0, 1


def router_topk(logits, dtype, K, gating=SOFTMAX, normalize=True):
    """[FMD] router top-k gating over scores [T, E] (f32, or bf16/f16 bits):
    returns (top_experts int32 [T, K], highest score first, lower id first on
    ties; weights f32 [T, K], softmax or sigmoid probabilities, renormalised
    over the K choices when ``normalize``)."""
    lg = np.ascontiguousarray(logits, dtype=_np_dtype(dtype))
    T, E = lg.shape
    top = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    rc = _load().pego_router_topk(_vp(lg), dtype, T, E, K, gating, 1 if normalize else 0, _p(top, c_int32),
                                  _p(w, c_float))
    if rc != 0:
        raise ValueError("oracle router_topk refused its arguments")
    return top, w


def validate_routing(indices, bin_ids, bins, padded_bins, T, K, E, n_indices):
    """[BIN]/[PAD] Ascend Guardrails: bitmask of violated routing preconditions."""
    return int(_load().pego_validate_routing(_p(_c(indices, np.int32), c_int32),
                                             _p(_c(bin_ids, np.int32), c_int32),
                                             _p(_c(bins, np.int32), c_int32),
                                             _p(_c(padded_bins, np.int32), c_int32), T, K, E, n_indices))
