"""MI355X (gfx950) MoE token-routing data path: Python binding of ``libpeg.so``.

Every function here marshals torch tensors into the C ABI declared in
``include/peg.h`` and returns; all computation runs in the library's HIP
kernels on torch's current stream. torch provides device memory and streams
only. There is no CPU fallback: on a machine without the GPU library or
without a GPU the calls raise.

Functions (same names as the C entry points without the ``peg_`` prefix):
  route_prep, route_prep_noalloc, gather_binned, gather_padded, scatter_combine, wgrad,
  combine_backward, router_topk, route_prep_logits, route_prep_windows,
  gather_rows, routing_map_compact,
  routing_map_compact_backward, validate_routing.
"""
import ctypes
import os
from ctypes import c_int32, c_int64, c_size_t, c_void_p

import torch  # loads torch's HIP runtime first; libpeg then binds to the same one

HERE = os.path.dirname(os.path.abspath(__file__))
# PEG_LIBRARY may name another build of the same sources (a tuning variant)
LIB_PATH = os.environ.get("PEG_LIBRARY") or os.path.join(HERE, "libpeg.so")

F32, BF16, F16 = 0, 1, 2
BINNED, PADDED = 0, 1
FLAG_BINS_NOT_MONOTONIC = 0x1
FLAG_BINS_TOTAL = 0x2
FLAG_BIN_IDS = 0x4
FLAG_PADDED_BINS = 0x8
FLAG_INDICES = 0x10
FLAG_OUT_ROWS = 0x20
SOFTMAX, SIGMOID = 0, 1

_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_lib = None


class PegError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if os.environ.get("PEG_LIBRARY"):
            raise OSError(f"PEG_LIBRARY names {LIB_PATH}, which does not exist")
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    st = c_int32
    sig = {
        "peg_status_string": ([c_int32], ctypes.c_char_p),
        "peg_abi_version": ([], c_int32),
        "peg_workspace_bytes": ([c_int64, c_int32, c_int32], c_size_t),
        "peg_route_prep": ([P, c_int64, c_int32, c_int32, c_int32, c_int32, c_int32, P, P, P, P, P, P, P, c_size_t,
                            P], st),
        "peg_route_prep_noalloc": ([P, c_int64, c_int32, c_int32, c_int32, c_int32, c_int32, P, P, P, P, P, P, P],
                                   st),
        "peg_gather_binned": ([P, c_int32, c_int64, c_int64, c_int32, c_int32, c_int32, P, P, P, P, P, P, c_size_t,
                               P], st),
        "peg_gather_padded": ([P, c_int32, c_int64, c_int64, c_int32, c_int32, P, P, P, P, P, P, c_int64, P, P,
                               c_size_t, P], st),
        "peg_scatter_combine": ([P, c_int32, c_int32, c_int64, c_int64, c_int32, c_int32, c_int32, P, P, P, P, P, P,
                                 P, P, c_size_t, P], st),
        "peg_wgrad": ([P, P, c_int32, c_int32, c_int64, c_int64, c_int32, c_int32, c_int32, P, P, P, P, P, P, P,
                       c_size_t, P], st),
        "peg_combine_backward": ([P, P, P, c_int32, c_int32, c_int64, c_int64, c_int32, c_int32, c_int32, P, P, P, P,
                                  P, P, c_int64, P, P, c_size_t, P], st),
        "peg_router_topk": ([P, c_int32, c_int64, c_int32, c_int32, c_int32, c_int32, P, P, P], st),
        "peg_route_prep_windows": ([P, c_int64, c_int32, c_int32, P, P, P, P, P, P, P, P, c_size_t, P], st),
        "peg_gather_rows": ([P, c_int32, c_int64, c_int64, c_int32, P, P, c_int64, P, P], st),
        "peg_route_prep_logits": ([P, c_int32, c_int64, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                   c_int32, P, P, P, P, P, P, P, P, P, c_size_t, P], st),
        "peg_routing_map_compact": ([P, c_int32, P, c_int64, c_int32, c_int32, P, P, P], st),
        "peg_routing_map_compact_backward": ([P, P, c_int64, c_int32, c_int32, P, P], st),
        "peg_validate_routing": ([P, P, P, P, c_int64, c_int32, c_int32, c_int64, P, P, c_size_t, P], st),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (builds it first if nothing is built)."""
    return _load()


def _check(status, what):
    if status != 0:
        msg = _load().peg_status_string(status).decode()
        exc = ValueError if status in (1, 2, 3, 4, 6, 7) else PegError
        raise exc(f"{what}: {msg} (status {status})")


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device):
    return c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t, name):
    if t.dtype not in _DT:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def workspace_bytes(T, K, E):
    return int(_load().peg_workspace_bytes(T, K, E))


def _ws(T, K, E, device, ws):
    need = workspace_bytes(T, K, E)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


class Routing:
    """Routing arrays on the device, as produced by :func:`route_prep`."""

    def __init__(self, T, K, E, layout, capacity, pad_multiple, indices, bin_ids, tokens_per_expert, bins,
                 padded_bins, slot_row):
        self.T, self.K, self.E = T, K, E
        self.layout, self.capacity, self.pad_multiple = layout, capacity, pad_multiple
        self.indices, self.bin_ids = indices, bin_ids
        self.tokens_per_expert, self.bins, self.padded_bins = tokens_per_expert, bins, padded_bins
        self.slot_row = slot_row

    def num_valid(self):
        """n = bins[E-1] (synchronises)."""
        return int(self.bins[-1].item())

    def expert_rows(self):
        """Rows of the expert tensor: E*C (binned) or padded_bins[E-1] (synchronises)."""
        if self.layout == BINNED:
            return self.E * self.capacity
        return int(self.padded_bins[-1].item())


def route_prep(top_experts, num_experts, capacity=None, pad_multiple=None, ws=None):
    """Stable sort of the assignments by expert, bins and padded bins.

    top_experts: [T, K] int32 on the GPU, -1 (or any id outside [0, E)) = no
    route. Binned layout when ``capacity`` is given, padded when only
    ``pad_multiple`` is; giving both builds padded_bins for a binned layout.
    """
    top = _dev(top_experts, "top_experts", torch.int32)
    if top.dim() != 2:
        raise ValueError("top_experts must be [T, K]")
    T, K = top.shape
    E = int(num_experts)
    if capacity is None and pad_multiple is None:
        raise ValueError("give capacity (binned) or pad_multiple (padded)")
    layout = BINNED if capacity is not None else PADDED
    dev = top.device
    total = T * K
    i32 = dict(dtype=torch.int32, device=dev)
    indices = torch.empty(total, **i32)
    bin_ids = torch.empty(total, **i32)
    tpe = torch.empty(E, **i32)
    bins = torch.empty(E, **i32)
    padded = torch.empty(E, **i32) if pad_multiple is not None else None
    slot_row = torch.empty(total, **i32)
    ws, wsb = _ws(T, K, E, dev, ws)
    with torch.cuda.device(dev):
        st = _load().peg_route_prep(_ptr(top), T, K, E, layout, int(capacity or 0), int(pad_multiple or 0),
                                    _ptr(indices), _ptr(bin_ids), _ptr(tpe), _ptr(bins), _ptr(padded),
                                    _ptr(slot_row), _ptr(ws), wsb, _stream(dev))
    _check(st, "route_prep")
    return Routing(T, K, E, layout, capacity, pad_multiple, indices, bin_ids, tpe, bins, padded, slot_row)


def route_prep_noalloc(top_experts, num_experts, capacity=None, pad_multiple=None, out=None):
    """route_prep through the allocation-free entry point (the library's own
    static device scratch, no workspace). ``out`` may hold preallocated
    output tensors (a Routing of the same sizes) so that nothing at all is
    allocated; otherwise they are allocated here, before the call."""
    top = _dev(top_experts, "top_experts", torch.int32)
    if top.dim() != 2:
        raise ValueError("top_experts must be [T, K]")
    T, K = top.shape
    E = int(num_experts)
    if capacity is None and pad_multiple is None:
        raise ValueError("give capacity (binned) or pad_multiple (padded)")
    layout = BINNED if capacity is not None else PADDED
    dev = top.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = Routing(T, K, E, layout, capacity, pad_multiple, torch.empty(T * K, **i32), torch.empty(T * K, **i32),
                      torch.empty(E, **i32), torch.empty(E, **i32),
                      torch.empty(E, **i32) if pad_multiple is not None else None, torch.empty(T * K, **i32))
    else:
        out.T, out.K, out.E, out.layout, out.capacity, out.pad_multiple = T, K, E, layout, capacity, pad_multiple
    for name, t, n in (("indices", out.indices, T * K), ("bin_ids", out.bin_ids, T * K),
                       ("tokens_per_expert", out.tokens_per_expert, E), ("bins", out.bins, E),
                       ("slot_row", out.slot_row, T * K)):
        _dev(t, name, torch.int32)
        if t.numel() < n:
            raise ValueError(f"{name} must hold {n} values")
    if pad_multiple is not None:
        if out.padded_bins is None or out.padded_bins.numel() < E:
            raise ValueError("padded_bins must hold E values")
    with torch.cuda.device(dev):
        st = _load().peg_route_prep_noalloc(_ptr(top), T, K, E, layout, int(capacity or 0), int(pad_multiple or 0),
                                            _ptr(out.indices), _ptr(out.bin_ids), _ptr(out.tokens_per_expert),
                                            _ptr(out.bins), _ptr(out.padded_bins if pad_multiple is not None
                                                                 else None),
                                            _ptr(out.slot_row), _stream(dev))
    _check(st, "route_prep_noalloc")
    return out


def route_prep_logits(logits, K, capacity=None, pad_multiple=None, gating=SOFTMAX, normalize=True, ws=None):
    """Router top-k gating fused with route_prep: router scores [T, E]
    (f32/bf16/f16) -> (Routing, top_experts int32 [T, K], weights f32 [T, K]).
    Same layouts as :func:`route_prep`."""
    logits = _dev(logits, "logits")
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    K = int(K)
    if capacity is None and pad_multiple is None:
        raise ValueError("give capacity (binned) or pad_multiple (padded)")
    layout = BINNED if capacity is not None else PADDED
    dev = logits.device
    total = T * K
    i32 = dict(dtype=torch.int32, device=dev)
    top = torch.empty((T, K), **i32)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    indices = torch.empty(total, **i32)
    bin_ids = torch.empty(total, **i32)
    tpe = torch.empty(E, **i32)
    bins = torch.empty(E, **i32)
    padded = torch.empty(E, **i32) if pad_multiple is not None else None
    slot_row = torch.empty(total, **i32)
    ws, wsb = _ws(T, K, E, dev, ws)
    with torch.cuda.device(dev):
        st = _load().peg_route_prep_logits(_ptr(logits), _dtype_code(logits, "logits"), T, E, K, int(gating),
                                           1 if normalize else 0, layout, int(capacity or 0),
                                           int(pad_multiple or 0), _ptr(top), _ptr(w), _ptr(indices),
                                           _ptr(bin_ids), _ptr(tpe), _ptr(bins), _ptr(padded), _ptr(slot_row),
                                           _ptr(ws), wsb, _stream(dev))
    _check(st, "route_prep_logits")
    return Routing(T, K, E, layout, capacity, pad_multiple, indices, bin_ids, tpe, bins, padded, slot_row), top, w


def route_prep_windows(top_experts, num_experts, row_base, row_limit, capacity=None, ws=None):
    """route_prep with expert e's rows in [row_base[e], row_limit[e]) (int32
    device tensors): same sorted arrays as route_prep, slot_row in the
    windows. ``capacity`` (optional) tags the result as a binned layout of E
    * capacity rows for the combine / wgrad calls that take it; its gaps are
    the caller's (see gather_rows)."""
    top = _dev(top_experts, "top_experts", torch.int32)
    if top.dim() != 2:
        raise ValueError("top_experts must be [T, K]")
    T, K = top.shape
    E = int(num_experts)
    base = _dev(row_base, "row_base", torch.int32)
    limit = _dev(row_limit, "row_limit", torch.int32)
    if base.numel() != E or limit.numel() != E:
        raise ValueError("row_base and row_limit must hold E values")
    dev = top.device
    i32 = dict(dtype=torch.int32, device=dev)
    indices = torch.empty(T * K, **i32)
    bin_ids = torch.empty(T * K, **i32)
    tpe = torch.empty(E, **i32)
    bins = torch.empty(E, **i32)
    slot_row = torch.empty(T * K, **i32)
    ws, wsb = _ws(T, K, E, dev, ws)
    with torch.cuda.device(dev):
        st = _load().peg_route_prep_windows(_ptr(top), T, K, E, _ptr(base), _ptr(limit), _ptr(indices),
                                            _ptr(bin_ids), _ptr(tpe), _ptr(bins), _ptr(slot_row), _ptr(ws), wsb,
                                            _stream(dev))
    _check(st, "route_prep_windows")
    return Routing(T, K, E, BINNED, capacity, None, indices, bin_ids, tpe, bins, None, slot_row)


def gather_rows(x, slot_row, K, out, err_flag=None):
    """out[slot_row[a]] = x[a // K] for every a with 0 <= slot_row[a] < rows
    of out; no other row of out is written."""
    x = _dev(x, "x")
    slot_row = _dev(slot_row, "slot_row", torch.int32)
    out = _dev(out, "out", x.dtype)
    T, H = x.shape
    if slot_row.numel() != T * int(K) or out.shape[1] != H:
        raise ValueError("slot_row must hold T*K rows and out must have rows of H elements")
    with torch.cuda.device(x.device):
        st = _load().peg_gather_rows(_ptr(x), _dtype_code(x, "x"), T, H, int(K), _ptr(slot_row), _ptr(out),
                                     out.shape[0], _ptr(err_flag), _stream(x.device))
    _check(st, "gather_rows")
    return out


def _slot(r, use_slot_row):
    return r.slot_row if use_slot_row else None


def _same_device(r, t, name):
    if r.bins.device != t.device:
        raise ValueError(f"{name} is on {t.device}, the routing on {r.bins.device}")


def _expert_tensor(y, r, name):
    """y must be a 2-D expert tensor on the routing's device; a binned layout
    needs at least E*C rows (a padded one padded_bins[E-1] rows, which the
    caller guarantees: checking it would synchronise)."""
    if y.dim() != 2:
        raise ValueError(f"{name} must be [rows, H]")
    _same_device(r, y, name)
    if r.layout == BINNED and r.capacity is not None and y.shape[0] < r.E * r.capacity:
        raise ValueError(f"{name} must have E*C = {r.E * r.capacity} rows, got {y.shape[0]}")


def gather_binned(x, r, out=None, ws=None, use_slot_row=True):
    """Binned dispatch: [E*C, H] with every row written (zeros for unused capacity)."""
    x = _dev(x, "x")
    if r.layout != BINNED and r.capacity is None:
        raise ValueError("routing has no capacity")
    if x.dim() != 2:
        raise ValueError("x must be [T, H]")
    _same_device(r, x, "x")
    T, H = x.shape
    if T != r.T:
        raise ValueError("x rows != T")
    rows = r.E * r.capacity
    if out is None:
        out = torch.empty((rows, H), dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype)
    if out.shape != (rows, H):
        raise ValueError(f"out must be [{rows}, {H}]")
    ws, wsb = _ws(r.T, r.K, r.E, x.device, ws)
    with torch.cuda.device(x.device):
        st = _load().peg_gather_binned(_ptr(x), _dtype_code(x, "x"), T, H, r.K, r.E, r.capacity, _ptr(r.indices),
                                       _ptr(r.bin_ids), _ptr(r.bins), _ptr(_slot(r, use_slot_row)), _ptr(out),
                                       _ptr(ws), wsb, _stream(x.device))
    _check(st, "gather_binned")
    return out


def gather_padded(x, r, out=None, out_rows=None, err_flag=None, ws=None, use_slot_row=True):
    """Padded dispatch: [padded_bins[E-1], H], gap rows zero. Without ``out`` or
    ``out_rows`` the row count is read back from the device (one sync)."""
    x = _dev(x, "x")
    if r.padded_bins is None:
        raise ValueError("routing has no padded_bins")
    if r.layout != PADDED and use_slot_row:
        # its slot_row holds binned rows (e*C + offset), not padded ones
        raise ValueError("routing was prepared for the binned layout: its slot_row does not address the padded "
                         "tensor; route with pad_multiple only, or pass use_slot_row=False")
    if x.dim() != 2:
        raise ValueError("x must be [T, H]")
    _same_device(r, x, "x")
    T, H = x.shape
    if T != r.T:
        raise ValueError("x rows != T")
    if out is None:
        rows = out_rows if out_rows is not None else int(r.padded_bins[-1].item())
        out = torch.empty((rows, H), dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype)
    if out.dim() != 2 or out.shape[1] != H:
        raise ValueError("out must be [rows, H]")
    ws, wsb = _ws(r.T, r.K, r.E, x.device, ws)
    with torch.cuda.device(x.device):
        st = _load().peg_gather_padded(_ptr(x), _dtype_code(x, "x"), T, H, r.K, r.E, _ptr(r.indices),
                                       _ptr(r.bin_ids), _ptr(r.bins), _ptr(r.padded_bins),
                                       _ptr(_slot(r, use_slot_row)), _ptr(out), out.shape[0], _ptr(err_flag),
                                       _ptr(ws), wsb, _stream(x.device))
    _check(st, "gather_padded")
    return out


def scatter_combine(y, r, weights=None, out=None, ws=None, use_slot_row=True):
    """out[t] = sum over kept k of w[t, k] * y[row(t, k)] (fp32 accumulate), [T, H] in y's dtype."""
    y = _dev(y, "y")
    _expert_tensor(y, r, "y")
    H = y.shape[1]
    if weights is not None:
        weights = _dev(weights, "weights", torch.float32)
        if weights.numel() != r.T * r.K:
            raise ValueError("weights must hold T*K values")
    if out is None:
        out = torch.empty((r.T, H), dtype=y.dtype, device=y.device)
    _dev(out, "out", y.dtype)
    if out.shape != (r.T, H):
        raise ValueError("out must be [T, H]")
    ws, wsb = _ws(r.T, r.K, r.E, y.device, ws)
    with torch.cuda.device(y.device):
        st = _load().peg_scatter_combine(_ptr(y), _dtype_code(y, "y"), r.layout, r.T, H, r.K, r.E,
                                         int(r.capacity or 0), _ptr(r.indices), _ptr(r.bin_ids), _ptr(r.bins),
                                         _ptr(r.padded_bins), _ptr(_slot(r, use_slot_row)), _ptr(weights),
                                         _ptr(out), _ptr(ws), wsb, _stream(y.device))
    _check(st, "scatter_combine")
    return out


def wgrad(y, grad, r, out=None, ws=None, use_slot_row=True):
    """Router-weight gradient: [T, K] float32, <y[row(t,k)], grad[t]> for kept routes, else 0."""
    y = _dev(y, "y")
    _expert_tensor(y, r, "y")
    grad = _dev(grad, "grad", y.dtype)
    H = y.shape[1]
    if grad.shape != (r.T, H):
        raise ValueError("grad must be [T, H]")
    if out is None:
        out = torch.empty((r.T, r.K), dtype=torch.float32, device=y.device)
    _dev(out, "out", torch.float32)
    if out.numel() != r.T * r.K:
        raise ValueError("out must hold T*K values")
    ws, wsb = _ws(r.T, r.K, r.E, y.device, ws)
    with torch.cuda.device(y.device):
        st = _load().peg_wgrad(_ptr(y), _ptr(grad), _dtype_code(y, "y"), r.layout, r.T, H, r.K, r.E,
                               int(r.capacity or 0), _ptr(r.indices), _ptr(r.bin_ids), _ptr(r.bins),
                               _ptr(r.padded_bins), _ptr(_slot(r, use_slot_row)), _ptr(out), _ptr(ws), wsb,
                               _stream(y.device))
    _check(st, "wgrad")
    return out


def combine_backward(y, dout, r, weights=None, dy=None, dy_rows=None, wgrad_out=None, ws=None, use_slot_row=True):
    """Backward of the combine with wgrad: returns (dy, wgrad) where
    dy[row(a)] = w[a] * dout[t] in the expert layout (gap rows zero; a raw copy
    when weights is None) and wgrad [T, K] f32 = <y[row(a)], dout[t]>.
    One fused pass for K <= 2; for larger K a dy gather, then the wgrad kernel."""
    y = _dev(y, "y")
    _expert_tensor(y, r, "y")
    dout = _dev(dout, "dout", y.dtype)
    H = y.shape[1]
    if dout.shape != (r.T, H):
        raise ValueError("dout must be [T, H]")
    if weights is not None:
        weights = _dev(weights, "weights", torch.float32)
        if weights.numel() != r.T * r.K:
            raise ValueError("weights must hold T*K values")
    if dy is None:
        rows = dy_rows if dy_rows is not None else (r.E * r.capacity if r.layout == BINNED else r.expert_rows())
        dy = torch.empty((rows, H), dtype=y.dtype, device=y.device)
    _dev(dy, "dy", y.dtype)
    if dy.dim() != 2 or dy.shape[1] != H:
        raise ValueError("dy must be [rows, H]")
    if wgrad_out is None:
        wgrad_out = torch.empty((r.T, r.K), dtype=torch.float32, device=y.device)
    _dev(wgrad_out, "wgrad_out", torch.float32)
    if wgrad_out.numel() != r.T * r.K:
        raise ValueError("wgrad_out must hold T*K values")
    ws, wsb = _ws(r.T, r.K, r.E, y.device, ws)
    with torch.cuda.device(y.device):
        st = _load().peg_combine_backward(_ptr(y), _ptr(dout), _ptr(weights), _dtype_code(y, "y"), r.layout, r.T, H,
                                          r.K, r.E, int(r.capacity or 0), _ptr(r.indices), _ptr(r.bin_ids),
                                          _ptr(r.bins), _ptr(r.padded_bins), _ptr(_slot(r, use_slot_row)), _ptr(dy),
                                          dy.shape[0], _ptr(wgrad_out), _ptr(ws), wsb, _stream(y.device))
    _check(st, "combine_backward")
    return dy, wgrad_out


def router_topk(logits, K, gating=SOFTMAX, normalize=True, top_experts=None, weights=None):
    """Router top-k gating over scores [T, E] (f32/bf16/f16): returns
    (top_experts int32 [T, K], highest score first, lower id first on ties;
    weights f32 [T, K], softmax or sigmoid, renormalised over K if asked)."""
    logits = _dev(logits, "logits")
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    if top_experts is None:
        top_experts = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    _dev(top_experts, "top_experts", torch.int32)
    _dev(weights, "weights", torch.float32)
    if top_experts.numel() != T * K or weights.numel() != T * K:
        raise ValueError("top_experts and weights must hold T*K values")
    with torch.cuda.device(logits.device):
        st = _load().peg_router_topk(_ptr(logits), _dtype_code(logits, "logits"), T, E, int(K), int(gating),
                                     1 if normalize else 0, _ptr(top_experts), _ptr(weights),
                                     _stream(logits.device))
    _check(st, "router_topk")
    return top_experts, weights


def routing_map_compact(probs, routing_map, topk, probs_out=None, route_experts=None):
    """Dense [T, E] routing map -> (probs_out f32 [T, topk], route_experts i32 [T, topk]),
    increasing expert order, padded with -1 / 0."""
    probs = _dev(probs, "probs")
    rmap = _dev(routing_map, "routing_map")
    if rmap.dtype == torch.bool:
        rmap = rmap.view(torch.uint8)
    if rmap.dtype != torch.uint8:
        raise ValueError("routing_map must be bool or uint8")
    T, E = probs.shape
    if rmap.shape != (T, E):
        raise ValueError("routing_map must match probs")
    if probs_out is None:
        probs_out = torch.empty((T, topk), dtype=torch.float32, device=probs.device)
    if route_experts is None:
        route_experts = torch.empty((T, topk), dtype=torch.int32, device=probs.device)
    _dev(probs_out, "probs_out", torch.float32)
    _dev(route_experts, "route_experts", torch.int32)
    if probs_out.numel() != T * topk or route_experts.numel() != T * topk:
        raise ValueError("probs_out and route_experts must hold T*topk values")
    with torch.cuda.device(probs.device):
        st = _load().peg_routing_map_compact(_ptr(probs), _dtype_code(probs, "probs"), _ptr(rmap), T, E, int(topk),
                                             _ptr(probs_out), _ptr(route_experts), _stream(probs.device))
    _check(st, "routing_map_compact")
    return probs_out, route_experts


def routing_map_compact_backward(grad_probs_out, route_experts, num_experts, out=None):
    """Scatter compact router gradients back to a dense [T, E] float32 tensor."""
    g = _dev(grad_probs_out, "grad_probs_out", torch.float32)
    idx = _dev(route_experts, "route_experts", torch.int32)
    if idx.dim() != 2:
        raise ValueError("route_experts must be [T, topk]")
    T, topk = idx.shape
    if g.numel() != T * topk:
        raise ValueError("grad_probs_out must match route_experts")
    if out is None:
        out = torch.empty((T, num_experts), dtype=torch.float32, device=g.device)
    _dev(out, "out", torch.float32)
    if out.numel() != T * int(num_experts):
        raise ValueError("out must be [T, num_experts]")
    with torch.cuda.device(g.device):
        st = _load().peg_routing_map_compact_backward(_ptr(g), _ptr(idx), T, int(num_experts), topk, _ptr(out),
                                                      _stream(g.device))
    _check(st, "routing_map_compact_backward")
    return out


def validate_routing(r, n_indices=-1, indices=None, bin_ids=None, bins=None, padded_bins=None, ws=None):
    """Device uint32 bitmask (as an int32 tensor of one element) of violated
    routing preconditions; the arrays default to those of ``r``."""
    indices = r.indices if indices is None else indices
    bin_ids = r.bin_ids if bin_ids is None else bin_ids
    bins = r.bins if bins is None else bins
    padded_bins = r.padded_bins if padded_bins is None else padded_bins
    for name, t, n in (("indices", indices, r.T * r.K), ("bin_ids", bin_ids, r.T * r.K), ("bins", bins, r.E),
                       ("padded_bins", padded_bins, r.E)):
        if t is not None:
            _dev(t, name, torch.int32)
            if t.numel() != n:
                raise ValueError(f"{name} must hold {n} values")
    dev = bins.device
    flags = torch.empty(1, dtype=torch.int32, device=dev)
    ws, wsb = _ws(r.T, r.K, r.E, dev, ws)
    with torch.cuda.device(dev):
        st = _load().peg_validate_routing(_ptr(indices), _ptr(bin_ids), _ptr(bins), _ptr(padded_bins), r.T, r.K,
                                          r.E, int(n_indices), _ptr(flags), _ptr(ws), wsb, _stream(dev))
    _check(st, "validate_routing")
    return flags
