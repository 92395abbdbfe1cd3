"""GPU: the entry points are capturable in a HIP graph (they allocate
nothing, synchronise nothing and record no memset), and graph replays give
the eager results. The combine backward at K = 4 (its dy gather and wgrad
launches, with a gap fill launch first for a binned dy of 128 MB) is captured
and replayed on its own the same way.

One step (route_prep -> gather -> combine -> wgrad -> combine backward) on
preallocated buffers is captured once, then replayed three times with new
inputs written into the captured input buffers between replays (eager work
and synchronisations in between); every replay is compared with the eager
results on the same inputs: index outputs and gathers bit for bit, floating
outputs bit for bit too (same kernels, same launch shapes). A second graph
holds the other entry points (router gating alone and fused with
route_prep, compaction and its backward, the validator, the binned gather,
combine and wgrad rebuilding the row map, row windows and the gather by row
map) and is checked the same way.
"""
import numpy as np
import pytest
import torch

import padded_expert_gather_amd as peg
import workloads as W
from gpu_util import DEV, to_dev

pytestmark = pytest.mark.gpu

T, H, E, K, M = 512, 256, 8, 2, 16


def _inputs(seed):
    rng = np.random.default_rng(seed)
    top, w = W.random_routing(rng, T, K, E, none_frac=0.05, skew=0.2)
    x = W.normal(rng, (T, H), W.BF16)
    grad = W.normal(rng, (T, H), W.BF16)
    return top, w, x, grad


def _step(top, w, x, grad, out):
    """All calls write into the preallocated tensors of `out`."""
    r = out["r"]
    lib = peg.library()
    st = torch.cuda.current_stream().cuda_stream
    P = lambda t: None if t is None else t.data_ptr()
    rc = lib.peg_route_prep(P(top), T, K, E, peg.PADDED, 0, M, P(r.indices), P(r.bin_ids), P(r.tokens_per_expert),
                            P(r.bins), P(r.padded_bins), P(r.slot_row), P(out["ws"]), out["ws"].numel(), st)
    assert rc == 0
    R = out["y"].shape[0]
    rc = lib.peg_gather_padded(P(x), peg.BF16, T, H, K, E, P(r.indices), P(r.bin_ids), P(r.bins), P(r.padded_bins),
                               P(r.slot_row), P(out["y"]), R, None, P(out["ws"]), out["ws"].numel(), st)
    assert rc == 0
    rc = lib.peg_scatter_combine(P(out["y"]), peg.BF16, peg.PADDED, T, H, K, E, 0, P(r.indices), P(r.bin_ids),
                                 P(r.bins), P(r.padded_bins), P(r.slot_row), P(w), P(out["comb"]), P(out["ws"]),
                                 out["ws"].numel(), st)
    assert rc == 0
    rc = lib.peg_wgrad(P(out["y"]), P(grad), peg.BF16, peg.PADDED, T, H, K, E, 0, P(r.indices), P(r.bin_ids),
                       P(r.bins), P(r.padded_bins), P(r.slot_row), P(out["wg"]), P(out["ws"]), out["ws"].numel(), st)
    assert rc == 0
    rc = lib.peg_combine_backward(P(out["y"]), P(grad), P(w), peg.BF16, peg.PADDED, T, H, K, E, 0, P(r.indices),
                                  P(r.bin_ids), P(r.bins), P(r.padded_bins), P(r.slot_row), P(out["dy"]), R,
                                  P(out["wgb"]), P(out["ws"]), out["ws"].numel(), st)
    assert rc == 0


def _buffers(R):
    i32 = dict(dtype=torch.int32, device=DEV)
    r = peg.Routing(T, K, E, peg.PADDED, None, M, torch.empty(T * K, **i32), torch.empty(T * K, **i32),
                    torch.empty(E, **i32), torch.empty(E, **i32), torch.empty(E, **i32), torch.empty(T * K, **i32))
    return {"r": r, "ws": torch.empty(peg.workspace_bytes(T, K, E), dtype=torch.uint8, device=DEV),
            "y": torch.empty((R, H), dtype=torch.bfloat16, device=DEV),
            "comb": torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
            "wg": torch.empty((T, K), dtype=torch.float32, device=DEV),
            "dy": torch.empty((R, H), dtype=torch.bfloat16, device=DEV),
            "wgb": torch.empty((T, K), dtype=torch.float32, device=DEV)}


def _snapshot(out):
    r = out["r"]
    return [t.clone() for t in (r.indices, r.bin_ids, r.bins, r.padded_bins, r.slot_row, out["y"], out["comb"],
                                out["wg"], out["dy"], out["wgb"])]


def test_graph_replays_match_eager():
    # every routing of a padded layout fits the largest row count (all
    # assignments in one expert: T*K + E*(M-1) rows)
    R = T * K + E * (M - 1)
    top0, w0, x0, g0 = _inputs(0)
    top, w, x, grad = to_dev(top0), to_dev(w0.reshape(-1)), to_dev(x0, W.BF16), to_dev(g0, W.BF16)
    cap = _buffers(R)
    _step(top, w, x, grad, cap)  # warm up (loads the kernels) before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(top, w, x, grad, cap)
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        tn, wn, xn, gn = _inputs(seed)
        top.copy_(to_dev(tn)); w.copy_(to_dev(wn.reshape(-1)))
        x.copy_(to_dev(xn, W.BF16)); grad.copy_(to_dev(gn, W.BF16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(cap)
        eager = _buffers(R)
        _step(top, w, x, grad, eager)
        torch.cuda.synchronize()
        want = _snapshot(eager)
        n_rows = int(want[3][-1].item())  # padded_bins[E-1]: rows the step defines
        for i, (g, e) in enumerate(zip(got, want)):
            if i in (5, 8):  # expert tensors: the rows the layout defines
                g, e = g[:n_rows], e[:n_rows]
            assert torch.equal(g.view(torch.int16) if g.dtype == torch.bfloat16 else g,
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e), (seed, i)


# ---------------------------------------------------------------------------
# The other entry points in one captured graph: router gating (alone and
# fused with route_prep), routing-map compaction and its backward, row
# windows with the gather by row map, the validator, and the binned gather,
# combine and wgrad rebuilding the row map from the sorted arrays.
# ---------------------------------------------------------------------------
E2, K2, TOPK, C2 = 16, 2, 4, 160


def _inputs2(seed):
    rng = np.random.default_rng(100 + seed)
    logits = rng.standard_normal((T, E2), dtype=np.float32)
    probs = rng.random((T, E2), dtype=np.float32)
    rmap = (rng.random((T, E2)) < 0.2).astype(np.uint8)
    gco = rng.standard_normal((T, TOPK), dtype=np.float32)
    x = W.normal(rng, (T, H), W.BF16)
    grad = W.normal(rng, (T, H), W.BF16)
    base = (np.arange(E2) * C2 + rng.integers(0, 20, size=E2)).astype(np.int32)
    limit = (np.arange(E2) * C2 + C2).astype(np.int32)
    return logits, probs, rmap, gco, x, grad, base, limit


def _buffers2():
    i32 = dict(dtype=torch.int32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    b = {"top": torch.empty((T, K2), **i32), "w": torch.empty((T, K2), **f32),
         "top2": torch.empty((T, K2), **i32), "w2": torch.empty((T, K2), **f32),
         "po": torch.empty((T, TOPK), **f32), "re": torch.empty((T, TOPK), **i32),
         "gp": torch.empty((T, E2), **f32),
         "flags": torch.empty(1, **i32), "y": torch.empty((E2 * C2, H), dtype=torch.bfloat16, device=DEV),
         "yw": torch.empty((E2 * C2, H), dtype=torch.bfloat16, device=DEV),
         "comb": torch.empty((T, H), dtype=torch.bfloat16, device=DEV), "wg": torch.empty((T, K2), **f32),
         "ws": torch.empty(peg.workspace_bytes(T, K2, E2), dtype=torch.uint8, device=DEV)}
    for name in ("idx", "bid", "slot", "idx_w", "bid_w", "slot_w"):
        b[name] = torch.empty(T * K2, **i32)
    for name in ("tpe", "bins", "tpe_w", "bins_w"):
        b[name] = torch.empty(E2, **i32)
    return b


def _step2(inp, b):
    logits, probs, rmap, gco, x, grad, base, limit = inp
    lib = peg.library()
    st = torch.cuda.current_stream().cuda_stream
    P = lambda t: None if t is None else t.data_ptr()
    ws, wsb = P(b["ws"]), b["ws"].numel()
    assert lib.peg_router_topk(P(logits), peg.F32, T, E2, K2, peg.SOFTMAX, 1, P(b["top"]), P(b["w"]), st) == 0
    assert lib.peg_route_prep_logits(P(logits), peg.F32, T, E2, K2, peg.SIGMOID, 0, peg.BINNED, C2, 0, P(b["top2"]),
                                     P(b["w2"]), P(b["idx"]), P(b["bid"]), P(b["tpe"]), P(b["bins"]), None,
                                     P(b["slot"]), ws, wsb, st) == 0
    assert lib.peg_routing_map_compact(P(probs), peg.F32, P(rmap), T, E2, TOPK, P(b["po"]), P(b["re"]), st) == 0
    assert lib.peg_routing_map_compact_backward(P(gco), P(b["re"]), T, E2, TOPK, P(b["gp"]), st) == 0
    assert lib.peg_validate_routing(P(b["idx"]), P(b["bid"]), P(b["bins"]), None, T, K2, E2, -1, P(b["flags"]), ws,
                                    wsb, st) == 0
    # binned gather / combine / wgrad with the row map rebuilt from the sorted arrays
    assert lib.peg_gather_binned(P(x), peg.BF16, T, H, K2, E2, C2, P(b["idx"]), P(b["bid"]), P(b["bins"]), None,
                                 P(b["y"]), ws, wsb, st) == 0
    assert lib.peg_scatter_combine(P(b["y"]), peg.BF16, peg.BINNED, T, H, K2, E2, C2, P(b["idx"]), P(b["bid"]),
                                   P(b["bins"]), None, None, P(b["w2"]), P(b["comb"]), ws, wsb, st) == 0
    assert lib.peg_wgrad(P(b["y"]), P(grad), peg.BF16, peg.BINNED, T, H, K2, E2, C2, P(b["idx"]), P(b["bid"]),
                         P(b["bins"]), None, None, P(b["wg"]), ws, wsb, st) == 0
    # row windows of the router's routes, then the gather by row map into a zeroed tensor
    assert lib.peg_route_prep_windows(P(b["top"]), T, K2, E2, P(base), P(limit), P(b["idx_w"]), P(b["bid_w"]),
                                      P(b["tpe_w"]), P(b["bins_w"]), P(b["slot_w"]), ws, wsb, st) == 0
    b["yw"].zero_()  # a fill kernel, not a memset
    assert lib.peg_gather_rows(P(x), peg.BF16, T, H, K2, P(b["slot_w"]), P(b["yw"]), E2 * C2, None, st) == 0


_SNAP2 = ("top", "w", "top2", "w2", "idx", "bid", "tpe", "bins", "slot", "po", "re", "gp", "flags", "y", "comb",
          "wg", "idx_w", "bid_w", "tpe_w", "bins_w", "slot_w", "yw")


def _dev2(arrs):
    return [to_dev(a, W.BF16) if i in (4, 5) else to_dev(a) for i, a in enumerate(arrs)]


def test_graph_other_entry_points_match_eager():
    inp = _dev2(_inputs2(0))
    cap = _buffers2()
    _step2(inp, cap)  # warm up before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step2(inp, cap)
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        for dst, src in zip(inp, _dev2(_inputs2(seed))):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: cap[k].clone() for k in _SNAP2}
        eager = _buffers2()
        _step2(inp, eager)
        torch.cuda.synchronize()
        for k in _SNAP2:
            g, e = got[k], eager[k]
            if g.dtype == torch.bfloat16:
                g, e = g.view(torch.int16), e.view(torch.int16)
            assert torch.equal(g, e), (seed, k)
        assert int(got["flags"].item()) == 0


@pytest.mark.parametrize("layout", [peg.PADDED, peg.BINNED])
def test_graph_split_combine_backward(layout):
    """The combine backward at K = 4 (a dy gather launch, then the wgrad
    kernel; for the binned dy of 128 MB and more a gap fill launch first)
    captured once and replayed three times with new upstream gradients and
    weights written into the captured buffers: every replay equals the eager
    call on the same inputs, bit for bit."""
    Tb, Hb, Eb, Kb = 1024, 512, 8, 4
    Cb = 16384 if layout == peg.BINNED else 0  # binned dy: 8 * 16384 rows * 1 KiB = 128 MiB
    print(f"[graph split backward] layout{layout} T{Tb} H{Hb} E{Eb} K{Kb} C{Cb}", flush=True)
    rng = np.random.default_rng(40 + layout)
    top, _ = W.random_routing(rng, Tb, Kb, Eb, none_frac=0.05, skew=0.3)
    top_d = to_dev(top)
    r = peg.route_prep(top_d, Eb, capacity=Cb) if layout == peg.BINNED else peg.route_prep(top_d, Eb, pad_multiple=M)
    R = Eb * Cb if layout == peg.BINNED else r.expert_rows()
    y = to_dev(W.normal(rng, (R, Hb), W.BF16), W.BF16)
    dout = torch.empty((Tb, Hb), dtype=torch.bfloat16, device=DEV)
    w = torch.empty(Tb * Kb, dtype=torch.float32, device=DEV)
    dy = torch.empty((R, Hb), dtype=torch.bfloat16, device=DEV)
    wg = torch.empty(Tb * Kb, dtype=torch.float32, device=DEV)
    ws = torch.empty(peg.workspace_bytes(Tb, Kb, Eb), dtype=torch.uint8, device=DEV)
    lib = peg.library()

    def call():
        st = torch.cuda.current_stream().cuda_stream
        P = lambda t: None if t is None else t.data_ptr()
        rc = lib.peg_combine_backward(P(y), P(dout), P(w), peg.BF16, layout, Tb, Hb, Kb, Eb, Cb, P(r.indices),
                                      P(r.bin_ids), P(r.bins), P(r.padded_bins), P(r.slot_row), P(dy), R, P(wg),
                                      P(ws), ws.numel(), st)
        assert rc == 0

    dout.copy_(to_dev(W.normal(rng, (Tb, Hb), W.BF16), W.BF16))
    w.copy_(torch.from_numpy(rng.random(Tb * Kb, dtype=np.float32)).to(DEV))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        dout.copy_(to_dev(W.normal(rng, (Tb, Hb), W.BF16), W.BF16))
        w.copy_(torch.from_numpy(rng.random(Tb * Kb, dtype=np.float32)).to(DEV))
        call()  # eager
        torch.cuda.synchronize()
        dy_e, wg_e = dy.clone(), wg.clone()
        dy.fill_(7.0)
        wg.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dy.view(torch.int16), dy_e.view(torch.int16)), f"replay {rep}: dy differs from eager"
        assert torch.equal(wg, wg_e), f"replay {rep}: wgrad differs from eager"
