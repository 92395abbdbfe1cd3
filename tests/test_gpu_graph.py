"""GPU: the entry points are capturable in a HIP graph (they allocate
nothing, synchronise nothing and record no memset), and graph replays give
the eager results.

One step (route_prep -> gather -> combine -> wgrad -> combine backward) on
preallocated buffers is captured once, then replayed three times with new
inputs written into the captured input buffers between replays (eager work
and synchronisations in between); every replay is compared with the eager
results on the same inputs: index outputs and gathers bit for bit, floating
outputs bit for bit too (same kernels, same launch shapes).
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
