"""GPU: seeded random shapes through the whole path, against the oracle.

Each seed draws a layout, element type, T (0..3000), K (1..16, at most E),
E (1..300), H (1..700), a capacity or padding multiple, a share of absent
routes and a skew, then checks route_prep, both forms of the gather, the
combine, wgrad and the combine backward with the rules of the edge tests:
integer outputs and gathers bit for bit, floating outputs within the
tolerance of tests/gpu_util.py. A second set of seeds draws shapes for the
compaction and its backward, the router gating alone and fused with
route_prep, and row windows. The seed is in the test id, so a failure names
its case. PEG_RANDOM_SEEDS=N in the environment runs N seeds of each set
(default 150 and 60).
"""
import os

import numpy as np
import pytest

import oracle
import padded_expert_gather_amd as peg
import workloads as W
from gpu_util import assert_close, bits_equal, to_dev, to_host
from test_gpu_edge import check_combine_backward

pytestmark = pytest.mark.gpu

# seeds of the two sets (150 and 60); PEG_RANDOM_SEEDS=N runs N of each
_N = os.environ.get("PEG_RANDOM_SEEDS")
SEEDS = list(range(int(_N) if _N else 150))
OTHER_SEEDS = list(range(int(_N) if _N else 60))


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([1, 2, 3, 8, 16, 33, 64, 129, 256, 300]))
    K = int(min(E, rng.choice([1, 2, 3, 4, 8, 9, 16])))
    T = int(rng.choice([0, 1, 7, 100, 777, 2048, 3000]))
    H = int(rng.choice([1, 2, 3, 8, 33, 64, 250, 512, 700]))
    dtype = int(rng.choice([W.F32, W.BF16, W.F16]))
    layout = int(rng.choice([W.BINNED, W.PADDED]))
    cap = int(rng.integers(1, max(2, 2 * T * K // E + 2))) if layout == W.BINNED else None
    m = int(rng.choice([1, 2, 8, 64, 128])) if layout == W.PADDED else None
    none_frac = float(rng.choice([0.0, 0.1, 0.5]))
    skew = float(rng.choice([0.0, 0.3, 1.0]))
    return rng, dict(T=T, K=K, E=E, H=H, dtype=dtype, layout=layout, cap=cap, m=m, none_frac=none_frac, skew=skew)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape(seed):
    rng, c = _draw(seed)
    T, K, E, H, dtype, layout, cap, m = (c[k] for k in ("T", "K", "E", "H", "dtype", "layout", "cap", "m"))
    print(f"[random] seed {seed}: {c}", flush=True)
    top, w = W.random_routing(rng, T, K, E, none_frac=c["none_frac"], skew=c["skew"])
    x = W.normal(rng, (T, H), dtype)
    grad = W.normal(rng, (T, H), dtype)
    ro = oracle.route_prep(top, E, pad_multiple=m)
    rg = peg.route_prep(to_dev(top), E, capacity=cap, pad_multiple=m)
    bits_equal(to_host(rg.indices), ro.indices, "indices")
    bits_equal(to_host(rg.bin_ids), ro.bin_ids, "bin_ids")
    bits_equal(to_host(rg.tokens_per_expert), ro.tokens_per_expert, "tokens_per_expert")
    bits_equal(to_host(rg.bins), ro.bins, "bins")
    if m is not None:
        bits_equal(to_host(rg.padded_bins), ro.padded_bins, "padded_bins")
    rows = oracle.assignment_rows(ro, layout, cap)
    bits_equal(to_host(rg.slot_row), rows, "slot_row")
    R = oracle.expert_rows(ro, layout, cap)
    xg = to_dev(x, dtype)
    gather = peg.gather_binned if layout == W.BINNED else peg.gather_padded
    yo = oracle.gather(x, ro, layout, cap)
    yg = gather(xg, rg)
    bits_equal(to_host(yg), yo, "gather")
    bits_equal(to_host(gather(xg, rg, use_slot_row=False)), yo, "gather (rebuilt map)")
    # T = 0 runs on: empty combine and wgrad outputs, an all-zero dy
    wg = to_dev(w.reshape(-1))
    so, S = oracle.scatter_combine(yo, dtype, ro, layout, cap, weights=w.reshape(-1), with_scale=True)
    assert_close(to_host(peg.scatter_combine(yg, rg, weights=wg)), so, S, dtype, "combine")
    yr = W.expert_tensor_rows(rng, R, H, dtype, used_rows=rows[rows >= 0])
    yrg = to_dev(yr, dtype)
    gg = to_dev(grad, dtype)
    wo, WS = oracle.wgrad(yr, grad, dtype, ro, layout, cap, with_scale=True)
    assert_close(to_host(peg.wgrad(yrg, gg, rg)), wo, WS, W.F32, "wgrad")
    check_combine_backward(yrg, yr, grad, gg, w, wg, ro, rg, layout, cap, dtype, R)


def _draw_aux(seed):
    rng = np.random.default_rng(5000 + seed)
    E = int(rng.choice([1, 2, 5, 8, 16, 64, 100, 256, 1024]))
    K = int(min(E, rng.choice([1, 2, 3, 8, 16])))
    T = int(rng.choice([0, 1, 9, 500, 3000]))
    return rng, T, K, E


@pytest.mark.parametrize("seed", OTHER_SEEDS)
def test_random_compaction_router_windows(seed):
    """Compaction (and its backward), router gating alone and fused with
    route_prep, and routing into row windows, at one random shape each."""
    rng, T, K, E = _draw_aux(seed)
    print(f"[random aux] seed {seed}: T{T} K{K} E{E}", flush=True)
    # compaction of a dense map with 0..max routes per row (max can exceed topk)
    dtype = int(rng.choice([W.F32, W.BF16, W.F16]))
    rmap = W.routing_map_rows(rng, T, E, int(min(E, K + rng.integers(0, 3))))
    probs = W.normal(rng, (T, E), dtype)
    po, re = oracle.routing_map_compact(probs, dtype, rmap, K)
    pg, rg_ = peg.routing_map_compact(to_dev(probs, dtype), to_dev(rmap), K)
    bits_equal(to_host(rg_), re, "route_experts")
    bits_equal(to_host(pg), po, "probs_out")
    gco = rng.standard_normal((T, K)).astype(np.float32)
    bits_equal(to_host(peg.routing_map_compact_backward(to_dev(gco), rg_, E)),
               oracle.routing_map_compact_backward(gco, re, E), "compaction backward")
    # router gating: selection bit for bit, weights within the router tolerance
    from test_gpu_router import check_weights
    logits = (rng.standard_normal((T, E)) * 3).astype(np.float32)
    gating = int(rng.choice([peg.SOFTMAX, peg.SIGMOID]))
    norm = bool(rng.integers(0, 2))
    to, wo = oracle.router_topk(logits, W.F32, K, gating, norm)
    tg, wg = peg.router_topk(to_dev(logits), K, gating=gating, normalize=norm)
    bits_equal(to_host(tg), to, "router top_experts")
    check_weights(to_host(wg), wo, "router weights")
    cap = int(rng.integers(1, 2 * max(1, T * K // E) + 2))
    rf, tf, wf = peg.route_prep_logits(to_dev(logits), K, capacity=cap, gating=gating, normalize=norm)
    bits_equal(to_host(tf), to, "fused top_experts")
    check_weights(to_host(wf), wo, "fused weights")
    ro = oracle.route_prep(to, E)
    bits_equal(to_host(rf.indices), ro.indices, "fused indices")
    bits_equal(to_host(rf.bins), ro.bins, "fused bins")
    bits_equal(to_host(rf.slot_row), oracle.assignment_rows(ro, W.BINNED, cap), "fused slot_row")
    # row windows of the same routing
    base = rng.integers(0, 5000, size=E).astype(np.int32)
    limit = (base + rng.integers(0, 2 * max(1, T * K // E) + 2, size=E)).astype(np.int32)
    rw = peg.route_prep_windows(to_dev(to), E, to_dev(base), to_dev(limit))
    bits_equal(to_host(rw.indices), ro.indices, "windows indices")
    bits_equal(to_host(rw.slot_row), oracle.assignment_rows_windows(ro, base, limit), "windows slot_row")
