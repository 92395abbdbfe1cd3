"""GPU parity of the router top-k gating (peg_router_topk) against the oracle.

Selection (top_experts) is compared bit for bit. Weights are float32 values
computed in fp32 on the GPU and in fp64 (rounded once) by the oracle; the
bound is
  |gpu - oracle| <= 1e-5 * |oracle| + 1e-30,
i.e. the fp32 relative tolerance used for every fp32 output here, plus an
absolute floor below which fp32 exp underflows (a probability under 1e-30
is zero to both). The fp32 evaluation error it has to cover: the rounding of
(score - max) scaled by its size (|score - max| * 2^-24 relative), the
hardware exponential's error (about (|x| * log2(e) + 1) * 2^-23 relative), a
sum of up to 1024 terms in a tree of depth <= 22, and two divisions: under
6e-6 for score gaps below 40. NaN must appear at the same places on both
sides (rows whose formulas give NaN).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import padded_expert_gather_amd as peg
import workloads as W
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

RTOL, AFLOOR = 1e-5, 1e-30


def check_weights(gpu, want, what):
    g = np.asarray(gpu, np.float64)
    o = np.asarray(want, np.float64)
    assert np.array_equal(np.isnan(g), np.isnan(o)), f"{what}: NaN at different places"
    fin = ~np.isnan(o)
    err = np.abs(g[fin] - o[fin])
    bound = RTOL * np.abs(o[fin]) + AFLOOR
    bad = err > bound
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError(f"{what}: {int(bad.sum())} weights out of tolerance; e.g. gpu={g[fin][i]!r} "
                             f"oracle={o[fin][i]!r}")


def scores(rng, T, E, kind):
    """Router scores [T, E] float32 of one of several kinds."""
    if kind == "normal":
        return (rng.standard_normal((T, E)) * 3).astype(np.float32)
    if kind == "ties":  # small integers: many exact ties
        return rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    if kind == "special":  # ties plus NaN, +-inf, signed zeros; a NaN row and a -inf row
        a = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
        sp = np.array([0.0, -0.0, np.inf, -np.inf, np.nan], np.float32)
        pick = rng.random((T, E)) < 0.2
        a[pick] = sp[rng.integers(0, len(sp), size=int(pick.sum()))]
        if T > 2:
            a[0] = np.nan
            a[1] = -np.inf
        return a
    if kind == "offset":  # large magnitudes: softmax needs the max shift, and renormalised
        # sigmoid of scores near -600 needs its common factor taken out in fp32
        return (rng.standard_normal((T, E)) * 2 + rng.choice([-600.0, -95.0, 300.0, 1e4], size=(T, 1))).astype(np.float32)
    raise ValueError(kind)


CASES = []
for E, Ks in [(1, (1,)), (3, (1, 3)), (8, (1, 2, 8)), (13, (4,)), (16, (2, 16)), (33, (6,)), (64, (8, 64)),
              (65, (8,)), (128, (8,)), (200, (10,)), (256, (8, 256)), (500, (3,)), (1024, (8, 1024))]:
    for K in Ks:
        CASES.append((E, K))


@pytest.mark.parametrize("E,K", CASES, ids=[f"E{e}-K{k}" for e, k in CASES])
def test_router_edge(E, K):
    print(f"[router] E{E} K{K}", flush=True)
    rng = np.random.default_rng(1000 * E + K)
    T = 61 if E * K < 100000 else 9
    for kind in ("normal", "ties", "special", "offset"):
        base = scores(rng, T, E, kind)
        for dtype in (W.F32, W.BF16, W.F16):
            lg = W.cast_from_f32(base, dtype)
            lgd = to_dev(lg, dtype)
            for gating in (peg.SOFTMAX, peg.SIGMOID):
                for norm in (True, False):
                    top_o, w_o = oracle.router_topk(lg, dtype, K, gating=gating, normalize=norm)
                    top_g, w_g = peg.router_topk(lgd, K, gating=gating, normalize=norm)
                    what = f"E{E} K{K} {kind} dt{dtype} g{gating} n{int(norm)}"
                    assert np.array_equal(to_host(top_g), top_o), f"{what}: top_experts differ"
                    check_weights(to_host(w_g), w_o, what)


def test_router_empty_and_single_token():
    lg = torch.empty((0, 8), dtype=torch.float32, device="cuda:0")
    top, w = peg.router_topk(lg, 2)
    assert top.shape == (0, 2) and w.shape == (0, 2)
    one = np.array([[0.5, 2.0, 2.0, -1.0]], np.float32)
    top, w = peg.router_topk(to_dev(one), 2)
    assert to_host(top).tolist() == [[1, 2]]  # tie at 2.0: lower id first
    assert to_host(w).tolist() == [[0.5, 0.5]]


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_router_workloads(cid):
    """The workloads' router scores at full size: the GPU gating equals the
    oracle's, and its routing equals the workload's own (numpy) routing."""
    print(f"[router] workload {cid}", flush=True)
    wl = W.config(cid, 0, with_rows=False)
    top_o, w_o = oracle.router_topk(wl.logits, W.F32, wl.K)
    top_g, w_g = peg.router_topk(to_dev(wl.logits), wl.K)
    assert np.array_equal(to_host(top_g), top_o)
    check_weights(to_host(w_g), w_o, f"workload {cid}")
    assert np.array_equal(top_o, wl.top_experts)
    sig_o = oracle.router_topk(wl.logits, W.F32, wl.K, gating=oracle.SIGMOID)
    sig_g = peg.router_topk(to_dev(wl.logits), wl.K, gating=peg.SIGMOID)
    assert np.array_equal(to_host(sig_g[0]), sig_o[0])
    check_weights(to_host(sig_g[1]), sig_o[1], f"workload {cid} sigmoid")


def test_router_feeds_route_prep():
    """Gating output drives route_prep directly on the device: same routing
    arrays as the oracle's route_prep of the oracle's gating."""
    wl = W.config(2, 1, with_rows=False)
    top_g, _ = peg.router_topk(to_dev(wl.logits), wl.K)
    rg = peg.route_prep(top_g, wl.E, pad_multiple=wl.pad_multiple)
    top_o, _ = oracle.router_topk(wl.logits, W.F32, wl.K)
    ro = oracle.route_prep(top_o, wl.E, pad_multiple=wl.pad_multiple)
    assert np.array_equal(to_host(rg.indices), ro.indices)
    assert np.array_equal(to_host(rg.padded_bins), ro.padded_bins)
    assert math.isclose(float(ro.n), wl.T * wl.K)


FUSED = [  # (T, E, K, layout, capacity or multiple, score kind)
    (0, 8, 2, W.BINNED, 4, "normal"),
    (1, 8, 2, W.PADDED, 4, "normal"),
    (4096, 8, 2, W.PADDED, 128, "normal"),      # 32 tiles of 256 ids
    (1000, 8, 3, W.BINNED, 300, "ties"),        # K does not divide the tile: tokens straddle tiles
    (777, 13, 5, W.PADDED, 8, "special"),
    (3000, 64, 8, W.BINNED, 300, "normal"),
    (20000, 8, 2, W.BINNED, 4000, "ties"),
    (8192, 256, 8, W.PADDED, 128, "normal"),
    (4096, 1024, 8, W.PADDED, 2, "normal"),      # expert x tile table too large: separate scan launch
    (2000, 1, 1, W.BINNED, 2000, "normal"),
]


@pytest.mark.parametrize("T,E,K,layout,cm,kind", FUSED,
                         ids=[f"T{c[0]}-E{c[1]}-K{c[2]}-{'bin' if c[3] == W.BINNED else 'pad'}" for c in FUSED])
def test_route_prep_logits(T, E, K, layout, cm, kind):
    """Gating fused with route_prep: gating outputs identical to
    peg_router_topk's; routing arrays identical to the oracle's route_prep of
    the oracle's gating (bit for bit); weights within the gating tolerance."""
    print(f"[fused] T{T} E{E} K{K} layout{layout} {kind}", flush=True)
    rng = np.random.default_rng(T + 7 * E + K)
    lg = scores(rng, T, E, kind) if T > 0 else np.zeros((0, E), np.float32)
    for gating in (peg.SOFTMAX, peg.SIGMOID):
        lgd = to_dev(lg)
        kw = dict(capacity=cm) if layout == W.BINNED else dict(pad_multiple=cm)
        rg, top_g, w_g = peg.route_prep_logits(lgd, K, gating=gating, **kw)
        top_s, w_s = peg.router_topk(lgd, K, gating=gating)
        assert np.array_equal(to_host(top_g), to_host(top_s)), "fused experts != router_topk"
        assert np.array_equal(to_host(w_g).view(np.uint32), to_host(w_s).view(np.uint32)), "fused weights"
        top_o, w_o = oracle.router_topk(lg, W.F32, K, gating=gating)
        assert np.array_equal(to_host(top_g), top_o)
        check_weights(to_host(w_g), w_o, "fused weights vs oracle")
        ro = oracle.route_prep(top_o, E, pad_multiple=cm if layout == W.PADDED else None)
        assert np.array_equal(to_host(rg.indices), ro.indices)
        assert np.array_equal(to_host(rg.bin_ids), ro.bin_ids)
        assert np.array_equal(to_host(rg.tokens_per_expert), ro.tokens_per_expert)
        assert np.array_equal(to_host(rg.bins), ro.bins)
        if layout == W.PADDED:
            assert np.array_equal(to_host(rg.padded_bins), ro.padded_bins)
        cap = cm if layout == W.BINNED else None
        assert np.array_equal(to_host(rg.slot_row), oracle.assignment_rows(ro, layout, cap))
