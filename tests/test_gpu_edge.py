"""GPU parity on the edge-case matrix (HIP library vs CPU oracle).

Cases follow the verification lists of the routing skill pages ("Build
Triton-Ascend Binned MoE Routing" and "... Padded MoE Routing", section
Verification): empty experts, expert overflow, exact capacity, several
experts inside one tile, TOP_K 1/2/4/8, unaligned hidden sizes, counts at
m-1/m/m+1, weighted scatter, large token counts; plus the degenerate cases
(T = 0, E = 1, K = E, C = 1, ample C, m = 1, all routes to one expert,
tokens whose routes are all dropped or absent, bit patterns that a float
path would alter, caller-supplied over-padded bins, a too-small output).

Integer outputs and gathers are compared bit for bit; combine and wgrad
within the tolerance rule of tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import oracle
import padded_expert_gather_amd as peg
import workloads as W
from gpu_util import DEV, assert_close, bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu


def _counts_routing(rng, counts, K=1):
    """K = 1 routing whose expert counts are exactly ``counts``, shuffled."""
    top = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    rng.shuffle(top)
    return top.reshape(-1, K)


def _case(name, T, K, E, H, dtype, layout, cap=None, m=None, none_frac=0.0, skew=0.0, one_expert=None, top=None,
          seed=0):
    return pytest.param(dict(T=T, K=K, E=E, H=H, dtype=dtype, layout=layout, cap=cap, m=m, none_frac=none_frac,
                             skew=skew, one_expert=one_expert, top=top, seed=seed), id=name)


B, P = W.BINNED, W.PADDED
CASES = [
    _case("empty_experts_f32", 64, 2, 8, 40, W.F32, B, cap=16, skew=1.0),
    _case("overflow_bf16", 128, 2, 4, 64, W.BF16, B, cap=20),
    _case("exact_capacity", 32, 2, 4, 48, W.BF16, B, cap=16,
          top=np.array([[(2 * t) % 4, (2 * t + 1) % 4] for t in range(32)], np.int32)),
    _case("topk1_padded", 100, 1, 16, 96, W.BF16, P, m=8),
    _case("topk4_binned", 100, 4, 16, 96, W.BF16, B, cap=20),
    _case("topk8_padded", 100, 8, 16, 96, W.F16, P, m=16),
    _case("topk8_binned_none", 77, 8, 32, 72, W.BF16, B, cap=12, none_frac=0.3),
    _case("h1_f32", 50, 2, 4, 1, W.F32, B, cap=20),
    _case("h3_f32_padded", 50, 2, 4, 3, W.F32, P, m=4),
    _case("h250_f32", 512, 2, 8, 250, W.F32, B, cap=128),
    _case("h4095_bf16", 40, 2, 4, 4095, W.BF16, P, m=8),
    _case("h4100_bf16", 40, 2, 4, 4100, W.BF16, B, cap=16),
    _case("h3_f16", 33, 3, 5, 3, W.F16, P, m=2),
    _case("large_T", 20000, 2, 8, 64, W.BF16, P, m=128),
    _case("many_experts_per_tile", 1500, 2, 64, 32, W.BF16, B, cap=40),
    _case("E1_identity", 64, 1, 1, 128, W.BF16, B, cap=64),
    _case("K_eq_E", 40, 4, 4, 64, W.F32, P, m=8),
    _case("C1", 60, 2, 6, 32, W.BF16, B, cap=1),
    _case("C_ample", 60, 2, 6, 32, W.BF16, B, cap=200),
    _case("m1_plain_permute", 90, 2, 6, 64, W.BF16, P, m=1),
    _case("all_one_expert_binned", 70, 1, 8, 64, W.BF16, B, cap=30, one_expert=3),
    _case("all_one_expert_padded", 70, 2, 8, 64, W.BF16, P, m=32, one_expert=5),
    _case("tokens_all_dropped", 200, 2, 4, 64, W.BF16, B, cap=10),
    _case("rows_all_none", 50, 2, 4, 64, W.BF16, P, m=4, none_frac=0.7),
    _case("padded_no_rows", 5, 2, 4, 64, W.BF16, P, m=4, none_frac=1.0),  # a padded tensor of 0 rows
    _case("binned_no_routes", 5, 2, 4, 64, W.F16, B, cap=3, none_frac=1.0),
    _case("E300_items4", 900, 2, 300, 16, W.BF16, P, m=4, skew=0.01),
    _case("E1024_items2", 1500, 2, 1024, 16, W.BF16, B, cap=3),
    _case("E1024_scan_launch", 10000, 2, 1024, 8, W.BF16, P, m=2),
    _case("E200_merged_bases", 3000, 8, 200, 8, W.BF16, P, m=16, none_frac=0.1),
    _case("E64_tile4096", 9000, 8, 64, 8, W.BF16, B, cap=1000, skew=0.05),
    _case("tiled_items1_12k", 6000, 2, 8, 8, W.BF16, P, m=64, none_frac=0.05),
    _case("small_staged_6k", 3000, 2, 8, 8, W.BF16, P, m=64, none_frac=0.05),
    _case("tiled_8192", 4096, 2, 8, 8, W.BF16, P, m=128),
    _case("tiled_E32", 5000, 4, 32, 8, W.BF16, B, cap=700, skew=0.05),
    _case("tiled_E17_none", 9000, 2, 17, 8, W.BF16, P, m=16, none_frac=0.1),
    _case("tiled_32768", 16384, 2, 8, 8, W.BF16, B, cap=5000, skew=0.3),
    _case("tiled_32770", 16385, 2, 8, 8, W.BF16, P, m=64),
    _case("small_unstaged", 4000, 2, 64, 8, W.BF16, B, cap=100),
    _case("tiled_E16_ragged", 5001, 3, 16, 24, W.BF16, P, m=8, none_frac=0.1, skew=0.2),
    _case("tiled_E1", 10000, 1, 1, 16, W.BF16, B, cap=5000),
    _case("tiled_16384_E13", 8192, 2, 13, 8, W.BF16, B, cap=900, skew=0.5),
    _case("tiled_16386_E16", 8193, 2, 16, 8, W.BF16, P, m=4),
    _case("tile_2048", 1024, 2, 8, 16, W.BF16, B, cap=300),
    _case("tile_2049", 683, 3, 8, 16, W.BF16, P, m=8),
    _case("tile_2047", 2047, 1, 8, 16, W.BF16, B, cap=300),
    _case("K12_binned", 300, 12, 16, 72, W.BF16, B, cap=150, skew=0.1),
    _case("K16_padded_f32", 200, 16, 32, 40, W.F32, P, m=8, none_frac=0.2),
    _case("K9_f16", 150, 9, 12, 24, W.F16, B, cap=90),
    _case("H16384_bf16", 64, 2, 4, 16384, W.BF16, P, m=16),
    _case("K4_long_rows", 300, 4, 16, 4100, W.BF16, B, cap=100, skew=0.1),
    _case("K3_long_rows_f32", 200, 3, 8, 1030, W.F32, P, m=8, none_frac=0.1),
    _case("T0_binned", 0, 2, 4, 32, W.BF16, B, cap=4),
    _case("T0_padded", 0, 2, 4, 32, W.BF16, P, m=4),
]


def _setup(c):
    rng = np.random.default_rng(c["seed"])
    T, K, E, H, dtype = c["T"], c["K"], c["E"], c["H"], c["dtype"]
    if c["top"] is not None:
        top = c["top"]
        w = (rng.random(top.shape, dtype=np.float32) + 0.1).astype(np.float32)
    else:
        top, w = W.random_routing(rng, T, K, E, none_frac=c["none_frac"], skew=c["skew"],
                                  one_expert=c["one_expert"])
    x = W.normal(rng, (T, H), dtype)
    grad = W.normal(rng, (T, H), dtype)
    return rng, top, w, x, grad


def _gpu_prep(top, c):
    if c["layout"] == W.BINNED:
        return peg.route_prep(to_dev(top), c["E"], capacity=c["cap"])
    return peg.route_prep(to_dev(top), c["E"], pad_multiple=c["m"])


def _gather(xg, rg, c, **kw):
    return peg.gather_binned(xg, rg, **kw) if c["layout"] == W.BINNED else peg.gather_padded(xg, rg, **kw)


@pytest.mark.parametrize("c", CASES)
def test_edge_case(c):
    print(f"[edge] {c['T']}x{c['H']} E{c['E']} K{c['K']} dtype{c['dtype']} layout{c['layout']}", flush=True)
    rng, top, w, x, grad = _setup(c)
    E, layout, cap, dtype = c["E"], c["layout"], c["cap"], c["dtype"]
    # --- route_prep: bit-exact
    ro = oracle.route_prep(top, E, pad_multiple=c["m"])
    rg = _gpu_prep(top, c)
    bits_equal(to_host(rg.indices), ro.indices, "indices")
    bits_equal(to_host(rg.bin_ids), ro.bin_ids, "bin_ids")
    bits_equal(to_host(rg.tokens_per_expert), ro.tokens_per_expert, "tokens_per_expert")
    bits_equal(to_host(rg.bins), ro.bins, "bins")
    if c["m"] is not None:
        bits_equal(to_host(rg.padded_bins), ro.padded_bins, "padded_bins")
    rows = oracle.assignment_rows(ro, layout, cap)
    bits_equal(to_host(rg.slot_row), rows, "slot_row")
    R = oracle.expert_rows(ro, layout, cap)
    # --- gathers: bit-exact, with the map and with the rebuild from sorted arrays
    xg = to_dev(x, dtype)
    yo = oracle.gather(x, ro, layout, cap)
    yg = _gather(xg, rg, c)
    bits_equal(to_host(yg), yo, "gather")
    bits_equal(to_host(_gather(xg, rg, c, use_slot_row=False)), yo, "gather (rebuilt map)")
    if c["T"] == 0:
        return
    wg = to_dev(w.reshape(-1))
    # --- combine on y = gather(x), weighted and unweighted
    so, S = oracle.scatter_combine(yo, dtype, ro, layout, cap, weights=w.reshape(-1), with_scale=True)
    assert_close(to_host(peg.scatter_combine(yg, rg, weights=wg)), so, S, dtype, "combine(gather(x))")
    so1, S1 = oracle.scatter_combine(yo, dtype, ro, layout, cap, with_scale=True)
    assert_close(to_host(peg.scatter_combine(yg, rg)), so1, S1, dtype, "combine unweighted")
    # --- combine and wgrad on an independent y whose unused rows are NaN
    yr = W.expert_tensor_rows(rng, R, c["H"], dtype, used_rows=rows[rows >= 0])
    yrg = to_dev(yr, dtype)
    so2, S2 = oracle.scatter_combine(yr, dtype, ro, layout, cap, weights=w.reshape(-1), with_scale=True)
    assert_close(to_host(peg.scatter_combine(yrg, rg, weights=wg)), so2, S2, dtype, "combine(y_rand)")
    assert_close(to_host(peg.scatter_combine(yrg, rg, weights=wg, use_slot_row=False)), so2, S2, dtype,
                 "combine(y_rand) rebuilt map")
    gg = to_dev(grad, dtype)
    wo, WS = oracle.wgrad(yr, grad, dtype, ro, layout, cap, with_scale=True)
    assert_close(to_host(peg.wgrad(yrg, gg, rg)), wo, WS, W.F32, "wgrad(y_rand)")
    assert_close(to_host(peg.wgrad(yrg, gg, rg, use_slot_row=False)), wo, WS, W.F32, "wgrad rebuilt map")
    wo2, WS2 = oracle.wgrad(yo, grad, dtype, ro, layout, cap, with_scale=True)
    assert_close(to_host(peg.wgrad(yg, gg, rg)), wo2, WS2, W.F32, "wgrad(gather(x))")
    # --- backward of the combine with wgrad (dout = grad)
    check_combine_backward(yrg, yr, grad, gg, w, wg, ro, rg, layout, cap, dtype, R)
    # --- the validator accepts what route_prep built
    assert int(peg.validate_routing(rg, n_indices=ro.n).item()) == 0


def check_combine_backward(yrg, yr, grad, gg, w, wg, ro, rg, layout, cap, dtype, R):
    """dy = w * dout at kept rows, zero elsewhere (tolerance: one rounding of
    a product); dy without weights = gather(dout) bit for bit; the fused
    wgrad equals the oracle's and, bit for bit, the stand-alone kernel's."""
    dyo = oracle.combine_backward_dy(grad, dtype, ro, layout, cap, weights=w.reshape(-1))
    dyg, wgb = peg.combine_backward(yrg, gg, rg, weights=wg, dy_rows=R)
    assert_close(to_host(dyg), dyo, np.abs(W.to_f32(dyo, dtype).astype(np.float64)), dtype, "combine backward dy")
    wo, WS = oracle.wgrad(yr, grad, dtype, ro, layout, cap, with_scale=True)
    assert_close(to_host(wgb), wo, WS, W.F32, "combine backward wgrad")
    bits_equal(to_host(wgb), to_host(peg.wgrad(yrg, gg, rg)), "fused wgrad == wgrad kernel")
    dyp, _ = peg.combine_backward(yrg, gg, rg, dy_rows=R, use_slot_row=False)
    bits_equal(to_host(dyp), oracle.gather(grad, ro, layout, cap), "unweighted combine backward == gather")


def test_gather_preserves_bit_patterns():
    """NaN payloads, -0.0, infinities and subnormals move unchanged."""
    rng = np.random.default_rng(3)
    pats = np.array([0x7FC1, 0x8000, 0x0001, 0xFF80, 0x7F81, 0x807F, 0x0000, 0xFFFF], np.uint16)
    T, H, E, K = 48, 24, 4, 2
    x = rng.choice(pats, size=(T, H)).astype(np.uint16)
    top, _ = W.random_routing(rng, T, K, E)
    for layout, cap, m in ((W.BINNED, 20, None), (W.PADDED, None, 8)):
        ro = oracle.route_prep(top, E, pad_multiple=m)
        rg = peg.route_prep(to_dev(top), E, capacity=cap, pad_multiple=m)
        xg = to_dev(x, W.BF16)
        yg = peg.gather_binned(xg, rg) if layout == W.BINNED else peg.gather_padded(xg, rg)
        bits_equal(to_host(yg), oracle.gather(x, ro, layout, cap), "bit patterns")


def test_identity_e1_k1():
    """E = 1, K = 1, C = T: gather reproduces x and combine(gather(x)) too."""
    rng = np.random.default_rng(4)
    T, H = 300, 520
    x = W.normal(rng, (T, H), W.BF16)
    top = np.zeros((T, 1), np.int32)
    xg = to_dev(x, W.BF16)
    for kw in (dict(capacity=T), dict(pad_multiple=1)):
        rg = peg.route_prep(to_dev(top), 1, **kw)
        yg = peg.gather_binned(xg, rg) if "capacity" in kw else peg.gather_padded(xg, rg)
        bits_equal(to_host(yg), x, "identity gather")
        bits_equal(to_host(peg.scatter_combine(yg, rg)), x, "identity combine")


def test_over_padded_bins_and_small_output():
    """Caller-supplied padded_bins with larger segments than the minimal
    round-up (accepted), and an output buffer smaller than padded_bins[-1]
    (rows past it skipped, flag raised, nothing written past the buffer)."""
    rng = np.random.default_rng(5)
    T, K, E, H = 120, 2, 6, 40
    top, w = W.random_routing(rng, T, K, E, skew=0.3)
    x = W.normal(rng, (T, H), W.BF16)
    ro = oracle.route_prep(top, E, pad_multiple=4)
    ro.padded_bins = (ro.padded_bins + 5 * np.arange(1, E + 1)).astype(np.int32)  # 5 extra rows per expert
    rg = peg.route_prep(to_dev(top), E, pad_multiple=4)
    rg.padded_bins = to_dev(ro.padded_bins)
    R = int(ro.padded_bins[-1])
    xg = to_dev(x, W.BF16)
    yo = oracle.gather(x, ro, W.PADDED)
    yg = peg.gather_padded(xg, rg, out_rows=R, use_slot_row=False)
    bits_equal(to_host(yg), yo, "over-padded gather")
    so, S = oracle.scatter_combine(yo, W.BF16, ro, W.PADDED, weights=w.reshape(-1), with_scale=True)
    assert_close(to_host(peg.scatter_combine(yg, rg, weights=to_dev(w.reshape(-1)), use_slot_row=False)), so, S,
                 W.BF16, "over-padded combine")
    assert int(peg.validate_routing(rg, n_indices=ro.n).item()) == 0
    # too-small output: guard rows past it with a sentinel region
    small = R // 2
    buf = torch.full((small + 7, H), -3.0, dtype=torch.bfloat16, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    peg.gather_padded(xg, rg, out=buf[:small], err_flag=flag, use_slot_row=False)
    torch.cuda.synchronize()
    assert int(flag.item()) & peg.FLAG_OUT_ROWS
    bits_equal(to_host(buf[:small]), yo[:small], "truncated gather")
    assert bool((buf[small:] == -3.0).all()), "rows past out_rows were written"


def test_validate_flags_match_oracle():
    """Planted violations of each guardrail give the oracle's flags exactly."""
    rng = np.random.default_rng(6)
    T, K, E = 40, 2, 5
    top, _ = W.random_routing(rng, T, K, E, none_frac=0.1)
    ro = oracle.route_prep(top, E, pad_multiple=4)
    rg = peg.route_prep(to_dev(top), E, pad_multiple=4)
    n = ro.n
    variants = []
    b = ro.bins.copy(); b[1], b[2] = b[2], b[1] - 1
    variants.append(("bins", dict(bins=b), -1))
    variants.append(("total", {}, n - 1))
    bid = ro.bin_ids.copy(); bid[0] = 4
    variants.append(("bin_ids", dict(bin_ids=bid), n))
    pb = ro.padded_bins.copy(); pb[0] = 0
    variants.append(("padded", dict(padded_bins=pb), n))
    idx = ro.indices.copy(); idx[1] = idx[0]
    variants.append(("dup", dict(indices=idx), n))
    idx2 = ro.indices.copy(); idx2[2] = T * K + 5
    variants.append(("range", dict(indices=idx2), n))
    variants.append(("valid", {}, n))
    for name, kw, nn in variants:
        arrs = dict(indices=ro.indices, bin_ids=ro.bin_ids, bins=ro.bins, padded_bins=ro.padded_bins)
        arrs.update(kw)
        want = oracle.validate_routing(arrs["indices"], arrs["bin_ids"], arrs["bins"], arrs["padded_bins"], T, K,
                                       E, nn)
        got = peg.validate_routing(rg, n_indices=nn, **{k: to_dev(v) for k, v in arrs.items()})
        assert int(got.item()) & 0xFFFFFFFF == want, name
        if name == "valid":
            assert want == 0


@pytest.mark.parametrize("E,topk,pdt", [(5, 3, W.F32), (64, 8, W.BF16), (256, 8, W.F32), (300, 4, W.F16),
                                        (1024, 16, W.BF16), (8, 8, W.F32), (130, 1, W.F32)])
def test_compaction(E, topk, pdt):
    print(f"[compact] E{E} topk{topk} dtype{pdt}", flush=True)
    rng = np.random.default_rng(E + topk)
    T = 333
    rmap = W.routing_map_rows(rng, T, E, min(E, topk + 3))  # some rows exceed topk
    rmap[0] = 0
    rmap[1] = 1  # every expert routed
    probs = W.normal(rng, (T, E), pdt)
    po, io = oracle.routing_map_compact(probs, pdt, rmap, topk)
    pg, ig = peg.routing_map_compact(to_dev(probs, pdt), to_dev(rmap), topk)
    bits_equal(to_host(ig), io, "route_experts")
    bits_equal(to_host(pg), po, "probs_out")
    # bool map accepted too
    pg2, ig2 = peg.routing_map_compact(to_dev(probs, pdt), to_dev(rmap).bool(), topk)
    bits_equal(to_host(ig2), io, "route_experts (bool map)")
    g = rng.standard_normal((T, topk)).astype(np.float32)
    do = oracle.routing_map_compact_backward(g, io, E)
    dg = peg.routing_map_compact_backward(to_dev(g), ig, E)
    bits_equal(to_host(dg), do, "compaction backward")


def test_binding_refuses_bad_buffers():
    """The binding checks every buffer it can check without a sync before
    anything is enqueued: output sizes, expert-tensor rows of the binned
    layout, dy's row length, devices."""
    rng = np.random.default_rng(8)
    T, K, E, H, C = 64, 2, 4, 32, 40
    top, w = W.random_routing(rng, T, K, E)
    rg = peg.route_prep(to_dev(top), E, capacity=C)
    xg = to_dev(W.normal(rng, (T, H), W.BF16), W.BF16)
    y = peg.gather_binned(xg, rg)
    with pytest.raises(ValueError):
        peg.scatter_combine(y[: E * C - 1], rg)                       # fewer than E*C rows
    with pytest.raises(ValueError):
        peg.wgrad(y, xg, rg, out=torch.empty(T * K - 1, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        peg.combine_backward(y, xg, rg, dy=torch.empty((E * C, H + 8), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        peg.combine_backward(y, xg, rg, wgrad_out=torch.empty(3, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        peg.gather_binned(xg.reshape(-1), rg)                         # x not [T, H]
    probs = torch.rand((T, E), dtype=torch.float32, device=DEV)
    rmap = torch.ones((T, E), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        peg.routing_map_compact(probs, rmap, 2, probs_out=torch.empty((T, 1), dtype=torch.float32, device=DEV))
    idx = torch.zeros((T, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        peg.routing_map_compact_backward(torch.zeros((T, 2), device=DEV), idx, E,
                                         out=torch.empty((T, E - 1), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        peg.validate_routing(rg, indices=rg.indices[:-1])
    torch.cuda.synchronize()
    assert int(peg.validate_routing(rg).item()) == 0                   # the routing itself is intact


@pytest.mark.parametrize("K", [2, 4])
@pytest.mark.parametrize("layout", [W.BINNED, W.PADDED])
def test_combine_backward_rows_past_layout(layout, K):
    """dy with more rows than the layout's R: the kept rows and gaps as
    usual, and every row of [R, dy_rows) zero (the buffer starts as a
    sentinel); nothing is written past dy_rows. K = 2 runs the fused pass,
    K = 4 the dy gather followed by the wgrad kernel."""
    print(f"[backward past layout] layout{layout} K{K}", flush=True)
    rng = np.random.default_rng(11 + layout + 7 * K)
    T, E, H, C, m = 150, 6, 72, 20 * K, 8
    top, w = W.random_routing(rng, T, K, E, skew=0.3, none_frac=0.1)
    grad = W.normal(rng, (T, H), W.BF16)
    cap = C if layout == W.BINNED else None
    ro = oracle.route_prep(top, E, pad_multiple=m)
    rg = peg.route_prep(to_dev(top), E, capacity=cap, pad_multiple=None if cap else m)
    R = oracle.expert_rows(ro, layout, cap)
    extra = 37
    buf = torch.full((R + extra + 5, H), -7.0, dtype=torch.bfloat16, device=DEV)
    yr = W.expert_tensor_rows(rng, R, H, W.BF16, used_rows=oracle.assignment_rows(ro, layout, cap)[
        oracle.assignment_rows(ro, layout, cap) >= 0])
    gg = to_dev(grad, W.BF16)
    dyg, _ = peg.combine_backward(to_dev(yr, W.BF16), gg, rg, dy=buf[: R + extra], use_slot_row=True)
    dyo = oracle.combine_backward_dy(grad, W.BF16, ro, layout, cap, weights=None)
    bits_equal(to_host(dyg[:R]), dyo, "dy rows [0, R)")
    assert int(buf[R: R + extra].view(torch.int16).count_nonzero().item()) == 0, "rows [R, dy_rows) not zero"
    assert bool((buf[R + extra:] == -7.0).all()), "a row past dy_rows was written"


@pytest.mark.parametrize("empty", [False, True])
@pytest.mark.parametrize("K", [2, 4])
@pytest.mark.parametrize("layout", [W.BINNED, W.PADDED])
def test_combine_backward_short_dy(layout, K, empty):
    """dy with fewer rows than the layout's R (about half of them, or none):
    rows [0, dy_rows) as the oracle's (kept rows w * dout, gaps zero),
    nothing written at or past dy_rows, and wgrad still computed for the
    routes whose rows lie there (equal, bit for bit, to the wgrad
    kernel's)."""
    print(f"[backward short dy] layout{layout} K{K} empty{empty}", flush=True)
    rng = np.random.default_rng(40 + layout + 7 * K)
    T, E, H, C, m = 200, 5, 136, 30 * K, 8
    top, w = W.random_routing(rng, T, K, E, skew=0.3, none_frac=0.1)
    grad = W.normal(rng, (T, H), W.BF16)
    cap = C if layout == W.BINNED else None
    ro = oracle.route_prep(top, E, pad_multiple=m)
    rg = peg.route_prep(to_dev(top), E, capacity=cap, pad_multiple=None if cap else m)
    R = oracle.expert_rows(ro, layout, cap)
    rows = oracle.assignment_rows(ro, layout, cap)
    short = 0 if empty else R // 2 + 3
    assert 0 <= short < R and (rows >= short).any()
    yr = W.expert_tensor_rows(rng, R, H, W.BF16, used_rows=rows[rows >= 0])
    yrg, gg, wg = to_dev(yr, W.BF16), to_dev(grad, W.BF16), to_dev(w.reshape(-1))
    buf = torch.full((R, H), -7.0, dtype=torch.bfloat16, device=DEV)
    dyg, wgb = peg.combine_backward(yrg, gg, rg, weights=wg, dy=buf[:short], use_slot_row=True)
    dyo = oracle.combine_backward_dy(grad, W.BF16, ro, layout, cap, weights=w.reshape(-1))
    assert_close(to_host(dyg), dyo[:short], np.abs(W.to_f32(dyo[:short], W.BF16).astype(np.float64)), W.BF16,
                 "dy rows [0, dy_rows)")
    assert bool((buf[short:] == -7.0).all()), "a row at or past dy_rows was written"
    wo, WS = oracle.wgrad(yr, grad, W.BF16, ro, layout, cap, with_scale=True)
    assert_close(to_host(wgb), wo, WS, W.F32, "wgrad with a short dy")
    bits_equal(to_host(wgb), to_host(peg.wgrad(yrg, gg, rg)), "wgrad with a short dy == wgrad kernel")


def test_gather_padded_refuses_binned_routing():
    """A routing prepared for the binned layout (capacity and pad_multiple
    both given) carries padded_bins, but its slot_row holds binned rows:
    gather_padded refuses it, and with use_slot_row=False rebuilds the
    padded map and matches the oracle's padded gather."""
    rng = np.random.default_rng(12)
    T, K, E, H, C, m = 90, 2, 5, 48, 12, 8
    top, _ = W.random_routing(rng, T, K, E, skew=0.5)
    x = W.normal(rng, (T, H), W.BF16)
    rg = peg.route_prep(to_dev(top), E, capacity=C, pad_multiple=m)
    xg = to_dev(x, W.BF16)
    with pytest.raises(ValueError):
        peg.gather_padded(xg, rg)
    ro = oracle.route_prep(top, E, pad_multiple=m)
    bits_equal(to_host(peg.gather_padded(xg, rg, use_slot_row=False)), oracle.gather(x, ro, W.PADDED),
               "padded gather of a binned routing, map rebuilt")
