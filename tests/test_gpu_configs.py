"""GPU parity on the five reference workloads at full size.

Workloads (workloads.config):
  1 binned f32  T512  H250  E8   K2 C128
  2 padded bf16 T4096 H4096 E8   K2 m128   (Mixtral-8x7B-shaped)
  3 binned bf16 T16384 H6144 E8  K2 C5120  (Mixtral-8x22B-shaped, Zipf skew)
  4 compaction + padded bf16 T8192 H7168 E256 K8 m128 (DeepSeek-V3-shaped)
  5 binned bf16 T32768 H3584 E64 K8 C4096  (Qwen2-MoE-57B-shaped, heavy skew)

Every index output is compared bit for bit in full. Gathers: full bit
comparison for 1-2; for 3-5 (seeds 0-4 at full width, and seeds 1-4 once
more with narrow rows) every kept row is checked against its token row
on the device, every other row is checked to be zero, and a row sample is
compared with the oracle. Combine / wgrad at 3-5: the oracle on every token
for seed 0 (y = gather(x), and an independent random y with NaN in unused
rows) and on sampled tokens for seeds 1-4, plus the closed forms on every
token ((sum of kept w) * x_t and <x_t, grad_t>, the latter in float64).
"""
import numpy as np
import pytest
import torch

import oracle
import padded_expert_gather_amd as peg
import workloads as W
from gpu_util import DEV, RTOL, assert_close, bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu


def _prep(wl):
    """Device and oracle routing for a workload (compaction first for 4)."""
    if wl.routing_map is not None:
        po, io = oracle.routing_map_compact(wl.probs, W.F32, wl.routing_map, wl.topk)
        pg, ig = peg.routing_map_compact(to_dev(wl.probs), to_dev(wl.routing_map), wl.topk)
        bits_equal(to_host(ig), io, "compaction route_experts")
        bits_equal(to_host(pg), po, "compaction probs")
        top_o, w_o, top_g, w_g = io, po, ig, pg
    else:
        top_o, w_o = wl.top_experts, wl.weights
        top_g, w_g = to_dev(wl.top_experts), to_dev(wl.weights)
    m = wl.pad_multiple if wl.layout == W.PADDED else None
    ro = oracle.route_prep(top_o, wl.E, pad_multiple=m)
    if wl.layout == W.BINNED:
        rg = peg.route_prep(top_g, wl.E, capacity=wl.capacity)
    else:
        rg = peg.route_prep(top_g, wl.E, pad_multiple=m)
    bits_equal(to_host(rg.indices), ro.indices, "indices")
    bits_equal(to_host(rg.bin_ids), ro.bin_ids, "bin_ids")
    bits_equal(to_host(rg.tokens_per_expert), ro.tokens_per_expert, "tokens_per_expert")
    bits_equal(to_host(rg.bins), ro.bins, "bins")
    if m is not None:
        bits_equal(to_host(rg.padded_bins), ro.padded_bins, "padded_bins")
    cap = wl.capacity if wl.layout == W.BINNED else None
    rows = oracle.assignment_rows(ro, wl.layout, cap)
    bits_equal(to_host(rg.slot_row), rows, "slot_row")
    return ro, rg, rows, cap, np.asarray(w_o, np.float32).reshape(-1), w_g.reshape(-1)


def _sample_tokens(rng, T, n=192):
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=min(n, T), replace=False)])).astype(np.int64)


@pytest.mark.parametrize("cid,seed", [(1, s) for s in range(5)] + [(2, s) for s in range(5)])
def test_small_configs_full(cid, seed):
    """Workloads 1 and 2, seeds 0-4: every output compared in full."""
    print(f"[config {cid} seed {seed}]", flush=True)
    wl = W.config(cid, seed)
    ro, rg, rows, cap, w_o, w_g = _prep(wl)
    xg = to_dev(wl.x, wl.dtype)
    yo = oracle.gather(wl.x, ro, wl.layout, cap)
    yg = peg.gather_binned(xg, rg) if wl.layout == W.BINNED else peg.gather_padded(xg, rg)
    bits_equal(to_host(yg), yo, "gather")
    so, S = oracle.scatter_combine(yo, wl.dtype, ro, wl.layout, cap, weights=w_o, with_scale=True)
    assert_close(to_host(peg.scatter_combine(yg, rg, weights=w_g)), so, S, wl.dtype, "combine")
    gg = to_dev(wl.grad, wl.dtype)
    wo, WS = oracle.wgrad(yo, wl.grad, wl.dtype, ro, wl.layout, cap, with_scale=True)
    assert_close(to_host(peg.wgrad(yg, gg, rg)), wo, WS, W.F32, "wgrad")
    rng = np.random.default_rng(100 + seed)
    R = yo.shape[0]
    yr = W.expert_tensor_rows(rng, R, wl.H, wl.dtype, used_rows=rows[rows >= 0])
    yrg = to_dev(yr, wl.dtype)
    so2, S2 = oracle.scatter_combine(yr, wl.dtype, ro, wl.layout, cap, weights=w_o, with_scale=True)
    assert_close(to_host(peg.scatter_combine(yrg, rg, weights=w_g)), so2, S2, wl.dtype, "combine(y_rand)")
    wo2, WS2 = oracle.wgrad(yr, wl.grad, wl.dtype, ro, wl.layout, cap, with_scale=True)
    assert_close(to_host(peg.wgrad(yrg, gg, rg)), wo2, WS2, W.F32, "wgrad(y_rand)")
    # backward of the combine with wgrad, upstream gradient = wl.grad
    dyo = oracle.combine_backward_dy(wl.grad, wl.dtype, ro, wl.layout, cap, weights=w_o)
    dyg, wgb = peg.combine_backward(yrg, gg, rg, weights=w_g, dy_rows=R)
    assert_close(to_host(dyg), dyo, np.abs(W.to_f32(dyo, wl.dtype).astype(np.float64)), wl.dtype, "backward dy")
    assert_close(to_host(wgb), wo2, WS2, W.F32, "backward wgrad")
    if cid == 1:
        assert sum(np.asarray(ro.tokens_per_expert) > wl.capacity) >= 1  # overflow present


def _check_gather_full(yg, xg, rows, K, what):
    kept = np.flatnonzero(rows >= 0)
    rk = torch.from_numpy(rows[kept].astype(np.int64)).to(DEV)
    tk = torch.from_numpy((kept // K).astype(np.int64)).to(DEV)
    a = yg.view(torch.int16)
    assert torch.equal(a[rk], xg.view(torch.int16)[tk]), f"{what}: a kept row differs from its token row"
    gap = torch.ones(yg.shape[0], dtype=torch.bool, device=DEV)
    gap[rk] = False
    assert int(a[gap].count_nonzero().item()) == 0, f"{what}: a gap row is not zero"
    return kept


@pytest.mark.parametrize("cid,seed", [(c, s) for s in range(5) for c in (3, 4, 5)])
def test_large_config(cid, seed):
    """Workloads 3-5, seeds 0-4, at full size."""
    print(f"[config {cid} seed {seed}] generating", flush=True)
    wl = W.config(cid, seed)
    ro, rg, rows, cap, w_o, w_g = _prep(wl)
    print(f"[config {cid}] routing ok; n={ro.n}", flush=True)
    if cid == 3:
        counts = np.asarray(ro.tokens_per_expert)
        assert int(np.sum(counts > wl.capacity)) == 2 and int(np.sum(counts == 0)) == 1
    rng = np.random.default_rng(1000 + cid + 100 * seed)
    xg = to_dev(wl.x, wl.dtype)
    gg = to_dev(wl.grad, wl.dtype)
    yg = peg.gather_binned(xg, rg) if wl.layout == W.BINNED else peg.gather_padded(xg, rg)
    R = yg.shape[0]
    assert R == oracle.expert_rows(ro, wl.layout, cap)
    kept = _check_gather_full(yg, xg, rows, wl.K, "gather")
    # oracle on a row sample: segment boundaries + random rows
    b = np.concatenate([[0], ro.padded_bins if wl.layout == W.PADDED else np.arange(1, wl.E + 1) * cap])
    sample = np.unique(np.concatenate([b[:-1], np.maximum(b[1:] - 1, 0), rng.choice(R, 1024, replace=False)]))
    sample = sample[(sample >= 0) & (sample < R)].astype(np.int64)
    yo_s = oracle.gather(wl.x, ro, wl.layout, cap, rows=sample)
    bits_equal(to_host(yg[torch.from_numpy(sample).to(DEV)]), yo_s, "gather sample")
    print(f"[config {cid}] gather ok", flush=True)

    # closed forms on every token, y = gather(x): the combine against
    # (sum of kept w) * x_t, wgrad against <x_t, grad_t> taken in float64
    keptmask = torch.from_numpy((rows >= 0).reshape(wl.T, wl.K)).to(DEV)
    wsum = torch.where(keptmask, w_g.reshape(wl.T, wl.K), torch.zeros((), device=DEV)).sum(1)
    xf = xg.float()
    sg = peg.scatter_combine(yg, rg, weights=w_g).float()
    want = wsum[:, None] * xf
    bound = RTOL[wl.dtype] * want.abs() + 1e-5 * (wsum.abs()[:, None] * xf.abs())
    assert bool(((sg - want).abs() <= bound).all()), "combine closed form"
    del sg, want, bound
    wgg = peg.wgrad(yg, gg, rg)
    prod = xg.double() * gg.double()
    dots = prod.sum(1)
    scale = prod.abs().sum(1)
    del prod
    wwant = torch.where(keptmask, dots[:, None], torch.zeros((), dtype=torch.float64, device=DEV))
    wbound = 1e-5 * wwant.abs() + 1e-5 * scale[:, None]
    assert bool(((wgg.double() - wwant).abs() <= wbound).all()), "wgrad closed form"
    print(f"[config {cid}] closed forms ok", flush=True)

    # the oracle, y = gather(x) (the oracle's own gather): every token for
    # seed 0, a token sample for the other seeds
    full = seed == 0
    tok = np.arange(wl.T, dtype=np.int64) if full else _sample_tokens(rng, wl.T)
    sel = None if full else tok
    tg = torch.from_numpy(tok).to(DEV)
    if full:
        y_part = oracle.gather(wl.x, ro, wl.layout, cap)
    else:
        need = np.unique(rows.reshape(wl.T, wl.K)[tok].reshape(-1))
        need = need[need >= 0].astype(np.int64)
        y_part = np.zeros((R, wl.H), dtype=wl.x.dtype)  # only the sampled tokens' rows are filled
        y_part[need] = oracle.gather(wl.x, ro, wl.layout, cap, rows=need)
    so, S = oracle.scatter_combine(y_part, wl.dtype, ro, wl.layout, cap, weights=w_o, tokens=sel, with_scale=True)
    what = "every token" if full else "sample"
    assert_close(to_host(peg.scatter_combine(yg, rg, weights=w_g)[tg]), so, S, wl.dtype, f"combine {what}")
    del so, S
    wo, WS = oracle.wgrad(y_part, wl.grad, wl.dtype, ro, wl.layout, cap, tokens=sel, with_scale=True)
    assert_close(to_host(wgg[tg]), wo, WS, W.F32, f"wgrad {what}")
    del y_part
    print(f"[config {cid}] combine and wgrad against the oracle ({what}) ok", flush=True)
    if cid in (3, 4) or full:
        # independent random y with NaN in every unused row
        yr = W.expert_tensor_rows(rng, R, wl.H, wl.dtype, used_rows=rows[kept])
        yrg = to_dev(yr, wl.dtype)
        so2, S2 = oracle.scatter_combine(yr, wl.dtype, ro, wl.layout, cap, weights=w_o, tokens=sel,
                                         with_scale=True)
        out = peg.scatter_combine(yrg, rg, weights=w_g)
        assert not bool(torch.isnan(out.float()).any()), "combine read an unused row"
        assert_close(to_host(out[tg]), so2, S2, wl.dtype, f"combine(y_rand) {what}")
        del so2, S2, out
        wo2, WS2 = oracle.wgrad(yr, wl.grad, wl.dtype, ro, wl.layout, cap, tokens=sel, with_scale=True)
        wr = peg.wgrad(yrg, gg, rg)
        assert not bool(torch.isnan(wr).any()), "wgrad read an unused row"
        assert_close(to_host(wr[tg]), wo2, WS2, W.F32, f"wgrad(y_rand) {what}")
        del yr, yrg
        print(f"[config {cid}] independent y ok", flush=True)
    # backward of the combine with wgrad: every kept row of dy equals
    # the fp32 product w * dout rounded once (computed here by torch on the
    # device), every other row is zero; the fused wgrad equals the wgrad
    # kernel bit for bit; a row sample against the oracle
    dyg, wgb = peg.combine_backward(yg, gg, rg, weights=w_g, dy_rows=R)
    kept_t = torch.from_numpy(kept.astype(np.int64)).to(DEV)
    rk = torch.from_numpy(rows[kept].astype(np.int64)).to(DEV)
    want_rows = (w_g[kept_t].unsqueeze(1) * gg[kept_t // wl.K].float()).to(gg.dtype)
    assert torch.equal(dyg[rk].view(torch.int16), want_rows.view(torch.int16)), "backward dy kept rows"
    gapm = torch.ones(R, dtype=torch.bool, device=DEV)
    gapm[rk] = False
    assert int(dyg[gapm].view(torch.int16).count_nonzero().item()) == 0, "backward dy gap rows"
    assert torch.equal(wgb, wgg), "fused wgrad == wgrad kernel"
    dyo_s = oracle.combine_backward_dy(wl.grad, wl.dtype, ro, wl.layout, cap, weights=w_o, rows=sample)
    assert_close(to_host(dyg[torch.from_numpy(sample).to(DEV)]), dyo_s,
                 np.abs(W.to_f32(dyo_s, wl.dtype).astype(np.float64)), wl.dtype, "backward dy sample")
    print(f"[config {cid}] done", flush=True)


@pytest.mark.parametrize("cid,seed", [(c, s) for c in (3, 4, 5) for s in (1, 2, 3, 4)])
def test_large_config_routing_seeds(cid, seed):
    """Workloads 3-5, seeds 1-4: the routing at full size (compaction for 4)
    bit for bit, and a gather of narrow rows (H = 40) through it, every row
    checked against its token (full-width rows: test_large_config)."""
    print(f"[config {cid} seed {seed}] routing", flush=True)
    wl = W.config(cid, seed, with_rows=False)
    ro, rg, rows, cap, _, _ = _prep(wl)
    if cid == 3:
        counts = np.asarray(ro.tokens_per_expert)
        assert int(np.sum(counts > wl.capacity)) == 2 and int(np.sum(counts == 0)) == 1
    rng = np.random.default_rng(2000 + 10 * cid + seed)
    x = W.normal(rng, (wl.T, 40), W.BF16)
    xg = to_dev(x, W.BF16)
    yg = peg.gather_binned(xg, rg) if wl.layout == W.BINNED else peg.gather_padded(xg, rg)
    assert yg.shape[0] == oracle.expert_rows(ro, wl.layout, cap)
    _check_gather_full(yg, xg, rows, wl.K, "narrow gather")
    assert int(peg.validate_routing(rg, n_indices=ro.n).item()) == 0
