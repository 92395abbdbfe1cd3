"""GPU: zeroing of the gap rows of large expert tensors (hundreds of MB,
mostly gap), against the oracle's gather, bit for bit; and one expert tensor
past 2^31 bytes through the gather, the combine, wgrad and the combine
backward.

Every output buffer is filled with 0xFF bytes first, so a gap row that is
not written shows up as a mismatch. Cases: 16-, 8-, 4- and 2-byte row
vectors, binned tensors above and below 128 MB (the gap rows of the former
come from a fill-shaped launch of their own); binned with dropped routes and mostly empty capacity; padded with a
large multiple; padded with a multiple of 2 and a buffer far longer than the
padded rows, so that each gap block's range crosses the gaps of many
experts (rows past padded_bins[E-1] must stay untouched); a buffer cut short
of padded_bins[E-1]; E = 1 and E = 64; all routes absent. Plus float16
and float32 through the K = 8 gather, combine, wgrad and combine backward
over a binned tensor of 128 / 256 MiB, against the oracle on every element.
"""
import numpy as np
import pytest
import torch

import oracle
import padded_expert_gather_amd as peg
import workloads as W
from gpu_util import DEV, bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

LARGE_UNITS = 1 << 24  # row vectors of every tensor here
ELEM = {W.F32: 4, W.BF16: 2, W.F16: 2}


def _vec_units(H, dtype):
    """Row vectors of the widest lane (16, 8, 4 or 2 bytes) dividing the row."""
    rb = H * ELEM[dtype]
    for v in (16, 8, 4, 2):
        if rb % v == 0 and v >= ELEM[dtype]:
            return rb // v
    raise AssertionError


W_TORCH = {W.F32: torch.float32, W.BF16: torch.bfloat16, W.F16: torch.float16}


def _filled(rows, H, dtype):
    t = torch.empty((rows, H), dtype=W_TORCH[dtype], device=DEV)
    t.view(torch.uint8).fill_(0xFF)
    return t


@pytest.mark.parametrize("T,K,E,H,dtype,C,none_frac,skew", [
    (100000, 4, 64, 64, W.BF16, 32768, 0.0, 0.3),    # 16-byte vectors, 87% gap rows, drops
    (60000, 2, 64, 12, W.BF16, 98304, 0.1, 0.0),     # 8-byte vectors
    (80000, 2, 32, 7, W.F32, 262144, 0.0, 0.5),      # 4-byte vectors
    (50000, 8, 64, 5, W.BF16, 65536, 0.0, 2.0),      # 2-byte vectors, heavy skew
    (50000, 8, 64, 5, W.BF16, 262144, 0.0, 2.0),     # 2-byte vectors, 168 MB: the fill-shaped gap launch
    (300000, 1, 1, 256, W.BF16, 524288, 0.2, 0.0),   # E = 1
    (20000, 2, 64, 64, W.BF16, 32768, 1.0, 0.0),     # no route at all: every row is gap
])
def test_large_gaps_binned(T, K, E, H, dtype, C, none_frac, skew):
    print(f"[gaps binned] T{T} K{K} E{E} H{H} C{C} dtype{dtype}", flush=True)
    assert E * C * _vec_units(H, dtype) >= LARGE_UNITS
    rng = np.random.default_rng(T + H)
    top, _ = W.random_routing(rng, T, K, E, none_frac=none_frac, skew=skew)
    x = W.normal(rng, (T, H), dtype)
    ro = oracle.route_prep(top, E)
    rg = peg.route_prep(to_dev(top), E, capacity=C)
    out = _filled(E * C, H, dtype)
    peg.gather_binned(to_dev(x, dtype), rg, out=out)
    bits_equal(to_host(out), oracle.gather(x, ro, W.BINNED, C), "binned gather")
    out.view(torch.uint8).fill_(0xFF)
    peg.gather_binned(to_dev(x, dtype), rg, out=out, use_slot_row=False)
    bits_equal(to_host(out), oracle.gather(x, ro, W.BINNED, C), "binned gather (rebuilt map)")


@pytest.mark.parametrize("T,K,E,H,dtype,m,extra_rows", [
    (200000, 2, 64, 5, W.BF16, 65536, 0),            # large multiple, 2-byte vectors
    (3000, 2, 64, 1, W.F32, 2, (1 << 24) + 11),      # gaps of 0-1 rows: a block's range spans many experts
    (5000, 4, 48, 64, W.BF16, 2, (1 << 21) + 5),     # same with 16-byte vectors
])
def test_large_gaps_padded(T, K, E, H, dtype, m, extra_rows):
    print(f"[gaps padded] T{T} K{K} E{E} H{H} m{m} extra{extra_rows}", flush=True)
    rng = np.random.default_rng(T + E)
    top, _ = W.random_routing(rng, T, K, E, skew=0.2)
    x = W.normal(rng, (T, H), dtype)
    ro = oracle.route_prep(top, E, pad_multiple=m)
    rg = peg.route_prep(to_dev(top), E, pad_multiple=m)
    R = int(ro.padded_bins[-1])
    rows = R + extra_rows
    assert rows * _vec_units(H, dtype) >= LARGE_UNITS
    out = _filled(rows, H, dtype)
    peg.gather_padded(to_dev(x, dtype), rg, out=out)
    host = to_host(out)
    bits_equal(host[:R], oracle.gather(x, ro, W.PADDED), "padded gather")
    assert (host[R:].view(np.uint8) == 0xFF).all(), "rows past padded_bins[E-1] were written"


def test_large_gaps_cut_buffer():
    """A buffer shorter than padded_bins[E-1]: the rows it holds match, the
    flag is raised and nothing past the buffer is written."""
    print("[gaps cut]", flush=True)
    rng = np.random.default_rng(11)
    T, K, E, H, m = 50000, 2, 64, 40, 65536
    top, _ = W.random_routing(rng, T, K, E, skew=0.1)
    x = W.normal(rng, (T, H), W.BF16)
    ro = oracle.route_prep(top, E, pad_multiple=m)
    rg = peg.route_prep(to_dev(top), E, pad_multiple=m)
    R = int(ro.padded_bins[-1])
    small = R - 3 * m - 17
    assert small * _vec_units(H, W.BF16) >= LARGE_UNITS
    buf = _filled(small + 100, H, W.BF16)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    peg.gather_padded(to_dev(x, W.BF16), rg, out=buf[:small], err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & peg.FLAG_OUT_ROWS
    host = to_host(buf)
    bits_equal(host[:small], oracle.gather(x, ro, W.PADDED)[:small], "cut padded gather")
    assert (host[small:].view(np.uint8) == 0xFF).all(), "rows past the buffer were written"


def test_tensor_beyond_2gib():
    """An expert tensor of 2.6 GB (byte offsets past 2^31): the gather, the
    combine, wgrad and the combine backward through it, checked on the device
    against the token rows (gather and dy: every row; combine and wgrad:
    their closed forms on every token) and against the oracle on a row
    sample."""
    print("[beyond 2 GiB]", flush=True)
    rng = np.random.default_rng(21)
    T, K, E, H, C = 65536, 4, 64, 4096, 5000
    assert E * C * H * 2 > 2 ** 31
    top, w = W.random_routing(rng, T, K, E, none_frac=0.02, skew=0.2)
    x = W.normal(rng, (T, H), W.BF16)
    ro = oracle.route_prep(top, E)
    rg = peg.route_prep(to_dev(top), E, capacity=C)
    rows = oracle.assignment_rows(ro, W.BINNED, C)
    bits_equal(to_host(rg.slot_row), rows, "slot_row")
    xg = to_dev(x, W.BF16)
    y = _filled(E * C, H, W.BF16)
    peg.gather_binned(xg, rg, out=y)
    kept = np.flatnonzero(rows >= 0)
    rk = torch.from_numpy(rows[kept].astype(np.int64)).to(DEV)
    tk = torch.from_numpy((kept // K).astype(np.int64)).to(DEV)
    yv, xv = y.view(torch.int16), xg.view(torch.int16)
    for lo in range(0, len(kept), 65536):  # kept rows against their tokens, in slices
        assert torch.equal(yv[rk[lo:lo + 65536]], xv[tk[lo:lo + 65536]]), "a kept row differs from its token"
    gap = torch.ones(E * C, dtype=torch.bool, device=DEV)
    gap[rk] = False
    assert int(yv[gap].count_nonzero().item()) == 0, "a gap row is not zero"
    sample = np.unique(np.concatenate([[0, E * C - 1], rng.choice(E * C, 512, replace=False),
                                       np.arange(E) * C + C - 1])).astype(np.int64)
    bits_equal(to_host(y[torch.from_numpy(sample).to(DEV)]), oracle.gather(x, ro, W.BINNED, C, rows=sample),
               "gather sample")
    # combine and wgrad through the 2.6 GB tensor: closed forms on every token
    wg = to_dev(w.reshape(-1))
    keptmask = torch.from_numpy((rows >= 0).reshape(T, K)).to(DEV)
    wsum = torch.where(keptmask, wg.reshape(T, K), torch.zeros((), device=DEV)).sum(1)
    xf = xg.float()
    comb = peg.scatter_combine(y, rg, weights=wg).float()
    want = wsum[:, None] * xf
    assert bool(((comb - want).abs() <= 2e-2 * want.abs() + 1e-5 * wsum.abs()[:, None] * xf.abs()).all()), \
        "combine closed form"
    grad = W.normal(rng, (T, H), W.BF16)
    gg = to_dev(grad, W.BF16)
    wgr = peg.wgrad(y, gg, rg)
    prod = xf * gg.float()
    wwant = torch.where(keptmask, prod.sum(1)[:, None], torch.zeros((), device=DEV))
    assert bool(((wgr - wwant).abs() <= 1e-5 * wwant.abs() + 2e-5 * prod.abs().sum(1)[:, None]).all()), \
        "wgrad closed form"
    # the combine backward writes a second 2.6 GB tensor: kept rows w * dout
    # (one rounding, computed here by torch), gap rows zero; its wgrad equals
    # the wgrad kernel's bit for bit
    del comb, want, prod
    dyg, wgb = peg.combine_backward(y, gg, rg, weights=wg, dy_rows=E * C)
    kept_t = torch.from_numpy(kept.astype(np.int64)).to(DEV)
    dv = dyg.view(torch.int16)
    for lo in range(0, len(kept), 65536):
        sl = slice(lo, lo + 65536)
        want_rows = (wg[kept_t[sl]].unsqueeze(1) * gg[kept_t[sl] // K].float()).to(torch.bfloat16)
        assert torch.equal(dv[rk[sl]], want_rows.view(torch.int16)), "backward dy kept rows"
    assert int(dv[gap].count_nonzero().item()) == 0, "backward dy gap rows"
    assert torch.equal(wgb, wgr), "fused wgrad == wgrad kernel"


@pytest.mark.parametrize("K", [2, 4])
def test_large_binned_dy_rows_past_layout(K):
    """The combine backward into a binned dy of more than 128 MB (its gap
    rows then come from the fill-shaped launch) with more rows than E*C:
    kept rows are w * dout, gap rows and the rows [E*C, dy_rows) are zero,
    rows past dy_rows untouched; the fused wgrad (K = 2) or the wgrad
    kernel's pass after the dy gather (K = 4) equals the wgrad kernel."""
    print(f"[gaps dy tail] K{K}", flush=True)
    rng = np.random.default_rng(31 + K)
    T, E, H, C = 20000, 8, 2048, 4096
    extra = 1000
    assert E * C * H * 2 >= 128 << 20
    top, w = W.random_routing(rng, T, K, E, none_frac=0.05, skew=0.4)
    dout = W.normal(rng, (T, H), W.BF16)
    ro = oracle.route_prep(top, E)
    rg = peg.route_prep(to_dev(top), E, capacity=C)
    xg = to_dev(W.normal(rng, (T, H), W.BF16), W.BF16)
    y = peg.gather_binned(xg, rg)
    buf = _filled(E * C + extra + 64, H, W.BF16)
    dg = to_dev(dout, W.BF16)
    wg = to_dev(w.reshape(-1))
    dy, wgb = peg.combine_backward(y, dg, rg, weights=wg, dy=buf[:E * C + extra])
    rows = oracle.assignment_rows(ro, W.BINNED, C)
    kept = np.flatnonzero(rows >= 0)
    rk = torch.from_numpy(rows[kept].astype(np.int64)).to(DEV)
    tk = torch.from_numpy(kept.astype(np.int64)).to(DEV)
    want = (wg[tk].unsqueeze(1) * dg[tk // K].float()).to(torch.bfloat16)
    assert torch.equal(dy[rk].view(torch.int16), want.view(torch.int16)), "kept rows of dy"
    gap = torch.ones(E * C + extra, dtype=torch.bool, device=DEV)
    gap[rk] = False
    assert int(dy[gap].view(torch.int16).count_nonzero().item()) == 0, "gap or tail rows of dy not zero"
    assert (to_host(buf[E * C + extra:]).view(np.uint8) == 0xFF).all(), "rows past dy_rows were written"
    assert torch.equal(wgb, peg.wgrad(y, dg, rg)), "fused wgrad == wgrad kernel"


@pytest.mark.parametrize("dtype", [W.F16, W.F32])
def test_large_binned_k8_against_oracle(dtype):
    """Float16 and float32 through the K = 8 paths over a binned tensor of
    128 / 256 MiB (its gap rows from the fill-shaped launch): the gather bit
    for bit, the combine and wgrad on an independent NaN-sentinel y, and the
    combine backward (its dy gather with scaling in the element type, then
    the wgrad kernel) against the oracle on every element; the backward's
    wgrad equals the wgrad kernel's bit for bit."""
    from gpu_util import assert_close
    print(f"[gaps K8 dtype{dtype}]", flush=True)
    rng = np.random.default_rng(51 + dtype)
    T, K, E, H, C = 8192, 8, 16, 1024, 4096
    assert E * C * H * ELEM[dtype] >= 128 << 20
    top, w = W.random_routing(rng, T, K, E, none_frac=0.05, skew=0.15)
    x = W.normal(rng, (T, H), dtype)
    grad = W.normal(rng, (T, H), dtype)
    ro = oracle.route_prep(top, E)
    rg = peg.route_prep(to_dev(top), E, capacity=C)
    rows = oracle.assignment_rows(ro, W.BINNED, C)
    bits_equal(to_host(rg.slot_row), rows, "slot_row")
    # gather into a 0xFF-filled buffer: every row written
    buf = _filled(E * C, H, dtype)
    peg.gather_binned(to_dev(x, dtype), rg, out=buf)
    bits_equal(to_host(buf), oracle.gather(x, ro, W.BINNED, C), "gather")
    del buf
    # combine and wgrad on an independent y whose unused rows are NaN
    yr = W.expert_tensor_rows(rng, E * C, H, dtype, used_rows=rows[rows >= 0])
    yg, gg, wg = to_dev(yr, dtype), to_dev(grad, dtype), to_dev(w.reshape(-1))
    so, S = oracle.scatter_combine(yr, dtype, ro, W.BINNED, C, weights=w.reshape(-1), with_scale=True)
    assert_close(to_host(peg.scatter_combine(yg, rg, weights=wg)), so, S, dtype, "combine")
    wo, WS = oracle.wgrad(yr, grad, dtype, ro, W.BINNED, C, with_scale=True)
    wk = peg.wgrad(yg, gg, rg)
    assert_close(to_host(wk), wo, WS, W.F32, "wgrad")
    # combine backward (K = 8: dy gather, then the wgrad kernel)
    dyo = oracle.combine_backward_dy(grad, dtype, ro, W.BINNED, C, weights=w.reshape(-1))
    dyg, wgb = peg.combine_backward(yg, gg, rg, weights=wg, dy_rows=E * C)
    assert_close(to_host(dyg), dyo, np.abs(W.to_f32(dyo, dtype).astype(np.float64)), dtype, "backward dy")
    assert torch.equal(wgb, wk), "backward wgrad == wgrad kernel"
