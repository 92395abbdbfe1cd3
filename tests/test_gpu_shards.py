"""GPU: routing into caller-given row windows, and a batch cut into token
shards that reproduces the one-call result exactly.

* peg_route_prep_windows against the oracle (sorted arrays and rows within
  random windows, some empty or shorter than their expert's count);
* a batch cut into contiguous token shards, each routed with windows that
  start where the earlier shards' assignments of each expert end (prefix sums
  of the shards' tokens_per_expert, on the device) and dispatched with
  peg_gather_rows into one cleared expert tensor: the tensor, the row map,
  the combine and wgrad of every shard equal those of one call over the
  whole batch, bit for bit (the same kernels see the same rows in the same
  order).
"""
import numpy as np
import pytest
import torch

import oracle
import padded_expert_gather_amd as peg
import workloads as W
from gpu_util import DEV, bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,K,E", [(1, 1, 1), (37, 2, 5), (600, 4, 16), (5000, 2, 8), (3000, 8, 64)])
def test_windows_match_oracle(T, K, E):
    print(f"[windows] T{T} K{K} E{E}", flush=True)
    rng = np.random.default_rng(T + K + E)
    top, _ = W.random_routing(rng, T, K, E, none_frac=0.1, skew=0.2)
    base = rng.integers(0, 10000, size=E).astype(np.int32)
    limit = (base + rng.integers(0, 2 * T * K // E + 2, size=E)).astype(np.int32)
    rg = peg.route_prep_windows(to_dev(top), E, to_dev(base), to_dev(limit))
    ro = oracle.route_prep(top, E)
    bits_equal(to_host(rg.indices), ro.indices, "indices")
    bits_equal(to_host(rg.bin_ids), ro.bin_ids, "bin_ids")
    bits_equal(to_host(rg.tokens_per_expert), ro.tokens_per_expert, "tokens_per_expert")
    bits_equal(to_host(rg.bins), ro.bins, "bins")
    bits_equal(to_host(rg.slot_row), oracle.assignment_rows_windows(ro, base, limit), "slot_row")


@pytest.mark.parametrize("T,K,E,H,C,cuts", [(4096, 2, 8, 512, 1100, (1000, 1001, 3000)),
                                           (2000, 8, 64, 96, 230, (700, 1300)),
                                           (1000, 2, 8, 6144, 300, (333,)),     # long rows: a token over 2 blocks
                                           (600, 4, 16, 4100, 180, (1, 599))])
def test_shards_reproduce_one_call(T, K, E, H, C, cuts):
    print(f"[shards] T{T} K{K} E{E} H{H} C{C}", flush=True)
    rng = np.random.default_rng(7 * T + E)
    top, w = W.random_routing(rng, T, K, E, none_frac=0.05, skew=0.3)
    x = W.normal(rng, (T, H), W.BF16)
    grad = W.normal(rng, (T, H), W.BF16)
    topg, wg = to_dev(top), to_dev(w)
    xg, gg = to_dev(x, W.BF16), to_dev(grad, W.BF16)
    # one call over the whole batch
    r = peg.route_prep(topg, E, capacity=C)
    y_full = peg.gather_binned(xg, r)
    out_full = peg.scatter_combine(y_full, r, weights=wg.reshape(-1))
    wg_full = peg.wgrad(y_full, gg, r)
    assert int((r.tokens_per_expert > C).sum().item()) >= 1  # some expert overflows
    # shards: counts first (any layout), then windows after the earlier shards
    bounds = [0, *cuts, T]
    shards = list(zip(bounds[:-1], bounds[1:]))
    counts = torch.stack([peg.route_prep(topg[lo:hi], E, capacity=C).tokens_per_expert for lo, hi in shards])
    before = torch.cumsum(counts, 0) - counts  # assignments of each expert in the earlier shards
    starts = torch.arange(E, dtype=torch.int32, device=DEV) * C
    y_sh = torch.zeros((E * C, H), dtype=torch.bfloat16, device=DEV)
    slots, outs, wgs = [], [], []
    routings = []
    for s, (lo, hi) in enumerate(shards):
        base = (starts + before[s]).to(torch.int32)
        rs = peg.route_prep_windows(topg[lo:hi], E, base, starts + C, capacity=C)
        peg.gather_rows(xg[lo:hi], rs.slot_row, K, y_sh)
        routings.append((lo, hi, rs))
        slots.append(rs.slot_row)
    torch.cuda.synchronize()
    bits_equal(to_host(torch.cat(slots)), to_host(r.slot_row), "row map of the shards")
    bits_equal(to_host(y_sh), to_host(y_full), "expert tensor assembled from the shards")
    for lo, hi, rs in routings:
        outs.append(peg.scatter_combine(y_sh, rs, weights=wg[lo:hi].reshape(-1)))
        wgs.append(peg.wgrad(y_sh, gg[lo:hi], rs))
    bits_equal(to_host(torch.cat(outs)), to_host(out_full), "combine of the shards")
    bits_equal(to_host(torch.cat(wgs)), to_host(wg_full), "wgrad of the shards")
