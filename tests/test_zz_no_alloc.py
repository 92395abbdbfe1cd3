"""GPU: the allocation-free routing preparation (peg_route_prep_noalloc,
the library's static device scratch instead of a workspace) against
peg_route_prep with a caller workspace, through the C ABI.

Two calls in a row on one GPU, the second with a smaller batch (its count
table then lands in scratch that still holds the first call's), then a
batch small enough for the one-block path, must each give the
workspace call's outputs bit for bit; sizes past the static scratch are
refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import padded_expert_gather_amd as peg
import workloads as W
from gpu_util import DEV, bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

FIELDS = ("indices", "bin_ids", "tokens_per_expert", "bins", "padded_bins", "slot_row")


def _same(a, b, what):
    for f in FIELDS:
        x, y = getattr(a, f), getattr(b, f)
        if x is None and y is None:
            continue
        bits_equal(to_host(x), to_host(y), f"{what}: {f}")


def _routing(seed, T, K, E, none_frac=0.0, skew=0.0):
    rng = np.random.default_rng(seed)
    top, _ = W.random_routing(rng, T, K, E, none_frac=none_frac, skew=skew)
    return to_dev(top)


@pytest.mark.parametrize("layout", ["binned", "padded"])
def test_noalloc_matches_workspace_call(layout):
    cases = [(32768, 8, 64, 0.0, 1.0, 4096, 128),   # 262,144 assignments: the tiled path
             (6000, 3, 40, 0.1, 0.3, 300, 16),       # smaller, still tiled: stale scratch underneath
             (1000, 2, 8, 0.05, 0.0, 200, 8)]        # one-block path: no scratch
    for i, (T, K, E, nf, skew, C, m) in enumerate(cases):
        print(f"[noalloc] {layout} call {i}: T{T} K{K} E{E}", flush=True)
        top = _routing(100 + i, T, K, E, nf, skew)
        kw = dict(capacity=C) if layout == "binned" else dict(pad_multiple=m)
        want = peg.route_prep(top, E, **kw)
        got = peg.route_prep_noalloc(top, E, **kw)
        torch.cuda.synchronize()
        _same(got, want, f"{layout} call {i}")


def test_noalloc_reuses_preallocated_outputs():
    """With preallocated outputs nothing is allocated around the call either;
    a second call into the same buffers with another batch overwrites them."""
    T, K, E = 9000, 2, 16
    out = peg.route_prep_noalloc(_routing(7, T, K, E), E, pad_multiple=32)
    for seed in (8, 9):
        top = _routing(seed, T, K, E, none_frac=0.2)
        before = torch.cuda.memory_allocated(DEV)
        peg.route_prep_noalloc(top, E, pad_multiple=32, out=out)
        assert torch.cuda.memory_allocated(DEV) == before
        torch.cuda.synchronize()
        _same(out, peg.route_prep(top, E, pad_multiple=32), f"preallocated outputs, seed {seed}")


def test_noalloc_refuses_sizes_past_its_scratch():
    """E = 1024 takes tiles of 512 assignments: 140,000 assignments need a
    (1024 x 274)-entry count table, 1.07 MiB, past the 1 MiB scratch; the
    workspace call still takes them."""
    T, K, E = 140000, 1, 1024
    top = _routing(10, T, K, E)
    with pytest.raises(ValueError, match="static scratch"):
        peg.route_prep_noalloc(top, E, capacity=200)
    # 131,072 assignments (256 tiles of 512) fill the scratch exactly
    top2 = top[:131072]
    _same(peg.route_prep_noalloc(top2, E, capacity=200), peg.route_prep(top2, E, capacity=200), "at the limit")
