"""GPU: the tiled routing preparation (8192 ids and more: a histogram
launch, then a placement launch whose blocks sum the tile-major count table
in the workspace), bit for bit against the oracle's route_prep ("Build
Triton-Ascend Padded MoE Routing" / "... Binned MoE Routing", Workflow steps
1-3):
  - one workspace reused by several routings of the same sizes (each call
    finds the previous call's table there), and workspaces of 0xFF bytes and
    of random bytes: nothing from an earlier call or from the workspace's
    prior contents reaches the result;
  - calls queued back to back on one stream with one workspace;
  - route_prep at a tiled size captured in a HIP graph and replayed with new
    routings.
Sizes span 32 to 256 tiles, few and many experts, and a ragged last tile.
"""
import numpy as np
import pytest
import torch

import oracle
import padded_expert_gather_amd as peg
import workloads as W
from gpu_util import DEV, bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

# (T, K, E, layout, capacity, pad multiple): tiled sizes from 32 to 256
# tiles, few and many experts, a ragged last tile
SHAPES = [
    (4096, 2, 8, W.PADDED, None, 128),          # 8192 ids, 32 tiles of 256
    (8192, 8, 256, W.PADDED, None, 128),        # 65536 ids, 64 tiles
    (32768, 8, 64, W.BINNED, 4096, None),       # 262144 ids, 256 tiles of 1024
    (5001, 3, 13, W.BINNED, 900, 16),           # ragged; binned with padded bins
    (16384, 2, 8, W.BINNED, 5120, None),        # 32768 ids, 64 tiles of 512
]


def _check(top, E, layout, cap, m, rg, what):
    ro = oracle.route_prep(top, E, pad_multiple=m)
    bits_equal(to_host(rg.indices), ro.indices, f"{what}: indices")
    bits_equal(to_host(rg.bin_ids), ro.bin_ids, f"{what}: bin_ids")
    bits_equal(to_host(rg.tokens_per_expert), ro.tokens_per_expert, f"{what}: tokens_per_expert")
    bits_equal(to_host(rg.bins), ro.bins, f"{what}: bins")
    if m is not None:
        bits_equal(to_host(rg.padded_bins), ro.padded_bins, f"{what}: padded_bins")
    bits_equal(to_host(rg.slot_row), oracle.assignment_rows(ro, layout, cap), f"{what}: slot_row")


def _routing(seed, T, K, E):
    rng = np.random.default_rng(seed)
    top, _ = W.random_routing(rng, T, K, E, none_frac=0.03, skew=0.3)
    return top


def _prep(top_dev, E, layout, cap, m, ws=None):
    if layout == W.BINNED:
        return peg.route_prep(top_dev, E, capacity=cap, pad_multiple=m, ws=ws)
    return peg.route_prep(top_dev, E, pad_multiple=m, ws=ws)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"T{s[0]}K{s[1]}E{s[2]}" for s in SHAPES])
def test_tiled_reused_and_dirty_workspace(shape):
    """One workspace for several routings of the same sizes in a row (each
    call finds the previous call's flags and counts there), then a
    workspace of 0xFF bytes and one of random bytes."""
    T, K, E, layout, cap, m = shape
    print(f"[tiled workspace] T{T} K{K} E{E} layout{layout}", flush=True)
    nb = peg.workspace_bytes(T, K, E)
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    for seed in (2, 3, 2, 4):
        top = _routing(seed, T, K, E)
        _check(top, E, layout, cap, m, _prep(to_dev(top), E, layout, cap, m, ws=ws), f"reused ws, seed {seed}")
    top = _routing(5, T, K, E)
    ws.fill_(0xFF)
    _check(top, E, layout, cap, m, _prep(to_dev(top), E, layout, cap, m, ws=ws), "0xFF workspace")
    g = torch.Generator(device="cpu").manual_seed(6)
    ws.copy_(torch.randint(0, 256, (nb,), dtype=torch.uint8, generator=g).to(DEV))
    _check(top, E, layout, cap, m, _prep(to_dev(top), E, layout, cap, m, ws=ws), "random workspace")


def test_tiled_back_to_back_calls_share_workspace():
    """Calls queued back to back on one stream with one workspace and
    different routings, without a synchronisation in between: each result
    matches its own routing."""
    T, K, E, m = 8192, 8, 256, 128
    print("[tiled back to back]", flush=True)
    ws = torch.empty(peg.workspace_bytes(T, K, E), dtype=torch.uint8, device=DEV)
    tops = [_routing(10 + i, T, K, E) for i in range(4)]
    outs = [_prep(to_dev(t), E, W.PADDED, None, m, ws=ws) for t in tops]
    torch.cuda.synchronize()
    for i, (t, rg) in enumerate(zip(tops, outs)):
        _check(t, E, W.PADDED, None, m, rg, f"call {i}")


def test_tiled_route_prep_graph_replays():
    """route_prep at a tiled size captured in a HIP graph and replayed three
    times with new routings written into the captured input buffer; every
    replay matches the eager result and the oracle."""
    T, K, E, m = 8192, 8, 256, 128
    print("[tiled graph]", flush=True)
    lib = peg.library()
    i32 = dict(dtype=torch.int32, device=DEV)
    top_buf = torch.zeros((T, K), **i32)
    n = T * K
    outs = dict(indices=torch.empty(n, **i32), bin_ids=torch.empty(n, **i32), tpe=torch.empty(E, **i32),
                bins=torch.empty(E, **i32), pb=torch.empty(E, **i32), slot=torch.empty(n, **i32))
    ws = torch.empty(peg.workspace_bytes(T, K, E), dtype=torch.uint8, device=DEV)

    def call():
        st = torch.cuda.current_stream().cuda_stream
        rc = lib.peg_route_prep(top_buf.data_ptr(), T, K, E, peg.PADDED, 0, m, outs["indices"].data_ptr(),
                                outs["bin_ids"].data_ptr(), outs["tpe"].data_ptr(), outs["bins"].data_ptr(),
                                outs["pb"].data_ptr(), outs["slot"].data_ptr(), ws.data_ptr(), ws.numel(), st)
        assert rc == 0

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
    for seed in (20, 21, 22):
        top = _routing(seed, T, K, E)
        top_buf.copy_(to_dev(top))
        call()  # eager, on the same buffers
        torch.cuda.synchronize()
        eager = {k: v.clone() for k, v in outs.items()}
        for v in outs.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], eager[k]), f"replay (seed {seed}): {k} differs from eager"
        ro = oracle.route_prep(top, E, pad_multiple=m)
        bits_equal(to_host(outs["indices"]), ro.indices, "replay indices")
        bits_equal(to_host(outs["slot"]), oracle.assignment_rows(ro, W.PADDED, None), "replay slot_row")
