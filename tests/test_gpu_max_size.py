"""GPU: route_prep at the largest batch the library accepts, T*K = 2^31 - 1
assignments (sorted positions and rows are int32), E = 8, padded layout with
m = 1 (rows = sorted positions), about a ninth of the routes absent.

At this size the oracle cannot run in seconds, so the outputs are checked on
the device against properties that define them ("Build Triton-Ascend Padded
MoE Routing", Workflow steps 1-3 and Implementation Pattern):
  - tokens_per_expert = the count of each expert id in top_experts, bins its
    inclusive sum, padded_bins = bins (m = 1);
  - in sorted positions [start(e), bins[e]) every bin_id is e, every
    top_experts[indices[p]] is e, and indices increase strictly (a stable
    sort: with the counts this makes each segment exactly the ids of that
    expert in ascending order);
  - positions [n, T*K) hold -1 in indices and bin_ids;
  - slot_row[indices[p]] = p for every p < n, and -1 where the route is absent.
"""
import pytest
import torch

import padded_expert_gather_amd as peg
from gpu_util import DEV

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27


def test_route_prep_at_the_assignment_limit():
    total = (1 << 31) - 1
    E = 8
    print(f"[max size] route_prep of {total} assignments, E{E}, padded m1", flush=True)
    g = torch.Generator(device=DEV).manual_seed(7)
    top = torch.randint(-1, E, (total, 1), dtype=torch.int32, device=DEV, generator=g)
    r = peg.route_prep(top, E, pad_multiple=1)
    torch.cuda.synchronize()
    print("[max size] route_prep done; checking", flush=True)
    flat = top.view(-1)
    counts = torch.stack([(flat == e).sum() for e in range(E)]).to(torch.int64)
    assert torch.equal(r.tokens_per_expert.to(torch.int64), counts), "tokens_per_expert"
    bins = torch.cumsum(counts, 0)
    assert torch.equal(r.bins.to(torch.int64), bins), "bins"
    assert torch.equal(r.padded_bins, r.bins), "padded_bins with m = 1"
    n = int(bins[-1].item())
    assert 0 < n < total
    starts = [0] + bins[:-1].tolist()
    for e in range(E):
        s, t = starts[e], int(bins[e].item())
        for c0 in range(s, t, CHUNK):
            c1 = min(t, c0 + CHUNK)
            ids = r.indices[c0:c1]
            assert bool((r.bin_ids[c0:c1] == e).all()), f"bin_ids of expert {e}"
            assert bool((flat[ids.long()] == e).all()), f"indices of expert {e} point at other experts"
            if c1 - c0 > 1:
                assert bool((ids[1:] > ids[:-1]).all()), f"indices of expert {e} not increasing"
            if c0 > s:  # across the chunk boundary
                assert int(r.indices[c0 - 1].item()) < int(ids[0].item()), f"expert {e} at {c0}"
            pos = torch.arange(c0, c1, dtype=torch.int32, device=DEV)
            assert torch.equal(r.slot_row[ids.long()], pos), f"slot_row of expert {e}"
        print(f"[max size] expert {e} checked", flush=True)
    for c0 in range(n, total, CHUNK):
        c1 = min(total, c0 + CHUNK)
        assert bool((r.indices[c0:c1] == -1).all()) and bool((r.bin_ids[c0:c1] == -1).all()), "tail not -1"
    for c0 in range(0, total, CHUNK):
        c1 = min(total, c0 + CHUNK)
        absent = flat[c0:c1] < 0
        assert bool((r.slot_row[c0:c1][absent] == -1).all()), "slot_row of an absent route"
