"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each function raises AssertionError when the oracle module ``o`` disagrees
with a fact fixed independently of it:
  * the hand-worked example in ``tests/golden/tiny_routing.json``;
  * library routines that compute a special case (numpy stable argsort,
    bincount, cumsum, fancy indexing, flatnonzero; numpy's float64->float16
    conversion; torch's float32->bfloat16 conversion; torch autograd;
    torch index_add);
  * brute force by enumeration on tiny inputs (per-expert enumeration of
    assignments, nearest-representable search over all 65536 16-bit codes);
  * closed forms (gather-then-combine equals the weight sum times the token
    row; gather-then-gradient equals <x_t, grad_t>);
  * the pages' invariants (bins monotonic, last bin equal to the number of
    indices, bin_ids consistent with bins, capacity overflow dropped, padding
    rows zero, unique assignment ids).
The same functions run against deliberately broken oracle builds in
``test_oracle_mutants.py``, where each broken build must fail at least one.
"""
import bisect
import itertools
import json
import math
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_routing.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# Independent re-derivations used by several pins.
# ----------------------------------------------------------------------------

def brute_rows(top, E, layout, capacity=None, pad_multiple=None):
    """Row of each assignment by per-expert enumeration: walk experts in
    order; an expert's assignments, in increasing id, take consecutive rows
    of its segment (segment = capacity rows, or its count rounded up)."""
    flat = [int(v) for v in np.asarray(top).reshape(-1)]
    rows = [-1] * len(flat)
    seg_start = 0
    for e in range(E):
        mine = [a for a in range(len(flat)) if flat[a] == e]
        if layout == W.BINNED:
            for j, a in enumerate(mine):
                if j < capacity:
                    rows[a] = e * capacity + j
            seg_start += capacity
        else:
            for j, a in enumerate(mine):
                rows[a] = seg_start + j
            seg_start += -(-len(mine) // pad_multiple) * pad_multiple
    return np.array(rows, np.int64), seg_start


def _nearest_even(table_vals, table_codes, v):
    """Nearest representable value to v among sorted finite codes; ties to the
    code with an even last bit. Returns None when v lies beyond the largest."""
    i = bisect.bisect_left(table_vals, v)
    cands = []
    for j in (i - 1, i):
        if 0 <= j < len(table_vals):
            cands.append((abs(table_vals[j] - v), table_codes[j] & 1, table_codes[j], table_vals[j]))
    cands.sort()
    if len(cands) == 2 and cands[0][0] == cands[1][0]:
        return cands[0][2] if cands[0][1] == 0 else cands[1][2]
    return cands[0][2]


def _code_table(kind):
    codes = np.arange(0x8000, dtype=np.uint32)  # non-negative codes
    with np.errstate(invalid="ignore"):
        if kind == "bf16":
            vals = (codes << 16).astype(np.uint32).view(np.float32).astype(np.float64)
        else:
            vals = codes.astype(np.uint16).view(np.float16).astype(np.float64)
    finite = np.isfinite(vals)
    order = np.argsort(vals[finite], kind="stable")
    return list(vals[finite][order]), [int(c) for c in codes[finite][order]]


# ----------------------------------------------------------------------------
# Number formats.
# ----------------------------------------------------------------------------

def pin_bf16_rounding(o):
    """bfloat16 rounding vs (a) torch's float32->bfloat16 on float32-exact
    values, (b) nearest-even search over all codes for arbitrary doubles."""
    import torch
    rng = np.random.default_rng(11)
    with np.errstate(over="ignore"):
        f = _bf16_inputs(rng)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([o.round_bf16(float(v)) for v in f], np.uint16)
    assert np.array_equal(got, ref), "bf16 rounding differs from torch on float32 inputs"
    _bf16_rest(o, rng)


def _bf16_inputs(rng):
    return np.concatenate([
        rng.standard_normal(2000).astype(np.float32),
        (rng.standard_normal(500) * 1e-39).astype(np.float32),  # subnormal range
        (rng.standard_normal(500) * 1e38).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.3895314e38,
                  np.float32(np.finfo(np.float32).max), 2 ** -133, 2 ** -134, 3 * 2 ** -135], np.float32),
    ])


def _bf16_rest(o, rng):
    vals, codes = _code_table("bf16")
    ds = np.concatenate([rng.standard_normal(800), rng.standard_normal(200) * 1e-38,
                         np.array([1.0 + 2 ** -8 + 2 ** -40, 1.0 + 2 ** -8 - 2 ** -40])])
    for d in ds:
        a = abs(float(d))
        want = _nearest_even(vals, codes, a) | (0x8000 if d < 0 else 0)
        assert o.round_bf16(float(d)) == want, f"bf16 rounding of {d!r}"
    assert o.round_bf16(float("inf")) == 0x7F80 and o.round_bf16(-float("inf")) == 0xFF80
    assert o.round_bf16(float("nan")) & 0x7FC0 == 0x7FC0
    assert o.round_bf16(2.0 ** 128) == 0x7F80  # beyond the largest finite -> infinity


def pin_f16_rounding(o):
    """binary16 rounding vs numpy's direct float64->float16 conversion."""
    rng = np.random.default_rng(12)
    ds = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 6, 3000),
                         np.array([0.0, -0.0, 65504.0, 65519.999, 65520.0, 2 ** -24, 2 ** -25,
                                   3 * 2 ** -26, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 6.1e-5])])
    with np.errstate(over="ignore"):
        ref = ds.astype(np.float16).view(np.uint16)
    got = np.array([o.round_f16(float(d)) for d in ds], np.uint16)
    assert np.array_equal(got, ref), "f16 rounding differs from numpy"


def pin_widening(o):
    """Element loads: exact widening of bf16 (torch) and f16 (numpy) codes."""
    import torch
    codes = np.arange(0, 0x10000, 97, dtype=np.uint16)
    bf = o.to_double(codes, W.BF16)
    ref_bf = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(bf), np.isnan(ref_bf))
    m = ~np.isnan(ref_bf)
    assert np.array_equal(bf[m], ref_bf[m])
    hf = o.to_double(codes, W.F16)
    ref_hf = codes.view(np.float16).astype(np.float64)
    m = ~np.isnan(ref_hf)
    assert np.array_equal(np.isnan(hf), np.isnan(ref_hf)) and np.array_equal(hf[m], ref_hf[m])


# ----------------------------------------------------------------------------
# Routing preparation.
# ----------------------------------------------------------------------------

def _check_prep_vs_numpy(o, top, E, m):
    r = o.route_prep(top, E, pad_multiple=m)
    flat = np.asarray(top, np.int64).reshape(-1)
    valid = np.flatnonzero((flat >= 0) & (flat < E))
    # stable argsort of the valid ids by expert
    order = valid[np.argsort(flat[valid], kind="stable")]
    n = order.shape[0]
    assert r.n == n
    assert np.array_equal(r.indices[:n], order), "indices != numpy stable argsort"
    assert np.all(r.indices[n:] == -1) and np.all(r.bin_ids[n:] == -1)
    assert np.array_equal(r.bin_ids[:n], flat[order])
    counts = np.bincount(flat[valid], minlength=E)
    assert np.array_equal(r.tokens_per_expert, counts)
    assert np.array_equal(r.bins, np.cumsum(counts))
    if m is not None:
        assert np.array_equal(r.padded_bins, np.cumsum(-(-counts // m) * m))
    return r


def pin_route_prep_numpy(o):
    """indices/bin_ids/counts/bins/padded_bins vs numpy argsort(kind=stable),
    bincount and cumsum, on random routings with -1 slots and skew."""
    rng = np.random.default_rng(21)
    for (T, K, E, nf, skew, m) in [(37, 2, 5, 0.0, 0.0, 4), (64, 4, 8, 0.2, 0.5, 3), (16, 3, 3, 0.5, 0.0, 1),
                                   (100, 8, 64, 0.1, 0.1, 16), (5, 1, 7, 0.0, 2.0, 2), (50, 2, 2, 0.3, 0.0, 7)]:
        top, _ = W.random_routing(rng, T, K, E, none_frac=nf, skew=skew)
        _check_prep_vs_numpy(o, top, E, m)
    # out-of-range expert ids also mean "no route"
    top = np.array([[0, 5], [-7, 1], [2, 3]], np.int32)
    _check_prep_vs_numpy(o, top, 3, 2)
    # empty input
    r = o.route_prep(np.zeros((0, 2), np.int32), 4, pad_multiple=8)
    assert r.n == 0 and np.all(r.bins == 0) and np.all(r.padded_bins == 0)


def pin_route_prep_exhaustive(o):
    """Every routing of T*K <= 6 slots over E <= 3 experts (with -1): sorted
    positions by Python's sorted() on (expert, id), padded bins by
    enumeration."""
    for (T, K, E) in [(3, 2, 3), (6, 1, 2), (2, 3, 3), (1, 1, 1)]:
        for combo in itertools.product(range(-1, E), repeat=T * K):
            top = np.array(combo, np.int32).reshape(T, K)
            r = o.route_prep(top, E, pad_multiple=2)
            ids = sorted((v, a) for a, v in enumerate(combo) if v >= 0)
            assert list(r.indices[:len(ids)]) == [a for _, a in ids]
            assert list(r.bin_ids[:len(ids)]) == [v for v, _ in ids]
            counts = [sum(1 for v in combo if v == e) for e in range(E)]
            assert list(r.bins) == list(itertools.accumulate(counts))
            assert list(r.padded_bins) == list(itertools.accumulate(c + (c % 2) for c in counts))


def pin_route_prep_invariants(o):
    """The pages' invariants on the workload routings: bins nondecreasing,
    bins[-1] == n, bin_ids consistent with bins, indices a permutation of the
    valid ids and ascending within each expert, padded segments >= counts,
    < counts + m and multiples of m."""
    for cid in (1, 3):
        wl = W.config(cid, seed=1, with_rows=False)
        m = 128
        r = o.route_prep(wl.top_experts, wl.E, pad_multiple=m)
        b = np.concatenate([[0], r.bins.astype(np.int64)])
        assert np.all(np.diff(b) >= 0) and r.bins[-1] == r.n
        for e in range(wl.E):
            seg = r.bin_ids[b[e]:b[e + 1]]
            assert np.all(seg == e)
            ids = r.indices[b[e]:b[e + 1]]
            assert np.all(np.diff(ids) > 0)
        valid = np.flatnonzero(wl.top_experts.reshape(-1) >= 0)
        assert np.array_equal(np.sort(r.indices[:r.n]), valid)
        pb = np.concatenate([[0], r.padded_bins.astype(np.int64)])
        segs, counts = np.diff(pb), np.diff(b)
        assert np.all(segs >= counts) and np.all(segs < counts + m) and np.all(segs % m == 0)
        if cid == 3:
            # the workload asks for two overflowing experts and one empty one
            assert int(np.sum(counts > wl.capacity)) == 2 and int(np.sum(counts == 0)) == 1


def pin_golden(o):
    """The hand-worked example: every integer output and every float output."""
    g = _golden()
    top = np.array(g["top_experts"], np.int32)
    E, K = g["E"], g["K"]
    r = o.route_prep(top, E, pad_multiple=g["pad_multiple"])
    assert list(r.indices) == g["indices"] and list(r.bin_ids) == g["bin_ids"]
    assert list(r.tokens_per_expert) == g["tokens_per_expert"] and list(r.bins) == g["bins"]
    assert list(r.padded_bins) == g["padded_bins"]
    C = g["capacity"]
    assert list(o.assignment_rows(r, W.BINNED, C)) == g["binned_rows"]
    assert list(o.assignment_rows(r, W.PADDED)) == g["padded_rows"]
    x = np.array(g["x"], np.float32)
    grad = np.array(g["grad"], np.float32)
    w = np.array(g["weights"], np.float32).reshape(-1)
    for layout, cap, key in ((W.BINNED, C, "binned"), (W.PADDED, None, "padded")):
        y = o.gather(x, r, layout, cap)
        assert np.array_equal(y, np.array(g[key + "_gather"], np.float32)), key + " gather"
        s = o.scatter_combine(y, W.F32, r, layout, cap, weights=w)
        assert np.array_equal(s, np.array(g[key + "_scatter"], np.float32)), key + " scatter"
        wg = o.wgrad(y, grad, W.F32, r, layout, cap)
        assert np.array_equal(wg, np.array(g[key + "_wgrad"], np.float32)), key + " wgrad"
    c = g["compaction"]
    T = len(c["routing_map"])
    probs = np.array([[(8 * t + e + 1) / 64 for e in range(c["E"])] for t in range(T)], np.float32)
    pout, idx = o.routing_map_compact(probs, W.F32, np.array(c["routing_map"], np.uint8), c["topk"])
    assert idx.tolist() == c["route_experts"]
    assert np.array_equal(pout, np.array(c["probs_out"], np.float32))


# ----------------------------------------------------------------------------
# Gathers.
# ----------------------------------------------------------------------------

def _tiny_cases():
    """Small routings covering the pages' verification lists: empty experts,
    overflow, exact capacity, several experts per block, TOP_K 1/2/4/8,
    counts m-1 / m / m+1, -1 slots."""
    rng = np.random.default_rng(31)
    cases = []
    for (T, K, E, nf, skew) in [(24, 2, 5, 0.1, 0.8), (16, 1, 4, 0.0, 0.0), (12, 4, 6, 0.2, 0.3),
                                (9, 8, 8, 0.1, 0.0), (30, 2, 3, 0.0, 1.5)]:
        top, w = W.random_routing(rng, T, K, E, none_frac=nf, skew=skew)
        cases.append((top, w, E))
    # exact capacity / multiple: expert 0 gets exactly 4 assignments
    top = np.array([[0, 1], [0, 2], [0, 1], [0, 2], [1, 2]], np.int32)
    cases.append((top, np.full((5, 2), 0.5, np.float32), 3))
    return cases


def pin_assignment_rows(o):
    """The row of every assignment (the map every GPU test compares slot_row
    with) against the per-expert enumeration, on the tiny routings, for both
    layouts and several capacities and padding multiples; plus the counts
    the pages fix: kept rows per expert = min(count, C) (binned) and the rows
    of a padded segment start at the previous segment's rounded-up end."""
    for top, _, E in _tiny_cases():
        flat = top.reshape(-1)
        counts = np.bincount(flat[flat >= 0], minlength=E)
        for C in (1, 2, 3, 5, 64):
            r = o.route_prep(top, E)
            got = o.assignment_rows(r, W.BINNED, C)
            want, _ = brute_rows(top, E, W.BINNED, capacity=C)
            assert np.array_equal(got, want), f"binned rows C={C}"
            kept = got[got >= 0]
            assert len(np.unique(kept)) == len(kept)
            assert np.array_equal(np.bincount(kept // C, minlength=E), np.minimum(counts, C))
        for m in (1, 2, 3, 4, 8):
            r = o.route_prep(top, E, pad_multiple=m)
            got = o.assignment_rows(r, W.PADDED)
            want, _ = brute_rows(top, E, W.PADDED, pad_multiple=m)
            assert np.array_equal(got, want), f"padded rows m={m}"
            starts = np.concatenate([[0], np.cumsum(-(-counts // m) * m)[:-1]])
            for e in range(E):
                mine = got[flat == e]
                assert np.array_equal(np.sort(mine), starts[e] + np.arange(counts[e])), f"padded segment {e}"


def pin_gather_numpy(o):
    """Gathers vs numpy fancy indexing into a zero tensor, with rows from the
    per-expert enumeration; also: zero rows are exactly zero, the number of
    dropped assignments is sum(max(0, count - C)), and the sampled-row form
    equals the full tensor's rows."""
    rng = np.random.default_rng(32)
    for top, _, E in _tiny_cases():
        T, K = top.shape
        x = W.normal(rng, (T, 5), W.F32)
        flat = top.reshape(-1)
        counts = np.bincount(flat[flat >= 0], minlength=E)
        for C in (1, 2, 3, 4, 64):
            r = o.route_prep(top, E)
            rows, R = brute_rows(top, E, W.BINNED, capacity=C)
            want = np.zeros((R, 5), np.float32)
            kept = np.flatnonzero(rows >= 0)
            want[rows[kept]] = x[kept // K]
            got = o.gather(x, r, W.BINNED, C)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"binned gather C={C}"
            assert len(kept) == int(np.sum(np.minimum(counts, C)))
            assert int(np.sum(flat >= 0)) - len(kept) == int(np.sum(np.maximum(0, counts - C)))
            sample = np.array([R - 1, 0, R // 2], np.int64)
            assert np.array_equal(o.gather(x, r, W.BINNED, C, rows=sample), got[sample])
        for m in (1, 2, 3, 4, 8):
            r = o.route_prep(top, E, pad_multiple=m)
            rows, R = brute_rows(top, E, W.PADDED, pad_multiple=m)
            assert R == o.expert_rows(r, W.PADDED)
            want = np.zeros((R, 5), np.float32)
            kept = np.flatnonzero(rows >= 0)
            want[rows[kept]] = x[kept // K]
            got = o.gather(x, r, W.PADDED)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"padded gather m={m}"


def pin_gather_empty_batch(o):
    """No tokens (T = 0): the binned tensor is E * C rows of zeros, the padded
    one has no rows, whatever memory the output is allocated in (freed
    non-zero buffers of the same size are reused by the allocator)."""
    for H, dtype in ((2, W.F32), (5, W.BF16)):
        x = W.normal(np.random.default_rng(33), (0, H), dtype)
        top = np.zeros((0, 3), np.int32)
        for E, C in ((129, 1), (4, 7)):
            r = o.route_prep(top, E, pad_multiple=4)
            for _ in range(3):
                junk = np.full((E * C, H), 0x55, x.dtype)
                del junk
                got = o.gather(x, r, W.BINNED, C)
                assert got.shape == (E * C, H) and not np.any(got.view(np.uint8)), "empty binned gather"
            assert o.gather(x, r, W.PADDED).shape == (0, H)


def pin_gather_bits_and_identity(o):
    """Gather is a bit copy (NaN payloads, -0.0, subnormals survive), and with
    E = 1, K = 1, C = T (or m = 1) it reproduces x exactly."""
    bits = np.array([[0x7FC1, 0x8000, 0x0001, 0xFF80], [0x3F80, 0x7F81, 0x807F, 0x0000],
                     [0x1234, 0xABCD, 0x7FFF, 0xFFFF]], np.uint16)
    top = np.zeros((3, 1), np.int32)
    r = o.route_prep(top, 1, pad_multiple=1)
    assert np.array_equal(o.gather(bits, r, W.BINNED, 3), bits)
    assert np.array_equal(o.gather(bits, r, W.PADDED), bits)


# ----------------------------------------------------------------------------
# Scatter-combine and wgrad.
# ----------------------------------------------------------------------------

def _ulp_close(got, want, dtype):
    """|got - want| <= 1 ulp of the output format at |want| (plus a floor)."""
    g = W.to_f32(got, dtype).astype(np.float64)
    eps = {W.F32: 2.0 ** -23, W.BF16: 2.0 ** -7, W.F16: 2.0 ** -10}[dtype]
    tiny = {W.F32: 2.0 ** -140, W.BF16: 2.0 ** -126, W.F16: 2.0 ** -24}[dtype]
    return np.all(np.abs(g - want) <= eps * np.abs(want) + tiny)


def pin_scatter_closed_form(o):
    """With y = gather(x): combine(y, w)[t] = (sum of kept w) * x_t;
    unweighted: kept_count(t) * x_t; E = K = 1 with ample capacity gives x
    back bit for bit."""
    rng = np.random.default_rng(41)
    for top, w, E in _tiny_cases():
        T, K = top.shape
        for dtype in (W.F32, W.BF16, W.F16):
            x = W.normal(rng, (T, 6), dtype)
            xf = W.to_f32(x, dtype).astype(np.float64)
            for layout, cap, m in ((W.BINNED, 2, None), (W.BINNED, 64, None), (W.PADDED, None, 4)):
                r = o.route_prep(top, E, pad_multiple=m)
                rows, _ = brute_rows(top, E, layout, capacity=cap, pad_multiple=m)
                kept = (rows >= 0).reshape(T, K)
                y = o.gather(x, r, layout, cap)
                s = o.scatter_combine(y, dtype, r, layout, cap, weights=w.reshape(-1))
                ws = np.where(kept, w.astype(np.float64), 0.0).sum(axis=1)
                assert _ulp_close(s, ws[:, None] * xf, dtype), "weighted closed form"
                s1 = o.scatter_combine(y, dtype, r, layout, cap)
                assert _ulp_close(s1, kept.sum(axis=1)[:, None] * xf, dtype), "unweighted closed form"
    x = W.normal(rng, (7, 5), W.BF16)
    r = o.route_prep(np.zeros((7, 1), np.int32), 1, pad_multiple=1)
    for layout, cap in ((W.BINNED, 7), (W.PADDED, None)):
        assert np.array_equal(o.scatter_combine(o.gather(x, r, layout, cap), W.BF16, r, layout, cap), x)


def _torch_combine(y64, rows, w64, T, K):
    """out = index_add over kept assignments of w * y[row] (torch, float64)."""
    import torch
    rows_t = torch.from_numpy(rows)
    kept = torch.nonzero(rows_t >= 0).reshape(-1)
    tok = kept // K
    terms = w64[kept].unsqueeze(1) * y64[rows_t[kept]]
    out = torch.zeros((T, y64.shape[1]), dtype=torch.float64)
    return out.index_add(0, tok, terms)


def pin_scatter_random_y(o):
    """Combine on an independent random expert tensor vs torch index_add in
    float64 (rounded output within one ulp); unused rows hold NaN and must
    not reach the output."""
    import torch
    rng = np.random.default_rng(42)
    for top, w, E in _tiny_cases():
        T, K = top.shape
        for dtype in (W.F32, W.BF16):
            for layout, cap, m in ((W.BINNED, 3, None), (W.PADDED, None, 2)):
                r = o.route_prep(top, E, pad_multiple=m)
                rows, R = brute_rows(top, E, layout, capacity=cap, pad_multiple=m)
                y = W.expert_tensor_rows(rng, R, 4, dtype, used_rows=rows[rows >= 0])
                s = o.scatter_combine(y, dtype, r, layout, cap, weights=w.reshape(-1))
                y64 = torch.from_numpy(W.to_f32(y, dtype).astype(np.float64))
                want = _torch_combine(y64, rows, torch.from_numpy(w.reshape(-1).astype(np.float64)), T, K)
                assert not np.any(np.isnan(W.to_f32(s, dtype)))
                assert _ulp_close(s, want.numpy(), dtype), "combine vs torch index_add"


def pin_wgrad_autograd(o):
    """wgrad == d/dw of sum(grad * combine(y, w)) by torch autograd (float64),
    on independent random y; dropped and unrouted assignments get 0."""
    import torch
    rng = np.random.default_rng(51)
    for top, w, E in _tiny_cases():
        T, K = top.shape
        for layout, cap, m in ((W.BINNED, 2, None), (W.PADDED, None, 3)):
            r = o.route_prep(top, E, pad_multiple=m)
            rows, R = brute_rows(top, E, layout, capacity=cap, pad_multiple=m)
            y = W.expert_tensor_rows(rng, R, 7, W.F32, used_rows=rows[rows >= 0])
            grad = W.normal(rng, (T, 7), W.F32)
            wg = o.wgrad(y, grad, W.F32, r, layout, cap)
            y64 = torch.from_numpy(np.nan_to_num(y.astype(np.float64)))
            wt = torch.from_numpy(w.reshape(-1).astype(np.float64)).requires_grad_(True)
            out = _torch_combine(y64, rows, wt, T, K)
            (out * torch.from_numpy(grad.astype(np.float64))).sum().backward()
            want = wt.grad.numpy().reshape(T, K)
            assert np.allclose(wg, want, rtol=2e-7, atol=1e-30), "wgrad vs autograd"
            assert np.all(wg.reshape(-1)[rows < 0] == 0.0)


def pin_wgrad_closed_form(o):
    """With y = gather(x): wgrad[t, k] = <x_t, grad_t> for each kept k."""
    rng = np.random.default_rng(52)
    for top, _, E in _tiny_cases():
        T, K = top.shape
        for dtype in (W.F32, W.BF16):
            x = W.normal(rng, (T, 9), dtype)
            grad = W.normal(rng, (T, 9), dtype)
            dots = (W.to_f32(x, dtype).astype(np.float64) * W.to_f32(grad, dtype).astype(np.float64)).sum(1)
            for layout, cap, m in ((W.BINNED, 3, None), (W.PADDED, None, 5)):
                r = o.route_prep(top, E, pad_multiple=m)
                rows, _ = brute_rows(top, E, layout, capacity=cap, pad_multiple=m)
                kept = (rows >= 0).reshape(T, K)
                wg = o.wgrad(o.gather(x, r, layout, cap), grad, dtype, r, layout, cap)
                want = np.where(kept, dots[:, None], 0.0).astype(np.float32)
                assert np.array_equal(wg, want), "wgrad closed form"


def pin_sampled_tokens(o):
    """Token-sampled combine and gradient equal the rows of the full result."""
    rng = np.random.default_rng(53)
    top, w, E = _tiny_cases()[0]
    T, K = top.shape
    r = o.route_prep(top, E, pad_multiple=4)
    y = o.gather(W.normal(rng, (T, 8), W.BF16), r, W.PADDED)
    grad = W.normal(rng, (T, 8), W.BF16)
    tok = np.array([T - 1, 3, 0, 3], np.int64)
    full = o.scatter_combine(y, W.BF16, r, W.PADDED, weights=w.reshape(-1))
    assert np.array_equal(o.scatter_combine(y, W.BF16, r, W.PADDED, weights=w.reshape(-1), tokens=tok), full[tok])
    fw = o.wgrad(y, grad, W.BF16, r, W.PADDED)
    assert np.array_equal(o.wgrad(y, grad, W.BF16, r, W.PADDED, tokens=tok), fw[tok])


def pin_combine_backward(o):
    """Gradient of the combine w.r.t. the expert tensor vs torch autograd of
    the index_add combine (float64, rounded output within one ulp); rows that
    hold no kept assignment get exactly 0; without weights it is the gather of
    the upstream gradient, bit for bit; the row sample equals the full rows."""
    import torch
    rng = np.random.default_rng(81)
    for top, w, E in _tiny_cases():
        T, K = top.shape
        for dtype in (W.F32, W.BF16):
            for layout, cap, m in ((W.BINNED, 2, None), (W.PADDED, None, 4)):
                r = o.route_prep(top, E, pad_multiple=m)
                rows, R = brute_rows(top, E, layout, capacity=cap, pad_multiple=m)
                dout = W.normal(rng, (T, 5), dtype)
                y64 = torch.zeros((R, 5), dtype=torch.float64, requires_grad=True)
                out = _torch_combine(y64, rows, torch.from_numpy(w.reshape(-1).astype(np.float64)), T, K)
                (out * torch.from_numpy(W.to_f32(dout, dtype).astype(np.float64))).sum().backward()
                dy = o.combine_backward_dy(dout, dtype, r, layout, cap, weights=w.reshape(-1))
                assert _ulp_close(dy, y64.grad.numpy(), dtype), "combine backward vs autograd"
                unused = np.ones(R, bool)
                unused[rows[rows >= 0]] = False
                assert np.all(W.to_f32(dy, dtype)[unused] == 0)
                plain = o.combine_backward_dy(dout, dtype, r, layout, cap)
                assert np.array_equal(plain.view(np.uint8), o.gather(dout, r, layout, cap).view(np.uint8))
                sample = np.array([R - 1, 0, R // 2], np.int64)
                assert np.array_equal(o.combine_backward_dy(dout, dtype, r, layout, cap, weights=w.reshape(-1),
                                                            rows=sample).view(np.uint8), dy[sample].view(np.uint8))


def pin_windows(o):
    """Rows within per-expert windows vs brute-force enumeration: windows
    [e*C, (e+1)*C) give the binned rows, windows [pstart(e), padded_bins[e])
    the padded rows, and a batch cut into contiguous token shards, each
    routed on its own with windows that start where the earlier shards'
    assignments of each expert end, reproduces the binned rows of the whole
    batch."""
    rng = np.random.default_rng(83)
    for top, w, E in _tiny_cases():
        T, K = top.shape
        r = o.route_prep(top, E)
        for C in (1, 2, 5):
            want, _ = brute_rows(top, E, W.BINNED, capacity=C)
            base = np.arange(E, dtype=np.int32) * C
            got = o.assignment_rows_windows(r, base, base + C)
            assert np.array_equal(got, want), "windows = binned rows"
        m = 3
        rp = o.route_prep(top, E, pad_multiple=m)
        want, _ = brute_rows(top, E, W.PADDED, pad_multiple=m)
        pstart = np.concatenate([[0], rp.padded_bins[:-1]]).astype(np.int32)
        assert np.array_equal(o.assignment_rows_windows(rp, pstart, rp.padded_bins), want), "windows = padded rows"
        if T >= 3:
            C = 2
            want, _ = brute_rows(top, E, W.BINNED, capacity=C)
            cuts = sorted(rng.choice(np.arange(1, T), size=2, replace=False).tolist())
            taken = np.zeros(E, np.int64)
            got = []
            for lo, hi in zip([0] + cuts, cuts + [T]):
                rs = o.route_prep(top[lo:hi], E)
                base = (np.arange(E) * C + taken).astype(np.int32)
                got.append(o.assignment_rows_windows(rs, base, (np.arange(E, dtype=np.int32) + 1) * C))
                taken += rs.tokens_per_expert
            assert np.array_equal(np.concatenate(got), want), "sharded windows = rows of the whole batch"


# ----------------------------------------------------------------------------
# Routing-map compaction.
# ----------------------------------------------------------------------------

def pin_compaction(o):
    """Compaction vs np.flatnonzero(row)[:topk] with probs gathered; valid
    prefix strictly increasing, -1 only as a suffix; backward vs torch
    autograd of the gather that defines the forward."""
    import torch
    rng = np.random.default_rng(61)
    for (T, E, topk, maxr) in [(40, 16, 4, 6), (33, 64, 8, 8), (10, 5, 5, 5), (8, 200, 3, 10)]:
        rmap = W.routing_map_rows(rng, T, E, maxr)
        for pdt in (W.F32, W.BF16):
            probs = W.normal(rng, (T, E), pdt)
            pout, idx = o.routing_map_compact(probs, pdt, rmap, topk)
            pf = W.to_f32(probs, pdt)
            for t in range(T):
                nz = np.flatnonzero(rmap[t])[:topk]
                c = len(nz)
                assert list(idx[t, :c]) == list(nz) and np.all(idx[t, c:] == -1)
                assert np.array_equal(pout[t, :c], pf[t, nz]) and np.all(pout[t, c:] == 0)
        g = rng.standard_normal((T, topk)).astype(np.float32)
        dense = o.routing_map_compact_backward(g, idx, E)
        pt = torch.zeros((T, E), dtype=torch.float64, requires_grad=True)
        it = torch.from_numpy(idx.astype(np.int64))
        fwd = torch.gather(pt, 1, it.clamp(min=0)) * (it >= 0)
        (fwd * torch.from_numpy(g.astype(np.float64))).sum().backward()
        assert np.array_equal(dense, pt.grad.numpy().astype(np.float32)), "compaction backward vs autograd"


# ----------------------------------------------------------------------------
# Router top-k gating.
# ----------------------------------------------------------------------------

def _brute_rank(row):
    """Experts of one score row in rank order, by a full sort: numbers by
    decreasing value (-0 and +0 equal), then NaN, lower id first on ties."""
    return sorted(range(len(row)), key=lambda e: (1, 0.0, e) if math.isnan(row[e]) else (0, -float(row[e]), e))


def _f32_ulps(a, b):
    """Distance in float32 units in the last place (finite, same sign)."""
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def pin_router_selection(o):
    """Top-k selection vs a full sort on rows full of ties, signed zeros,
    infinities and NaN, in all three score formats."""
    rng = np.random.default_rng(91)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1.0, -1.0, 2.0], np.float32)
    for E, K in [(1, 1), (5, 2), (8, 8), (16, 3), (64, 8), (70, 5), (257, 9)]:
        T = 24
        base = rng.integers(-3, 4, size=(T, E)).astype(np.float32)  # many exact ties
        pick = rng.random((T, E)) < 0.15
        base[pick] = specials[rng.integers(0, len(specials), size=int(pick.sum()))]
        base[0] = np.nan                       # a row of NaN only
        base[1] = -np.inf                      # a row of -inf only
        for dtype in (W.F32, W.BF16, W.F16):
            lg = W.cast_from_f32(base, dtype)  # exact: small integers and specials
            top, _ = o.router_topk(lg, dtype, K)
            for t in range(T):
                assert list(top[t]) == _brute_rank(base[t])[:K], (E, K, dtype, t)
            top_s, _ = o.router_topk(lg, dtype, K, gating=o.SIGMOID)
            assert np.array_equal(top_s, top)  # the ranking does not depend on the gating


def pin_router_weights_library(o):
    """Weights vs scipy.special.softmax (and the logistic function from
    scipy.special.expit) in float64, rounded to float32: equal within one
    float32 ulp (both are double evaluations rounded once); large offsets
    included, where exp without the maximum shift overflows."""
    from scipy.special import expit, softmax
    rng = np.random.default_rng(92)
    for E, K, off in [(8, 2, 0.0), (64, 8, 0.0), (256, 8, 0.0), (33, 33, 0.0), (8, 2, 800.0), (16, 4, -900.0)]:
        T = 16
        lg = (rng.standard_normal((T, E)) * 3 + off).astype(np.float32)
        for gating in (o.SOFTMAX, o.SIGMOID):
            for norm in (True, False):
                top, w = o.router_topk(lg, W.F32, K, gating=gating, normalize=norm)
                for t in range(T):
                    sel = np.array(_brute_rank(lg[t])[:K])
                    assert np.array_equal(top[t], sel)
                    x = lg[t].astype(np.float64)
                    p = softmax(x)[sel] if gating == o.SOFTMAX else expit(x[sel])
                    if norm:
                        with np.errstate(invalid="ignore"):
                            p = p / p.sum()
                    want = p.astype(np.float32)
                    nan = np.isnan(want)  # 0/0: every selected sigmoid underflowed
                    assert np.array_equal(np.isnan(w[t]), nan), (E, K, off, gating, norm, t)
                    ok = _f32_ulps(w[t][~nan], want[~nan]) <= 1
                    assert ok.all(), (E, K, off, gating, norm, t, w[t], want)


def pin_router_matches_workload_router(o):
    """The 512-token workload's routing (numpy float32 softmax, stable argsort
    of the probabilities, renormalised) is the oracle's softmax gating with
    renormalisation: same experts (its probabilities have no ties), weights
    within float32 evaluation error."""
    wl = W.config(1, 0, with_rows=False)
    top, w = o.router_topk(wl.logits, W.F32, wl.K)
    assert np.array_equal(top, wl.top_experts)
    assert np.all(np.abs(w.astype(np.float64) - wl.weights) <= 1e-6 * np.abs(wl.weights))


def pin_router_closed_forms(o):
    """Hand-worked values: scores (ln 6, ln 3, 0) give softmax (0.6, 0.3, 0.1)
    and top-2 renormalised (2/3, 1/3); scores (ln 3, 0, -ln 3) give sigmoid
    (0.75, 0.5, 0.25), renormalised (0.5, 1/3, 1/6); bf16 scores (0, 0)
    tie -> experts (0, 1), weights (0.5, 0.5)."""
    def near(got, want):
        return bool(np.all(np.abs(np.asarray(got, np.float64) - np.asarray(want)) <= 2e-7 * np.abs(want)))

    lg = np.array([[0.0, math.log(3.0), math.log(6.0)]], np.float32)
    top, w = o.router_topk(lg, W.F32, 3, normalize=False)
    assert list(top[0]) == [2, 1, 0] and near(w[0], [0.6, 0.3, 0.1])
    top, w = o.router_topk(lg, W.F32, 2)
    assert list(top[0]) == [2, 1] and near(w[0], [2 / 3, 1 / 3])
    lg = np.array([[-math.log(3.0), 0.0, math.log(3.0)]], np.float32)
    top, w = o.router_topk(lg, W.F32, 3, gating=o.SIGMOID, normalize=False)
    assert list(top[0]) == [2, 1, 0] and near(w[0], [0.75, 0.5, 0.25])
    top, w = o.router_topk(lg, W.F32, 3, gating=o.SIGMOID)
    assert near(w[0], [0.5, 1 / 3, 1 / 6])
    top, w = o.router_topk(np.zeros((1, 2), np.uint16), W.BF16, 2)
    assert list(top[0]) == [0, 1] and list(w[0]) == [0.5, 0.5]


# ----------------------------------------------------------------------------
# Validation.
# ----------------------------------------------------------------------------

def pin_validate(o):
    """Each planted violation of a page guardrail raises exactly its flag;
    oracle-built routings raise none."""
    rng = np.random.default_rng(71)
    top, _ = W.random_routing(rng, 20, 2, 5, none_frac=0.1)
    r = o.route_prep(top, 5, pad_multiple=4)
    T, K, E, n = 20, 2, 5, r.n
    assert o.validate_routing(r.indices, r.bin_ids, r.bins, r.padded_bins, T, K, E, n) == 0
    assert o.validate_routing(r.indices, r.bin_ids, r.bins, None, T, K, E, -1) == 0
    bins = r.bins.copy(); bins[1], bins[2] = bins[2], bins[1] - 1
    assert o.validate_routing(r.indices, r.bin_ids, bins, None, T, K, E, -1) & 0x1
    assert o.validate_routing(r.indices, r.bin_ids, r.bins, None, T, K, E, n - 1) == 0x2
    bid = r.bin_ids.copy(); bid[0] = 4
    assert o.validate_routing(r.indices, bid, r.bins, None, T, K, E, n) == 0x4
    pb = r.padded_bins.copy(); pb[0] = 0
    assert o.validate_routing(r.indices, r.bin_ids, r.bins, pb, T, K, E, n) == 0x8
    idx = r.indices.copy(); idx[1] = idx[0]
    assert o.validate_routing(idx, r.bin_ids, r.bins, None, T, K, E, n) == 0x10
    idx = r.indices.copy(); idx[2] = T * K
    assert o.validate_routing(idx, r.bin_ids, r.bins, None, T, K, E, n) == 0x10


ALL_PINS = [pin_bf16_rounding, pin_f16_rounding, pin_widening, pin_route_prep_numpy, pin_route_prep_exhaustive,
            pin_route_prep_invariants, pin_golden, pin_assignment_rows, pin_gather_numpy, pin_gather_empty_batch,
            pin_gather_bits_and_identity,
            pin_scatter_closed_form, pin_scatter_random_y, pin_wgrad_autograd, pin_wgrad_closed_form,
            pin_sampled_tokens, pin_combine_backward, pin_windows, pin_compaction, pin_router_selection,
            pin_router_weights_library, pin_router_matches_workload_router, pin_router_closed_forms, pin_validate]
