"""Seeded synthetic inputs for the MoE token-routing data path.

This module is shared by the GPU tests, the benchmark and the oracle tests.
It holds none of the data path's own arithmetic (no sorting by expert, no
bins, no row mapping, no gather/combine/gradient math). It only draws
inputs: router top-k choices (the router sits upstream of the path),
weights, token rows, upstream gradients and dense routing maps.

Recipe (numpy ``default_rng(seed)``; draws in this fixed order):
  1. configuration-specific expert bias or route draws;
  2. router logits [T, E] ~ N(0, 1), float32, plus the bias;
  3. token rows x [T, H] ~ N(0, 1);
  4. upstream gradient grad [T, H] ~ N(0, 1).
Floats are drawn as float32; bfloat16 / float16 inputs are the
round-to-nearest-even images of those draws (raw bit patterns in uint16).
Router: softmax over E in float32, top-K by descending probability with the
lower expert id first on ties, weights renormalised over the K choices.
"""
import math
from dataclasses import dataclass, field

import numpy as np

F32, BF16, F16 = 0, 1, 2
BINNED, PADDED = 0, 1
DTYPE_NAMES = {F32: "f32", BF16: "bf16", F16: "f16"}


def f32_to_bf16_bits(a):
    """Round float32 values to bfloat16 (nearest even); returns uint16 bits.
    Processed in slices so that large draws need little temporary memory."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    flat = a.reshape(-1)
    out = np.empty(flat.shape[0], np.uint16)
    step = 1 << 24
    for s in range(0, flat.shape[0], step):
        u = flat[s:s + step].view(np.uint32)
        # finite inputs: u + 0x8000 never wraps (largest finite pattern 0xFF7FFFFF)
        r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
        nan = np.isnan(flat[s:s + step])
        if nan.any():
            r[nan] = 0x7FC0
        out[s:s + step] = r
    return out.reshape(a.shape)


def bf16_bits_to_f32(b):
    """Widen bfloat16 bits to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def cast_from_f32(a, dtype):
    """Input-generation cast of float32 draws to the element type's storage."""
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(a)
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_f32(a, dtype):
    """Element storage back to float32 (exact for all three types)."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float32)


def normal(rng, shape, dtype):
    """N(0, 1) float32 draws stored in ``dtype``."""
    return cast_from_f32(rng.standard_normal(shape, dtype=np.float32), dtype)


def softmax_topk(logits, K):
    """Router: float32 softmax, top-K (ties -> lower id), renormalised weights."""
    logits = np.asarray(logits, dtype=np.float32)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m, dtype=np.float32)
    p = p / p.sum(axis=1, keepdims=True, dtype=np.float32)
    order = np.argsort(-p, axis=1, kind="stable")[:, :K]
    w = np.take_along_axis(p, order, axis=1).astype(np.float32)
    w = (w / w.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return order.astype(np.int32), w


@dataclass
class Workload:
    """One synthetic routed batch."""
    name: str
    T: int
    H: int
    E: int
    K: int
    dtype: int
    layout: int
    capacity: int = 0          # binned
    pad_multiple: int = 0      # padded
    top_experts: np.ndarray = None   # [T, K] int32 (-1 = none); None when compaction makes it
    weights: np.ndarray = None       # [T, K] float32
    x: np.ndarray = None             # [T, H] dtype storage
    grad: np.ndarray = None          # [T, H] dtype storage
    logits: np.ndarray = None        # [T, E] float32 router scores (bias included) the routing came from
    probs: np.ndarray = None         # [T, E] float32 (compaction configs)
    routing_map: np.ndarray = None   # [T, E] uint8 (compaction configs)
    topk: int = 0                    # compaction width
    seed: int = 0
    notes: dict = field(default_factory=dict)


def _finish(rng, wl, with_rows=True):
    if with_rows:
        wl.x = normal(rng, (wl.T, wl.H), wl.dtype)
        wl.grad = normal(rng, (wl.T, wl.H), wl.dtype)
    return wl


def config(cid, seed=0, with_rows=True):
    """The five reference workloads (cid 1..5)."""
    rng = np.random.default_rng(seed)
    if cid == 1:
        # Binned, fp32, T512 H250 E8 K2, capacity = ceil(T*K/E) = 128.
        T, H, E, K = 512, 250, 8, 2
        logits = rng.standard_normal((T, E), dtype=np.float32)
        top, w = softmax_topk(logits, K)
        wl = Workload("binned-f32-T512-H250-E8-K2-C128", T, H, E, K, F32, BINNED,
                      capacity=math.ceil(T * K / E), top_experts=top, weights=w, logits=logits, seed=seed)
        return _finish(rng, wl, with_rows)
    if cid == 2:
        # Padded, bf16, Mixtral-8x7B-shaped: T4096 H4096 E8 K2, multiple 128.
        T, H, E, K = 4096, 4096, 8, 2
        logits = rng.standard_normal((T, E), dtype=np.float32)
        top, w = softmax_topk(logits, K)
        wl = Workload("padded-bf16-T4096-H4096-E8-K2-m128", T, H, E, K, BF16, PADDED,
                      pad_multiple=128, top_experts=top, weights=w, logits=logits, seed=seed)
        return _finish(rng, wl, with_rows)
    if cid == 3:
        # Binned, bf16, Mixtral-8x22B-shaped: T16384 H6144 E8 K2, capacity factor
        # 1.25. Zipf(1.2) log-bias over a seeded expert permutation; the
        # lowest-ranked expert is masked so that exactly one receives no token.
        T, H, E, K = 16384, 6144, 8, 2
        ranks = np.arange(1, E + 1, dtype=np.float64)
        p = ranks ** -1.2
        p /= p.sum()
        perm = rng.permutation(E)
        bias = np.empty(E, np.float32)
        bias[perm] = np.log(p).astype(np.float32)
        bias[perm[E - 1]] = -np.inf
        logits = rng.standard_normal((T, E), dtype=np.float32) + bias
        top, w = softmax_topk(logits, K)
        wl = Workload("binned-bf16-T16384-H6144-E8-K2-C5120", T, H, E, K, BF16, BINNED,
                      capacity=math.ceil(1.25 * T * K / E), top_experts=top, weights=w, logits=logits, seed=seed,
                      notes={"zipf_perm": perm.tolist()})
        return _finish(rng, wl, with_rows)
    if cid == 4:
        # Routing-map compaction + padded, bf16, DeepSeek-V3-shaped:
        # T8192 H7168 E256 topk 8; 0..8 routed experts per row, uniformly;
        # probs = softmax(N(0,1)) over 256, not renormalised; multiple 128.
        T, H, E, K = 8192, 7168, 256, 8
        counts = rng.integers(0, K + 1, size=T)
        rmap = np.zeros((T, E), np.uint8)
        for t in range(T):
            rmap[t, rng.choice(E, counts[t], replace=False)] = 1
        z = rng.standard_normal((T, E), dtype=np.float32)
        z = z - z.max(axis=1, keepdims=True)
        pe = np.exp(z, dtype=np.float32)
        probs = (pe / pe.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
        wl = Workload("compact-padded-bf16-T8192-H7168-E256-K8-m128", T, H, E, K, BF16, PADDED,
                      pad_multiple=128, probs=probs, routing_map=rmap, topk=K, seed=seed)
        return _finish(rng, wl, with_rows)
    if cid == 5:
        # Binned, bf16, Qwen2-MoE-57B-shaped: T32768 H3584 E64 K8, capacity
        # factor 1.0; per-expert bias ~ N(0, 2) read as standard deviation 2.
        T, H, E, K = 32768, 3584, 64, 8
        bias = rng.normal(0.0, 2.0, E).astype(np.float32)
        logits = rng.standard_normal((T, E), dtype=np.float32) + bias
        top, w = softmax_topk(logits, K)
        wl = Workload("binned-bf16-T32768-H3584-E64-K8-C4096", T, H, E, K, BF16, BINNED,
                      capacity=math.ceil(1.0 * T * K / E), top_experts=top, weights=w, logits=logits, seed=seed)
        return _finish(rng, wl, with_rows)
    raise ValueError(f"unknown workload {cid}")


def random_routing(rng, T, K, E, none_frac=0.0, skew=0.0, one_expert=None):
    """Top-K routes without repeats per token: random experts (optionally
    skewed towards low ids), a fraction of slots set to -1 (no route), or all
    routes of every token sent to the same expert set when ``one_expert``."""
    top = np.empty((T, K), np.int32)
    if skew > 0:
        p = np.exp(-skew * np.arange(E))
        p /= p.sum()
    else:
        p = None
    for t in range(T):
        if one_expert is not None:
            top[t] = (one_expert + np.arange(K)) % E
        else:
            top[t] = rng.choice(E, K, replace=False, p=p)
    if none_frac > 0:
        top[rng.random((T, K)) < none_frac] = -1
    w = rng.random((T, K), dtype=np.float32) + np.float32(0.05)
    w = (w / w.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return top, w


def routing_map_rows(rng, T, E, max_routes):
    """Dense routing map with a uniform 0..max_routes routed experts per row."""
    counts = rng.integers(0, max_routes + 1, size=T)
    rmap = np.zeros((T, E), np.uint8)
    for t in range(T):
        rmap[t, rng.choice(E, min(counts[t], E), replace=False)] = 1
    return rmap


def expert_tensor_rows(rng, R, H, dtype, used_rows=None):
    """Independent random expert tensor [R, H]; rows not in ``used_rows`` hold
    NaN (a sentinel: a correct combine/gradient never reads them)."""
    y = normal(rng, (R, H), dtype)
    if used_rows is not None:
        mask = np.ones(R, bool)
        mask[np.asarray(used_rows, dtype=np.int64)] = False
        nan = {F32: np.array(np.nan, np.float32), BF16: np.uint16(0x7FC0), F16: np.uint16(0x7E00)}[dtype]
        y[mask] = nan
    return y
