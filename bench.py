"""Benchmark of the MoE token-routing data path on one MI355X.

One step = one pass of the whole path over one routed batch: (routing-map
compaction, for the compaction workload) -> route_prep -> gather (binned or
padded) -> weighted scatter-combine -> wgrad, with every buffer preallocated
and every call going through the C ABI of libpeg.so on torch's current
stream. With --from-logits a step starts from the router scores instead:
gating fused with route_prep replaces route_prep. Steps rotate over several copies of the input (distinct buffers) so
that the bytes of a step are not served from the 256 MB Infinity Cache left
warm by the previous step.

Printed: one JSON line. ``value`` is the effective HBM bandwidth of the step,
(algorithmic bytes of gather + combine + wgrad) / (wall time of the step,
route_prep and compaction included); ``roofline`` is the dominant kernel's
algorithmic bytes / its average duration (HIP events on its stream);
``cpu_baseline`` is the CPU oracle on the same workload, one thread;
``cpu_baseline_threads`` runs independent whole oracle steps on the host
threads this process may use, at most 16 (one GPU's share of the host), with
the host's CPU count and model recorded. ``kernels`` holds per-kernel
durations inside the back-to-back steps; ``kernels_flushed`` the same
kernels with 1 GiB of scratch written and read back before each one
(outside its event pair), so that none of its bytes come from L2 or the
256 MB Infinity Cache and no dirty lines of the flush are written back
during it.
``outside_step`` times (back to back, and with the caches flushed before
each launch),
outside the step, the backward of the combine with wgrad on the same
buffers (dy in the expert layout + the routing-weight gradient), and the
router top-k gating (softmax, renormalised) of the workload's router scores,
alone and fused with route_prep.

Algorithmic bytes per launch (s = element bytes, U = tokens with a kept
route, N = kept assignments, R = expert-tensor rows):
  gather  = U*H*s + R*H*s + 4*T*K + 8*E
  combine = N*H*s + T*H*s + 8*T*K
  wgrad   = N*H*s + U*H*s + 8*T*K
  combine backward = N*H*s (y) + U*H*s (dout) + R*H*s (dy) + 12*T*K
  router gating    = 4*T*E (f32 scores) + 8*T*K (experts + weights)
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0  # MI355X HBM3E
EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


KERNEL_SOURCES = {"gather": "gather.hip", "combine": "combine.hip", "wgrad": "combine.hip",
                  "backward": "combine.hip", "route_prep": "route_prep.hip", "compact": "compact.hip"}


def source_hash(kernel=None):
    """Hash of a kernel's source file and the shared headers (all sources when
    kernel is None): counter data recorded for a kernel is used only while
    this hash is unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "padded_expert_gather_amd", "csrc")
    names = sorted(os.listdir(csrc))
    if kernel is not None:
        names = [n for n in names if n.endswith(".hpp") or n == KERNEL_SOURCES[kernel]]
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    with open(os.path.join(ROOT, "include", "peg.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5,
                    help="workload id 1-5 (default 5: Qwen2-MoE-57B-shaped, the largest one-GPU batch)")
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate over (0: enough for 2 GiB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle time")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the multi-thread CPU-oracle leg (0: the CPUs this process may use, at most 16, "
                         "one GPU's share of the host; 1: skip it)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache-flushed per-op region")
    ap.add_argument("--flush-bytes", type=int, default=1 << 30,
                    help="bytes written and read back before every op of the cache-flushed region "
                         "(>= 1 GiB evicts L2 and MALL)")
    ap.add_argument("--no-events", action="store_true", help="no per-kernel events inside the timed steps")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the fused combine backward")
    ap.add_argument("--no-router", action="store_true", help="skip timing the router gating")
    ap.add_argument("--graph", action="store_true",
                    help="region 1 replays one captured HIP graph per input copy instead of launching the calls")
    ap.add_argument("--from-logits", action="store_true",
                    help="start each step from the router scores: gating fused with route_prep replaces route_prep "
                         "(workloads with router scores)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 1 GiB device-to-device copies (reference for the HBM byte counters) and exit")
    return ap.parse_args()


def copy_calibration(torch):
    """Plain copies of known size: what FETCH_SIZE / WRITE_SIZE read for
    1 GiB in and 1 GiB out calibrates the counters of the data-path kernels."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    for i in range(4):
        bufs[i % 2].copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 4}), flush=True)


def copy_ceiling(torch, hip, tstream):
    """Streaming rates of this GPU measured with torch's own kernels on 1 GiB
    buffers, timed with HIP events (median of 5): device-to-device copy (read
    + write bytes per second), fill (write only), a float32 sum (read only)
    and a bfloat16 add of two buffers into a third (two bytes read per byte
    written). Returns {"copy": GB/s, "write": GB/s, "read": GB/s,
    "add": GB/s}."""
    n = 1 << 30
    stream = ctypes.c_void_p(tstream.cuda_stream)
    with torch.cuda.stream(tstream):
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        def timed(fn):
            fn()
            torch.cuda.synchronize()
            ms = []
            for _ in range(5):
                a, b = hip.create(), hip.create()
                hip.record(a, stream)
                fn()
                hip.record(b, stream)
                torch.cuda.synchronize()
                ms.append(hip.elapsed_ms(a, b))
            return median(ms) / 1e3

        t_copy = timed(lambda: dst.copy_(src))
        t_fill = timed(lambda: dst.fill_(3))
        t_sum = timed(lambda: src.view(torch.float32).sum())
        src2 = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(2)
        a16, b16, c16 = src.view(torch.bfloat16), src2.view(torch.bfloat16), dst.view(torch.bfloat16)
        t_add = timed(lambda: torch.add(a16, b16, out=c16))
    del src, src2, dst
    return {"copy": round(2 * n / t_copy / 1e9, 1), "write": round(n / t_fill / 1e9, 1),
            "read": round(n / t_sum / 1e9, 1), "add": round(3 * n / t_add / 1e9, 1)}


def median(xs):
    ys = sorted(xs)
    return ys[len(ys) // 2]


class HipEvents:
    """HIP events from the process's HIP runtime (the one torch loaded),
    created without the system-scope fence so that recording one between two
    kernels adds no cache flush."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


class Step:
    """Preallocated buffers and precomputed C-ABI arguments of one input copy."""

    def __init__(self, peg, torch, wl, dev, host):
        import workloads as W
        self.W = W
        lib = peg.library()
        self.lib = lib
        T, H, E, K = wl.T, wl.H, wl.E, wl.K
        self.wl = wl
        i32 = dict(dtype=torch.int32, device=dev)
        tdt = {W.F32: torch.float32, W.BF16: torch.bfloat16, W.F16: torch.float16}[wl.dtype]
        self.x = host["x"].to(dev)
        self.grad = host["grad"].to(dev)
        if wl.routing_map is not None:
            self.probs = host["probs"].to(dev)
            self.rmap = host["rmap"].to(dev)
            self.top = torch.empty((T, K), **i32)
            self.w = torch.empty((T, K), dtype=torch.float32, device=dev)
        else:
            self.top = host["top"].to(dev)
            self.w = host["w"].to(dev)
        total = T * K
        self.indices = torch.empty(total, **i32)
        self.bin_ids = torch.empty(total, **i32)
        self.tpe = torch.empty(E, **i32)
        self.bins = torch.empty(E, **i32)
        self.padded_bins = torch.empty(E, **i32) if wl.layout == W.PADDED else None
        self.slot_row = torch.empty(total, **i32)
        self.ws = torch.empty(peg.workspace_bytes(T, K, E), dtype=torch.uint8, device=dev)
        self.R = host["R"]
        self.y = torch.empty((self.R, H), dtype=tdt, device=dev)
        self.out = torch.empty((T, H), dtype=tdt, device=dev)
        self.wg = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.dy = None if host.get("no_backward") else torch.empty((self.R, H), dtype=tdt, device=dev)
        self.wg_b = torch.empty((T, K), dtype=torch.float32, device=dev)
        P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        self.stream = st
        wsb = self.ws.numel()
        cap = wl.capacity or 0
        m = wl.pad_multiple or 0
        self.calls = {}
        if wl.routing_map is not None:
            self.calls["compact"] = (lib.peg_routing_map_compact,
                                     (P(self.probs), 0, P(self.rmap), T, E, wl.topk, P(self.w), P(self.top), st))
        if host.get("from_logits"):
            # gating of the router scores fused with route_prep, into the
            # step's own routing and weight buffers
            self.logits_step = host["logits"].to(dev)
            self.calls["route_prep_logits"] = (
                lib.peg_route_prep_logits,
                (P(self.logits_step), 0, T, E, K, 0, 1, wl.layout, cap, m, P(self.top), P(self.w), P(self.indices),
                 P(self.bin_ids), P(self.tpe), P(self.bins), P(self.padded_bins), P(self.slot_row), P(self.ws), wsb,
                 st))
        else:
            self.calls["route_prep"] = (lib.peg_route_prep,
                                        (P(self.top), T, K, E, wl.layout, cap, m, P(self.indices), P(self.bin_ids),
                                         P(self.tpe), P(self.bins), P(self.padded_bins), P(self.slot_row),
                                         P(self.ws), wsb, st))
        if wl.layout == W.BINNED:
            self.calls["gather"] = (lib.peg_gather_binned,
                                    (P(self.x), wl.dtype, T, H, K, E, cap, P(self.indices), P(self.bin_ids),
                                     P(self.bins), P(self.slot_row), P(self.y), P(self.ws), wsb, st))
        else:
            self.calls["gather"] = (lib.peg_gather_padded,
                                    (P(self.x), wl.dtype, T, H, K, E, P(self.indices), P(self.bin_ids), P(self.bins),
                                     P(self.padded_bins), P(self.slot_row), P(self.y), self.R, None, P(self.ws), wsb,
                                     st))
        self.calls["combine"] = (lib.peg_scatter_combine,
                                 (P(self.y), wl.dtype, wl.layout, T, H, K, E, cap, P(self.indices), P(self.bin_ids),
                                  P(self.bins), P(self.padded_bins), P(self.slot_row), P(self.w), P(self.out),
                                  P(self.ws), wsb, st))
        self.calls["wgrad"] = (lib.peg_wgrad,
                               (P(self.y), P(self.grad), wl.dtype, wl.layout, T, H, K, E, cap, P(self.indices),
                                P(self.bin_ids), P(self.bins), P(self.padded_bins), P(self.slot_row), P(self.wg),
                                P(self.ws), wsb, st))
        self.order = list(self.calls)
        # not part of the step, timed alone: the backward of the combine
        # (dout = grad) and the router gating of the workload's scores
        self.extras = {}
        if self.dy is not None:
            self.extras["combine_backward"] = (
                lib.peg_combine_backward,
                (P(self.y), P(self.grad), P(self.w), wl.dtype, wl.layout, T, H, K, E, cap, P(self.indices),
                 P(self.bin_ids), P(self.bins), P(self.padded_bins), P(self.slot_row), P(self.dy), self.R,
                 P(self.wg_b), P(self.ws), wsb, st))
        if wl.logits is not None and not host.get("no_router"):
            self.logits = host["logits"].to(dev)
            self.r_top = torch.empty((T, K), **i32)
            self.r_w = torch.empty((T, K), dtype=torch.float32, device=dev)
            self.extras["router_topk"] = (lib.peg_router_topk, (P(self.logits), 0, T, E, K, 0, 1, P(self.r_top),
                                                                P(self.r_w), st))
            # gating fused with route_prep, into buffers of its own
            self.f_idx = torch.empty(total, **i32)
            self.f_bid = torch.empty(total, **i32)
            self.f_tpe = torch.empty(E, **i32)
            self.f_bins = torch.empty(E, **i32)
            self.f_pb = torch.empty(E, **i32) if wl.layout == W.PADDED else None
            self.f_slot = torch.empty(total, **i32)
            self.f_ws = torch.empty(peg.workspace_bytes(T, K, E), dtype=torch.uint8, device=dev)
            self.extras["route_prep_logits"] = (
                lib.peg_route_prep_logits,
                (P(self.logits), 0, T, E, K, 0, 1, wl.layout, cap, m, P(self.r_top), P(self.r_w), P(self.f_idx),
                 P(self.f_bid), P(self.f_tpe), P(self.f_bins), P(self.f_pb), P(self.f_slot), P(self.f_ws),
                 self.f_ws.numel(), st))

    def run_extra(self, name, ev=None, hip=None):
        fn, args = self.extras[name]
        if ev is not None:
            hip.record(ev[0], self.stream)
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"{name} failed with status {rc}")
        if ev is not None:
            hip.record(ev[1], self.stream)

    def run(self, events=None, hip=None, before=None):
        """One step; events: {op: (start, end)} recorded around each call;
        before: called before each call (and before its start event)."""
        for name in self.order:
            fn, args = self.calls[name]
            if before is not None:
                before()
            if events is not None:
                hip.record(events[name][0], self.stream)
            rc = fn(*args)
            if rc != 0:
                raise RuntimeError(f"{name} failed with status {rc}")
            if events is not None:
                hip.record(events[name][1], self.stream)


def host_inputs(torch, W, wl, peg, dev):
    """Host tensors of a workload and its expert-tensor row count."""
    def t16(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16 if wl.dtype == W.BF16 else torch.float16)
    conv = (lambda a: torch.from_numpy(a)) if wl.dtype == W.F32 else t16
    host = {"x": conv(wl.x), "grad": conv(wl.grad)}
    if wl.logits is not None:
        host["logits"] = torch.from_numpy(wl.logits)
    if wl.routing_map is not None:
        host["probs"] = torch.from_numpy(wl.probs)
        host["rmap"] = torch.from_numpy(wl.routing_map)
        pg, ig = peg.routing_map_compact(host["probs"].to(dev), host["rmap"].to(dev), wl.topk)
        top_dev = ig
    else:
        host["top"] = torch.from_numpy(wl.top_experts)
        host["w"] = torch.from_numpy(wl.weights)
        top_dev = host["top"].to(dev)
    if wl.layout == W.BINNED:
        r = peg.route_prep(top_dev, wl.E, capacity=wl.capacity)
        R = wl.E * wl.capacity
    else:
        r = peg.route_prep(top_dev, wl.E, pad_multiple=wl.pad_multiple)
        R = r.expert_rows()
    host["R"] = R
    # sizes for the algorithmic byte counts, from the device routing
    kept = (r.slot_row >= 0).reshape(wl.T, wl.K)
    N = int(kept.sum().item())
    U = int(kept.any(dim=1).sum().item())
    return host, dict(R=R, N=N, U=U, n=r.num_valid())


def algorithmic_bytes(wl, sz, s):
    T, H, E, K = wl.T, wl.H, wl.E, wl.K
    return {
        "gather": sz["U"] * H * s + sz["R"] * H * s + 4 * T * K + 8 * E,
        "combine": sz["N"] * H * s + T * H * s + 8 * T * K,
        "wgrad": sz["N"] * H * s + sz["U"] * H * s + 8 * T * K,
    }


def backward_bytes(wl, sz, s):
    T, H, K = wl.T, wl.H, wl.K
    return sz["N"] * H * s + sz["U"] * H * s + sz["R"] * H * s + 12 * T * K


def oracle_step(wl, W):
    """One whole step of the CPU oracle on the workload: compaction (if the
    workload has a routing map), route_prep, gather, combine, wgrad."""
    import oracle
    if wl.routing_map is not None:
        w, top = oracle.routing_map_compact(wl.probs, W.F32, wl.routing_map, wl.topk)
    else:
        w, top = wl.weights, wl.top_experts
    m = wl.pad_multiple if wl.layout == W.PADDED else None
    cap = wl.capacity if wl.layout == W.BINNED else None
    r = oracle.route_prep(top, wl.E, pad_multiple=m)
    y = oracle.gather(wl.x, r, wl.layout, cap)
    oracle.scatter_combine(y, wl.dtype, r, wl.layout, cap, weights=w.reshape(-1))
    oracle.wgrad(y, wl.grad, wl.dtype, r, wl.layout, cap)


def cpu_baseline(wl, W, seconds, bytes_step):
    """The CPU oracle, as it stands, on the same workload: whole steps
    (compaction, route_prep, gather, combine, wgrad) repeated until about
    ``seconds`` of CPU time; single-threaded scalar C."""
    reps, t_total = 0, 0.0
    while True:
        t0 = time.perf_counter()
        oracle_step(wl, W)
        t_total += time.perf_counter() - t0
        reps += 1
        if t_total >= seconds or reps >= 50:
            break
    per_step = t_total / reps
    return {"value": round(bytes_step / per_step / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} whole step(s) of the same workload (seed 0), {per_step * 1e3:.1f} ms per step, "
                      f"1 thread; tokens/s {wl.T / per_step:.1f}",
            **host_record()}


def allowed_cpus():
    """CPUs this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_threads():
    """Host threads for the multi-thread oracle leg: the CPUs this process may
    run on, at most 16 (one GPU's share of the host)."""
    return max(1, min(allowed_cpus(), 16))


def host_record():
    """What the CPU figures ran on: the host's CPU count, the CPUs this
    process may use, and the CPU model string."""
    return {"host_cpus": os.cpu_count(), "allowed_cpus": allowed_cpus(), "cpu_model": cpu_model()}


def cpu_baseline_threads(wl, W, seconds, bytes_step, threads):
    """The same oracle steps on ``threads`` host threads at once, each thread
    running whole independent steps of the workload until ``seconds`` of wall
    time have passed (a step under way then finishes). The oracle's C calls
    release the interpreter lock, so the threads run on separate cores; the
    figure is whole-job throughput: completed steps x step bytes / wall time."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    oracle.round_bf16(0.0)  # opens the oracle library once, before the threads start

    t_start = time.perf_counter()
    deadline = t_start + seconds

    def worker(_):
        done = 0
        while True:
            oracle_step(wl, W)
            done += 1
            if time.perf_counter() >= deadline:
                return done

    with ThreadPoolExecutor(max_workers=threads) as pool:
        steps = sum(pool.map(worker, range(threads)))
    wall = time.perf_counter() - t_start
    return {"value": round(steps * bytes_step / wall / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} whole independent step(s) of the same workload (seed 0) on {threads} threads "
                      f"in {wall:.1f} s; tokens/s {steps * wl.T / wall:.1f}",
            "thread_cap": "16 threads: one GPU's share of the host", **host_record()}


def cpu_model():
    """The host CPU's model name, as /proc/cpuinfo gives it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def traffic_for(kernel, workload_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(workload_name, {}).get(kernel)
    if not e or e.get("source_hash") != source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (the data path is a "
              f"single-GPU library; it has no multi-GPU code)", file=sys.stderr)
        sys.exit(2)
    import torch
    import padded_expert_gather_amd as peg
    import workloads as W

    if args.copy_calibration:
        copy_calibration(torch)
        return

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating workload {args.workload}")
    wl = W.config(args.workload, 0)
    host, sz = host_inputs(torch, W, wl, peg, dev)
    s = 4 if wl.dtype == W.F32 else 2
    ab = algorithmic_bytes(wl, sz, s)
    bytes_step = sum(ab.values())
    host["no_backward"] = args.no_backward
    host["no_router"] = args.no_router
    if args.from_logits and wl.logits is None:
        print(f"--from-logits: workload {wl.name} has no router scores", file=sys.stderr)
        sys.exit(2)
    host["from_logits"] = args.from_logits
    per_set = (wl.T * wl.H * s) * 3 + sz["R"] * wl.H * s * (1 if args.no_backward else 2)
    sets = args.sets or max(2, min(16, math.ceil(2 * 2 ** 30 / per_set)))
    log(f"R={sz['R']} N={sz['N']} U={sz['U']} step bytes={bytes_step / 1e6:.1f} MB, {sets} input copies")
    # every call goes to one stream of its own (default priority), which a
    # graph capture can also use
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        steps_obj = [Step(peg, torch, wl, dev, host) for _ in range(sets)]
    torch.cuda.synchronize()

    names = steps_obj[0].order
    for i in range(args.warmup):
        steps_obj[i % sets].run()
    torch.cuda.synchronize()
    graphs = None
    if args.graph:
        graphs = []
        for st in steps_obj:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                st.run()
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(min(args.warmup, sets)):
            graphs[i % sets].replay()
        torch.cuda.synchronize()

    # Timed region 1 (the headline): K whole steps back to back, nothing else
    # on the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            if graphs:
                graphs[(args.warmup + i) % sets].replay()
            else:
                steps_obj[(args.warmup + i) % sets].run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = bytes_step / (ms_step / 1e3) / 1e9

    # Timed region 2 (per-kernel durations): the same K steps with a HIP event
    # before and after every kernel. The event markers add a few microseconds
    # between kernels, which is why they stay out of region 1.
    use_ev = not args.no_events

    def timed_steps(before=None):
        """K steps with a HIP event pair around every kernel; returns the
        per-kernel statistics."""
        hip = HipEvents()
        evs = [{n: (hip.create(), hip.create()) for n in names} for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            steps_obj[(args.warmup + i) % sets].run(evs[i], hip, before)
        torch.cuda.synchronize()
        out = {}
        for n in names:
            ms = [hip.elapsed_ms(evs[i][n][0], evs[i][n][1]) for i in range(args.steps)]
            avg = sum(ms) / len(ms)
            entry = {"avg_us": round(avg * 1e3, 2), "median_us": round(median(ms) * 1e3, 2),
                     "min_us": round(min(ms) * 1e3, 2), "tokens_per_s": round(wl.T / (avg / 1e3), 1),
                     "assignments_per_s": round(sz["n"] / (avg / 1e3), 1)}
            if n in ab:
                entry["bytes"] = ab[n]
                entry["GBps"] = round(ab[n] / (avg / 1e3) / 1e9, 1)
                entry["frac_peak"] = round(ab[n] / (avg / 1e3) / 1e9 / PEAK_GBS, 4)
            out[n] = entry
        return out

    kernels = timed_steps() if use_ev else {}
    # Timed region 2b (cache-flushed per-kernel durations): the same K steps
    # with --flush-bytes (1 GiB) of scratch written and then read back on the
    # stream before every kernel, outside its event pair. The write evicts
    # L2 and the 256 MB Infinity Cache (the kernel's inputs, even those the
    # kernel before it has just written); the read then evicts the dirty
    # lines the write leaves, so that their write-back does not fall inside
    # the next kernel's events.
    kernels_flushed = None
    flush = None
    if use_ev and not args.no_flush:
        flush_buf = torch.empty(args.flush_bytes, dtype=torch.uint8, device=dev)
        flush_sum = torch.empty((), dtype=torch.float32, device=dev)
        fills = [0]

        def flush():
            fills[0] += 1
            with torch.cuda.stream(stream):
                flush_buf.fill_(fills[0] & 255)
                torch.sum(flush_buf.view(torch.float32), dim=0, out=flush_sum)

        kernels_flushed = timed_steps(flush)
    dominant = max(ab, key=lambda n: kernels[n]["avg_us"]) if use_ev else None
    roofline = None
    if dominant:
        achieved = kernels[dominant]["GBps"]
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic_for(dominant, wl.name),
                    "bytes_per_launch": ab[dominant], "avg_us": kernels[dominant]["avg_us"]}
    # Timed region 3 (outside the step): each extra operation alone, one
    # launch per input copy in turn, a HIP event pair around each launch.
    extras = {}
    extra_bytes = {"combine_backward": backward_bytes(wl, sz, s),
                   "router_topk": wl.T * wl.E * 4 + wl.T * wl.K * 8,
                   "route_prep_logits": wl.T * wl.E * 4 + wl.T * wl.K * 8 + 16 * wl.T * wl.K}
    for name in steps_obj[0].extras:
        hip = HipEvents()
        for i in range(max(2, args.warmup)):
            steps_obj[i % sets].run_extra(name)
        torch.cuda.synchronize()

        def timed_extra(before=None):
            bevs = [(hip.create(), hip.create()) for _ in range(args.steps)]
            for i in range(args.steps):
                if before is not None:
                    before()
                steps_obj[i % sets].run_extra(name, bevs[i], hip)
            torch.cuda.synchronize()
            ms = [hip.elapsed_ms(a, b) for a, b in bevs]
            return ms, sum(ms) / len(ms)

        ms, avg = timed_extra()
        bb = extra_bytes[name]
        extras[name] = {"avg_us": round(avg * 1e3, 2), "median_us": round(median(ms) * 1e3, 2),
                        "min_us": round(min(ms) * 1e3, 2), "bytes": bb,
                        "GBps": round(bb / (avg / 1e3) / 1e9, 1),
                        "frac_peak": round(bb / (avg / 1e3) / 1e9 / PEAK_GBS, 4)}
        if flush is not None:
            # the same launches with the caches flushed before each one
            _, avg_f = timed_extra(flush)
            extras[name]["avg_us_flushed"] = round(avg_f * 1e3, 2)
            extras[name]["frac_peak_flushed"] = round(bb / (avg_f / 1e3) / 1e9 / PEAK_GBS, 4)
        if name == "combine_backward":
            extras[name]["traffic"] = traffic_for("backward", wl.name)
        if name in ("router_topk", "route_prep_logits"):
            extras[name]["tokens_per_s"] = round(wl.T / (avg / 1e3), 1)
    if flush is not None:
        del flush_buf
    ceilings = copy_ceiling(torch, HipEvents(), stream) if not args.no_events else None
    if roofline and ceilings:
        roofline["frac_of_copy_ceiling"] = round(roofline["achieved"] / ceilings["copy"], 4)
    cpu = cpu_all = None
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_baseline(wl, W, args.cpu_seconds, bytes_step)
        threads = args.cpu_threads or cpu_threads()
        if threads > 1:
            log(f"timing the CPU oracle on {threads} threads")
            cpu_all = cpu_baseline_threads(wl, W, args.cpu_seconds, bytes_step, threads)

    dtype_name = W.DTYPE_NAMES[wl.dtype]
    line = {
        "metric": "effective HBM GB/s (and % of peak) for gather+scatter+wgrad; routed tokens/s",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_name, "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "K": wl.K,
                   "layout": "binned" if wl.layout == W.BINNED else "padded",
                   "capacity": wl.capacity or None, "pad_multiple": wl.pad_multiple or None,
                   "compaction": wl.routing_map is not None, "input_copies": sets, "from_logits": args.from_logits,
        "launch": "hip graph per step" if args.graph else "calls",
                   "rows": sz["R"], "kept": sz["N"], "tokens_with_route": sz["U"]},
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "routed_tokens_per_s": round(wl.T / (ms_step / 1e3), 1),
        "step_bytes": bytes_step,
        "kernels": kernels,
        "kernels_flushed": kernels_flushed,
        "flush_bytes": None if kernels_flushed is None else args.flush_bytes,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_all,
        "streaming_GBps": ceilings,
        "outside_step": extras,
        "source_hash": {k: source_hash(k) for k in ("gather", "combine", "route_prep")},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
