"""Throughput of the mHC boundary on one MI355X.

A step is one mhc_boundary call (residual update, projection, pre/post/comb,
layer input) over one batch of synthetic tokens already resident in HBM.  The
headline workload is prefill, d=7168, T=8192; the decode batch (d=7168, T=32)
is reported beside it, hot (same buffers every call) and cold (rotating
through input and weight sets larger than the 256 MB last-level cache).

Prints one JSON line.  Algorithmic bytes per call:
    T * (20 d + 192) + 386 d + 108
(X read 8d, x read 2d, X' write 8d, layer input write 2d, 96 B of previous
coefficients read and 96 B of new ones written per token; prepared weight
384 d, norm_w 2 d, scale and base 108 B per call).

Before the W warmup steps the prefill call runs untimed for --settle seconds
(0.3 by default): in a fresh process the first hundred or so calls are about
3% slower than the steady state.  Exactly K steps are timed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mHC boundary tokens/s at d=7168 (decode T=32, prefill T=8192); % HBM roofline"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
# The sources whose text decides each boundary kernel's memory traffic (the
# names are those mhc_boundary_kernels reports).
KERNEL_FILES = {  # (build.py: the fused kernels' compiler flags)
    "k_fused_w4": ("mhc_fused.hip", "mhc_device.h", "../build.py"),
    "k_fused": ("mhc_fused.hip", "mhc_device.h", "../build.py"),
    "k_stream": ("mhc_stream.hip", "mhc_device.h"),
    "k_partial+k_finish": ("mhc_kernels.hip", "mhc_device.h"),
}
COPY_BYTES = 1 << 30


def traffic_profile_path(kernel: str) -> str:
    return os.path.join(PROFILES, f"{kernel.replace('+', '_')}_prefill_traffic.txt")


def kernel_sources_sha256(kernel: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_FILES[kernel]:
        with open(os.path.join(ROOT, "mhc_hyper_connection_boundary_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel: str):
    """HBM bytes per call of the kernel(s) from the committed counter summary,
    if it was taken on the current kernel sources (else None)."""
    if kernel not in KERNEL_FILES:
        return None
    try:
        with open(traffic_profile_path(kernel)) as f:
            kv = dict(l.split(":", 1) for l in f if ":" in l and not l.startswith(" "))
    except OSError:
        return None
    if kv.get("sources_sha256", "").strip() != kernel_sources_sha256(kernel):
        return None
    return float(kv["traffic_bytes_per_call"])


def algorithmic_bytes(T: int, d: int) -> int:
    return T * (20 * d + 192) + 386 * d + 108


class Workload:
    def __init__(self, name, T=None, schedule="auto"):
        import torch

        from mhc_hyper_connection_boundary_amd import api
        from mhc_hyper_connection_boundary_amd import workloads as WL

        self.api, self.torch = api, torch
        self.inp = WL.make_inputs(name, T=T)
        i = self.inp
        dev = torch.device("cuda")
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
        self.t = dict(x=bf(i.x), X=bf(i.X), post=f(i.post_prev), comb=f(i.comb_prev),
                      pre_lag=f(i.pre_lag), scale=f(i.scale), base=f(i.base), norm_w=bf(i.norm_w))
        self.wp = api.prepare_weight(f(i.W))
        self.prm = api.params(**i.params(), schedule=schedule)
        T, d = i.T, i.d
        self.out = dict(residual_out=torch.empty_like(self.t["X"]),
                        layer_input=torch.empty(T, d, dtype=torch.bfloat16, device=dev),
                        pre=torch.empty(T, 4, device=dev), post=torch.empty(T, 4, 1, device=dev),
                        comb=torch.empty(T, 4, 4, device=dev))
        self.ws = api.workspace(T, d, dev)

    def call(self, t=None, wp=None):
        t = t or self.t
        self.api.boundary(t["x"], t["X"], t["post"], t["comb"], t["pre_lag"], wp if wp is not None else self.wp,
                          t["scale"], t["base"], t["norm_w"], prm=self.prm, ws=self.ws, out=self.out)


def settle(torch, fn, seconds=0.3):
    """Untimed calls for about `seconds` before the warmup steps.  In a fresh
    process the first hundred or so prefill calls run about 3% slower than
    the rest (the device's clocks and caches settle); the timed steps should
    see the steady state."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            fn()
        torch.cuda.synchronize()


def time_calls(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for k in range(steps):
        fn(k)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall


def graph_time(torch, calls, reps):
    """Capture `calls` (a list of thunks) once into a HIP graph and time
    `reps` replays: the per-call device time without host launch overhead."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / (reps * len(calls))


def decode_numbers(steps, schedule):
    import torch

    w = Workload("decode", schedule=schedule)
    T, d = w.inp.T, w.inp.d
    b = algorithmic_bytes(T, d)
    eager_ms, _ = time_calls(torch, lambda k: w.call(), steps, 20)
    hot_ms = graph_time(torch, [w.call] * 20, max(1, steps // 20))
    # cold: 64 copies of the inputs and weights (~320 MB in all, more than the
    # 256 MB last-level cache), used in turn, so every call reads from HBM
    sets = [({k: v.clone() for k, v in w.t.items()}, w.wp.clone()) for _ in range(64)]
    cold_ms = graph_time(torch, [lambda t=t, wp=wp: w.call(t, wp) for t, wp in sets], 4)
    # With a stand-in producer of x (a 16 MB device copy, as the block before
    # the boundary would be) in front of every call: the boundary alone, then
    # with the weight prefetch on a forked stream overlapping the producer.
    src = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    side = torch.cuda.Stream()

    def produced(t, wp, prefetch):
        def run():
            main = torch.cuda.current_stream()
            if prefetch:
                side.wait_stream(main)
                with torch.cuda.stream(side):
                    w.api.prefetch_weight(wp, d, side)
            dst.copy_(src)
            if prefetch:
                main.wait_stream(side)
            w.call(t, wp)
        return run

    prod_ms = graph_time(torch, [lambda: dst.copy_(src)] * 64, 4)
    cold_prod_ms = graph_time(torch, [produced(t, wp, False) for t, wp in sets], 4)
    cold_pref_ms = graph_time(torch, [produced(t, wp, True) for t, wp in sets], 4)
    return dict(workload="decode d=7168 T=32", timing="HIP graph replay",
                us_per_call_hot=hot_ms * 1e3, us_per_call_cold=cold_ms * 1e3,
                producer_us=prod_ms * 1e3,
                us_per_call_cold_after_producer=(cold_prod_ms - prod_ms) * 1e3,
                us_per_call_cold_after_producer_with_prefetch=(cold_pref_ms - prod_ms) * 1e3,
                us_per_call_eager=eager_ms * 1e3,
                tokens_per_s_hot=T / (hot_ms * 1e-3), tokens_per_s_cold=T / (cold_ms * 1e-3),
                gbs_cold=b / (cold_ms * 1e-3) / 1e9,
                roofline_frac_cold=b / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)


def decode_phases_run(schedule, reps=8):
    """Cold decode calls (T=32, 64 rotating input sets) replayed from a HIP
    graph, for a kernel trace: rocprofv3 --kernel-trace then gives each
    kernel's duration and the gaps between the launches of a call."""
    import torch

    w = Workload("decode", schedule=schedule)
    sets = [({k: v.clone() for k, v in w.t.items()}, w.wp.clone()) for _ in range(64)]
    ms = graph_time(torch, [lambda t=t, wp=wp: w.call(t, wp) for t, wp in sets], reps)
    return dict(workload="decode d=7168 T=32", schedule=schedule,
                kernels=w.api.boundary_kernels(w.inp.T, w.inp.d, schedule),
                timing="HIP graph replay, cold (64 rotating input sets)", us_per_call=ms * 1e3)


def write_decode_profile(trace_dir, schedule):
    """Summarises the kernel trace of --decode-phases into
    profiles/boundary_decode_t32_phases.txt: per call, the duration of each
    kernel and the idle time before it (from the previous kernel's end)."""
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    names = ("k_partial", "k_finish", "k_stream", "k_fused")
    short = lambda n: next((k for k in names if k in n), None)
    seq = [(s, e, short(n)) for s, e, n in rows if short(n)]
    # the last 64 * reps calls are the timed graph replays (after one capture run and one warm replay)
    first = seq[0][2]
    calls, cur = [], []
    for s, e, n in seq:
        if n == first and cur:
            calls.append(cur)
            cur = []
        cur.append((s, e, n))
    calls.append(cur)
    calls = calls[-64 * 8:]
    kinds = [n for _, _, n in calls[-1]]
    med = lambda v: sorted(v)[len(v) // 2] / 1e3
    lines = [f"mhc_boundary decode d=7168 T=32, schedule {schedule} ({' + '.join(kinds)}): "
             "per-phase breakdown of cold graph-replayed calls from a rocprofv3 kernel trace, MI355X",
             "commands (from the repository root, TMPDIR=/tmp):",
             f"  rocprofv3 --kernel-trace --output-format csv -d <dir> -o run -- python bench.py --decode-phases --schedule {schedule}",
             f"  python bench.py --write-decode-profile <dir> --schedule {schedule}",
             f"calls summarised: {len(calls)} (the last 512 replayed calls; medians in us)"]
    prev_end = None
    for i, k in enumerate(kinds):
        durs = [c[i][1] - c[i][0] for c in calls if len(c) == len(kinds)]
        if i == 0:
            gaps = [c2[0][0] - c1[-1][1] for c1, c2 in zip(calls, calls[1:])]
            what = "idle before it (from the previous call's last kernel)"
        else:
            gaps = [c[i][0] - c[i - 1][1] for c in calls if len(c) == len(kinds)]
            what = f"idle before it (from the end of {kinds[i - 1]})"
        lines.append(f"  {k:10s} duration {med(durs):6.2f}   {what} {med(gaps):6.2f}")
    span = [c[-1][1] - c[0][0] for c in calls if len(c) == len(kinds)]
    period = [c2[0][0] - c1[0][0] for c1, c2 in zip(calls, calls[1:])]
    lines.append(f"  first kernel start to last kernel end {med(span):6.2f}; call period {med(period):6.2f}")
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"boundary_decode_t32_{schedule}_phases.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def percentiles_us(torch, fn, n=30):
    """Per-call HIP-event times of n back-to-back calls (µs): p10, median, p90."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    q = lambda p: ts[min(n - 1, int(round(p * (n - 1))))]
    return dict(p10=q(0.1), p50=q(0.5), p90=q(0.9))


def config_numbers():
    """The two other timed configurations of the workload table: the decode wave
    limit (d=7168, T=256; graph replays, hot and cold) and the numerical stress
    batch (d=4096, T=16384, mixed-scale residual; eager calls like the headline)."""
    import torch

    out = {}
    w = Workload("decode_wave")
    T, d = w.inp.T, w.inp.d
    b = algorithmic_bytes(T, d)
    hot_ms = graph_time(torch, [w.call] * 20, 10)
    sets = [({k: v.clone() for k, v in w.t.items()}, w.wp.clone()) for _ in range(_sets_for(b))]
    cold_ms = graph_time(torch, [lambda t=t, wp=wp: w.call(t, wp) for t, wp in sets] * 2, 4)
    out["decode wave limit d=7168 T=256"] = dict(
        kernels=w.api.boundary_kernels(T, d), timing="HIP graph replay",
        us_per_call_hot=hot_ms * 1e3, us_per_call_cold=cold_ms * 1e3,
        tokens_per_s_cold=T / (cold_ms * 1e-3), bytes_per_call=b,
        gbs_cold=b / (cold_ms * 1e-3) / 1e9, roofline_frac_cold=b / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    del w, sets
    torch.cuda.empty_cache()
    w = Workload("stress")
    T, d = w.inp.T, w.inp.d
    b = algorithmic_bytes(T, d)
    settle(torch, w.call, 0.1)
    ms, _ = time_calls(torch, lambda k: w.call(), 30, 5)
    out["stress d=4096 T=16384"] = dict(
        kernels=w.api.boundary_kernels(T, d), timing="HIP events over 30 eager calls",
        us_per_call=ms * 1e3,
        us_per_call_percentiles=percentiles_us(torch, w.call), tokens_per_s=T / (ms * 1e-3),
        bytes_per_call=b, gbs=b / (ms * 1e-3) / 1e9, roofline_frac=b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    del w
    torch.cuda.empty_cache()
    return out


def cold_graph_time(torch, make_call, sets, reps=3, min_calls=24):
    """Per-call device time of make_call(set) rotated over `sets` (distinct
    buffers whose total exceeds the last-level cache), replayed from a HIP graph."""
    calls = [make_call(st) for st in sets]
    calls = calls * max(1, -(-min_calls // len(calls)))
    return graph_time(torch, calls, reps)


def _sets_for(bytes_per_set, cap=64, llc_bytes=256 << 20):
    return max(2, min(cap, -(-2 * llc_bytes // max(1, bytes_per_set))))


def entry_point_numbers(only=None):
    """The other entry points and schedules, each on its own workload, timed
    cold from HIP graph replays against its algorithmic bytes:
      mhc_pre_mixes (partials made elsewhere, no norm): T*(10d + 96 + 100*splits) + 108
      mhc_pre (no norm):                                  T*(10d + 96) + 384d + 108
      mhc_post:                                           T*(18d + 80)
      mhc_boundary, batch-invariant schedule:             T*(20d + 192) + 386d + 108
    (X read 8d, x read 2d, X' write 8d, layer input write 2d per token; 96 B of
    coefficients written; 96+4 B of partials read per split.)  `only` keeps the
    legs whose name contains it (for profiling one kernel at a time)."""
    import torch

    from mhc_hyper_connection_boundary_amd import api
    from mhc_hyper_connection_boundary_amd import workloads as WL

    dev = torch.device("cuda")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    out = {}

    def record(name, T, d, nbytes, us, **extra):
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = dict(T=T, d=d, us_per_call=us, tokens_per_s=T / (us * 1e-6),
                         bytes_per_call=nbytes, gbs=gbs, roofline_frac=gbs / HBM_PEAK_GBS,
                         timing="HIP graph replay, cold (rotating buffer sets)", **extra)
        print(f"[bench] {name}: {us:.2f} us, {gbs:.0f} GB/s", file=sys.stderr, flush=True)

    def wanted(name):
        if only is None:
            return True
        exact = any(n == only for n, *_ in legs)
        return name == only if exact else only in name

    def pre_mixes_leg(T, d, S):
        inp = WL.make_inputs(WL.Config("pm", d=d, T=T, seed=11))
        dm, sq = WL.make_partials(T, d, S, seed=11)
        base = dict(X=bf(inp.X), dm=f(dm), sq=f(sq), scale=f(inp.scale), base=f(inp.base))
        nbytes = T * (10 * d + 96 + 100 * S) + 108
        sets = [base] + [{k: v.clone() for k, v in base.items()}
                         for _ in range(_sets_for(nbytes) - 1)]
        prm = api.params(**inp.params())
        mk = lambda st: (lambda: api.pre_mixes(st["X"], st["dm"], st["sq"], st["scale"],
                                               st["base"], None, prm=prm))
        return nbytes, cold_graph_time(torch, mk, sets) * 1e3

    def residual_sets(T, d, nbytes):
        inp = WL.make_inputs("prefill" if T == 8192 else "decode", T=T)
        base = dict(X=bf(inp.X), x=bf(inp.x), post=f(inp.post_prev), comb=f(inp.comb_prev),
                    pre_lag=f(inp.pre_lag), scale=f(inp.scale), base=f(inp.base),
                    norm_w=bf(inp.norm_w))
        W = f(inp.W)
        sets = []
        for k in range(_sets_for(nbytes)):
            st = base if k == 0 else {kk: v.clone() for kk, v in base.items()}
            st = dict(st, wp=api.prepare_weight(W), ws=api.workspace(T, d, dev))
            sets.append(st)
        return inp, sets

    def pre_leg(T, d, schedule="auto"):
        nbytes = T * (10 * d + 96) + 384 * d + 108
        inp, sets = residual_sets(T, d, nbytes)
        prm = api.params(**inp.params(), schedule=schedule)
        mk = lambda st: (lambda: api.pre(st["X"], st["wp"], st["scale"], st["base"], None,
                                         prm=prm, ws=st["ws"]))
        return nbytes, cold_graph_time(torch, mk, sets) * 1e3

    def post_leg(T, d):
        nbytes = T * (18 * d + 80)
        _, sets = residual_sets(T, d, nbytes)
        for st in sets:
            st["out"] = torch.empty_like(st["X"])
        mk = lambda st: (lambda: api.post(st["x"], st["X"], st["post"], st["comb"], out=st["out"]))
        return nbytes, cold_graph_time(torch, mk, sets) * 1e3

    def invariant_leg(T, d):
        nbytes = algorithmic_bytes(T, d)
        inp, sets = residual_sets(T, d, nbytes)
        prm = api.params(**inp.params(), schedule="invariant")
        for st in sets:
            st["o"] = dict(residual_out=torch.empty_like(st["X"]),
                           layer_input=torch.empty(T, d, dtype=torch.bfloat16, device=dev),
                           pre=torch.empty(T, 4, device=dev), post=torch.empty(T, 4, 1, device=dev),
                           comb=torch.empty(T, 4, 4, device=dev))
        mk = lambda st: (lambda: api.boundary(st["x"], st["X"], st["post"], st["comb"],
                                              st["pre_lag"], st["wp"], st["scale"], st["base"],
                                              st["norm_w"], prm=prm, ws=st["ws"], out=st["o"]))
        return nbytes, cold_graph_time(torch, mk, sets) * 1e3

    legs = []
    for T, d, S in ((4096, 7168, 1), (4096, 4096, 1), (128, 7168, 1), (4096, 7168, 16)):
        legs.append((f"mhc_pre_mixes T={T} d={d} splits={S}", T, d,
                     lambda T=T, d=d, S=S: pre_mixes_leg(T, d, S), dict(splits=S)))
    for T in (1, 32, 64):
        # the single pass (X read once, one launch) beside the split schedule
        for sched in ("onepass", "split"):
            legs.append((f"mhc_pre {sched} T={T} d=7168", T, 7168,
                         lambda T=T, sched=sched: pre_leg(T, 7168, sched), dict(schedule=sched)))
    for T in (8192, 32):
        legs.append((f"mhc_pre T={T} d=7168", T, 7168, lambda T=T: pre_leg(T, 7168), {}))
        legs.append((f"mhc_post T={T} d=7168", T, 7168, lambda T=T: post_leg(T, 7168), {}))
        legs.append((f"mhc_boundary invariant T={T} d=7168", T, 7168,
                     lambda T=T: invariant_leg(T, 7168), {}))
    for name, T, d, fn, extra in legs:
        if wanted(name):
            nbytes, us = fn()
            record(name, T, d, nbytes, us, **extra)
            torch.cuda.empty_cache()
    return out


def cpu_baseline(inp, budget_s=10.0):
    """The oracle, as it stands, on tokens of the prefill batch: whole passes
    over the batch until about budget_s seconds of wall time have run."""
    from oracle import oracle as O

    O.lib()
    t0 = time.perf_counter()
    passes, tokens = 0, 0
    while True:
        O.boundary(inp)
        passes += 1
        tokens += inp.T
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            break
    return dict(value=tokens / dt, unit="tokens/s", cores=O.max_threads(), kind="oracle",
                cpu=cpu_model(), logical_cpus=os.cpu_count(),
                sample=f"{passes} pass(es) over the prefill batch (T={inp.T}, d={inp.d}), "
                       f"{dt:.1f} s wall")


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


MOVER_MODES = {
    0: "tile-major 32x256 items, 2 rows x 512 B per instruction, nontemporal",
    1: "tile-major 32x256 items, 2 rows x 512 B per instruction, plain",
    2: "streaming-schedule pattern: persistent, 64x256 items in 64-element steps, lockstep waves",
    3: "tile-major 32x512 items, 1 row x 1024 B per instruction, nontemporal",
}


def mover_numbers(T=8192, d=7168, steps=10):
    """The movers of libmhc_mover.so on the prefill shape: each reads X and x
    and writes X' and a layer-input-sized buffer (the boundary's activation
    bytes, 20*T*d) and computes nothing.  Their rate is the ceiling of an
    HBM-bound kernel with that access pattern on this device."""
    import ctypes

    import torch

    from mhc_hyper_connection_boundary_amd import build as B

    L = ctypes.CDLL(B.MOVER_LIB)
    L.mhc_mover_run.restype = ctypes.c_int
    L.mhc_mover_run.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda")
    X = torch.ones(T, 4, d, dtype=torch.bfloat16, device=dev)
    x = torch.ones(T, d, dtype=torch.bfloat16, device=dev)
    Xo, lo = torch.empty_like(X), torch.empty_like(x)
    moved = 2 * (X.numel() + x.numel()) * 2
    st = torch.cuda.current_stream().cuda_stream
    out = {}
    for mode, what in MOVER_MODES.items():
        run = lambda k: L.mhc_mover_run(T, d, X.data_ptr(), x.data_ptr(), Xo.data_ptr(), lo.data_ptr(), mode, st)
        if run(0) != 0:
            raise RuntimeError(f"mhc_mover_run mode {mode} refused the shape")
        ms, _ = time_calls(torch, run, steps, 3)
        out[f"mode {mode}"] = dict(pattern=what, us=ms * 1e3, gbs=moved / (ms * 1e-3) / 1e9,
                                   frac=moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    del X, x, Xo, lo
    torch.cuda.empty_cache()
    return dict(workload=f"activation bytes of the prefill boundary (T={T}, d={d}): {moved} B per call",
                **out)


def copy_calibration():
    """A plain 1 GiB device copy: the device's practical streaming ceiling and the
    reference reading for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    ms, _ = time_calls(torch, lambda k: b.copy_(a), 5, 3)
    return dict(copy_bytes=COPY_BYTES, us=ms * 1e3, gbs_read_plus_write=2 * COPY_BYTES / (ms * 1e-3) / 1e9)


def _counter_median(directory, counter, kernel_substr):
    import csv
    import glob

    vals = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr} under {directory}")
    vals.sort()
    return vals[len(vals) // 2], len(vals)


def write_traffic_profile(prof_dir, kernel, schedule):
    """Summarises four rocprofv3 --pmc runs (see the command list written into
    the summary) into profiles/<kernel>_prefill_traffic.txt.  For a schedule of
    two kernels the per-call figure adds the two kernels' medians."""
    f_k = w_k = 0.0
    for name in kernel.split("+"):
        fk, nf = _counter_median(os.path.join(prof_dir, "fetch_boundary"), "FETCH_SIZE", name)
        wk, nw = _counter_median(os.path.join(prof_dir, "write_boundary"), "WRITE_SIZE", name)
        f_k += fk
        w_k += wk
    f_c, _ = _counter_median(os.path.join(prof_dir, "fetch_copy"), "FETCH_SIZE", "copyBuffer")
    w_c, _ = _counter_median(os.path.join(prof_dir, "write_copy"), "WRITE_SIZE", "copyBuffer")
    f_scale = COPY_BYTES / (f_c * 1024)
    w_scale = COPY_BYTES / (w_c * 1024)
    traffic = f_k * 1024 * f_scale + w_k * 1024 * w_scale
    T, d = 8192, 7168
    sched = f" --schedule {schedule}" if schedule != "auto" else ""
    lines = [
        f"{kernel} prefill (d=7168, T=8192): HBM traffic per call from rocprofv3 counters",
        f"sources_sha256: {kernel_sources_sha256(kernel)}",
        f"sources_hashed: {' '.join(KERNEL_FILES[kernel])} (under the package's csrc/)",
        f"fetch_size_kib_per_dispatch: {f_k:.1f}",
        f"write_size_kib_per_dispatch: {w_k:.1f}",
        f"dispatches: {nf} / {nw}",
        f"copy_1GiB_fetch_size_kib: {f_c:.1f}",
        f"copy_1GiB_write_size_kib: {w_c:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"read_bytes_per_call: {f_k * 1024 * f_scale:.0f}",
        f"written_bytes_per_call: {w_k * 1024 * w_scale:.0f}",
        f"traffic_bytes_per_call: {traffic:.0f}",
        f"algorithmic_bytes_per_call: {algorithmic_bytes(T, d)}",
        f"traffic_over_algorithmic: {traffic / algorithmic_bytes(T, d):.3f}",
        "commands (from the repository root, TMPDIR=/tmp):",
        f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch_boundary -o run -- python bench.py --steps 5 --warmup 2 --no-decode --no-cpu-baseline --no-entry-points --no-configs --no-mover{sched}",
        f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write_boundary -o run -- python bench.py --steps 5 --warmup 2 --no-decode --no-cpu-baseline --no-entry-points --no-configs --no-mover{sched}",
        "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch_copy -o run -- python bench.py --copy-calibration",
        "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write_copy -o run -- python bench.py --copy-calibration",
        f"  python bench.py --write-traffic-profile <dir> --traffic-kernel {kernel}{sched}",
    ]
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_profile_path(kernel), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed prefill calls before the warmup steps")
    ap.add_argument("--schedule", default="auto", choices=["auto", "split", "fused", "stream"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the decode wave limit (T=256) and stress (d=4096, T=16384) lines")
    ap.add_argument("--no-entry-points", action="store_true",
                    help="skip the mhc_pre / mhc_pre_mixes / mhc_post / invariant legs")
    ap.add_argument("--leg", metavar="NAME",
                    help="run only the entry-point legs whose name contains NAME and exit")
    ap.add_argument("--decode-phases", action="store_true",
                    help="cold graph-replayed decode calls for a kernel trace, then exit")
    ap.add_argument("--write-decode-profile", metavar="DIR",
                    help="summarise the kernel trace of --decode-phases under DIR into profiles/")
    ap.add_argument("--mover", action="store_true",
                    help="time the movers (the access-pattern ceilings) and exit")
    ap.add_argument("--no-mover", action="store_true", help="leave the mover ceilings out of the line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device copy and exit")
    ap.add_argument("--write-traffic-profile", metavar="DIR",
                    help="summarise rocprofv3 counter runs under DIR into profiles/")
    ap.add_argument("--traffic-kernel", default="k_fused_w4", choices=sorted(KERNEL_FILES),
                    help="the kernel(s) the counter runs of --write-traffic-profile timed")
    a = ap.parse_args()
    if a.write_traffic_profile:
        write_traffic_profile(a.write_traffic_profile, a.traffic_kernel, a.schedule)
        return
    if a.write_decode_profile:
        write_decode_profile(a.write_decode_profile, a.schedule)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the boundary has "
              "no cross-GPU step to measure", file=sys.stderr)
        sys.exit(2)

    if a.copy_calibration:
        print(json.dumps(copy_calibration()), flush=True)
        return
    if a.mover:
        print(json.dumps(mover_numbers()), flush=True)
        return
    if a.decode_phases:
        print(json.dumps(decode_phases_run(a.schedule)), flush=True)
        return
    if a.leg:
        print(json.dumps(entry_point_numbers(a.leg)), flush=True)
        return

    import torch

    w = Workload("prefill", schedule=a.schedule)
    T, d = w.inp.T, w.inp.d
    print(f"[bench] prefill T={T} d={d} schedule={a.schedule}: warmup {a.warmup}, steps {a.steps}",
          file=sys.stderr, flush=True)
    settle(torch, w.call, a.settle)
    ms, wall = time_calls(torch, lambda k: w.call(), a.steps, a.warmup)
    pct = percentiles_us(torch, w.call)
    b = algorithmic_bytes(T, d)
    gbs = b / (ms * 1e-3) / 1e9
    # the kernels the library itself runs for this shape and schedule
    kernel = w.api.boundary_kernels(T, d, a.schedule)
    traffic = recorded_traffic(kernel)
    line = dict(
        metric=METRIC, value=T / (ms * 1e-3), unit="tokens/s", n_gpus=1, steps=a.steps,
        warmup=a.warmup, ms_per_step=ms, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload="prefill d=7168 T=8192", d=d, T=T, n_hc=4, sinkhorn_iters=20,
                    schedule=a.schedule),
        roofline=dict(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=gbs / HBM_PEAK_GBS, traffic=traffic, bytes_per_call=b,
                      kernel=kernel, launches_per_call=len(kernel.split("+"))),
        us_per_call_percentiles=pct,
    )
    if not a.no_mover:
        print("[bench] movers (access-pattern ceilings)", file=sys.stderr, flush=True)
        line["mover_ceiling"] = mover_numbers()
    if not a.no_decode:
        print("[bench] decode T=32", file=sys.stderr, flush=True)
        line["decode_t32"] = decode_numbers(200, a.schedule)
    if not a.no_configs:
        print("[bench] decode wave limit T=256, stress d=4096 T=16384", file=sys.stderr, flush=True)
        line["configs"] = config_numbers()
    if not a.no_entry_points:
        del w
        torch.cuda.empty_cache()
        line["entry_points"] = entry_point_numbers()
        w = None
    if not a.no_cpu_baseline:
        if w is None:
            from mhc_hyper_connection_boundary_amd import workloads as WL
            inp = WL.make_inputs("prefill")
        else:
            inp = w.inp
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
