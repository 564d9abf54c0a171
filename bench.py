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
    return dict(workload="decode d=7168 T=32", timing="HIP graph replay",
                us_per_call_hot=hot_ms * 1e3, us_per_call_cold=cold_ms * 1e3,
                us_per_call_eager=eager_ms * 1e3,
                tokens_per_s_hot=T / (hot_ms * 1e-3), tokens_per_s_cold=T / (cold_ms * 1e-3),
                gbs_cold=b / (cold_ms * 1e-3) / 1e9,
                roofline_frac_cold=b / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)


def cpu_baseline(inp, budget_s=10.0):
    from oracle import oracle as O

    O.lib()
    rng = np.random.default_rng(7)
    probe = np.sort(rng.choice(inp.T, size=32, replace=False)).astype(np.int32)
    t0 = time.perf_counter()
    O.boundary(inp, tokens=probe)
    per_tok = (time.perf_counter() - t0) / len(probe)
    n = int(min(inp.T, max(64, budget_s / max(per_tok, 1e-9))))
    tok = np.sort(rng.choice(inp.T, size=n, replace=False)).astype(np.int32)
    t0 = time.perf_counter()
    O.boundary(inp, tokens=tok)
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="tokens/s", cores=O.max_threads(), kind="oracle",
                sample=f"{n} random tokens of the prefill batch (d={inp.d}), {dt:.1f} s wall")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--schedule", default="auto", choices=["auto", "split", "fused"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the boundary has "
              "no cross-GPU step to measure", file=sys.stderr)
        sys.exit(2)

    import torch

    w = Workload("prefill", schedule=a.schedule)
    T, d = w.inp.T, w.inp.d
    print(f"[bench] prefill T={T} d={d} schedule={a.schedule}: warmup {a.warmup}, steps {a.steps}",
          file=sys.stderr, flush=True)
    ms, wall = time_calls(torch, lambda k: w.call(), a.steps, a.warmup)
    b = algorithmic_bytes(T, d)
    gbs = b / (ms * 1e-3) / 1e9
    line = dict(
        metric=METRIC, value=T / (ms * 1e-3), unit="tokens/s", n_gpus=1, steps=a.steps,
        warmup=a.warmup, ms_per_step=ms, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload="prefill d=7168 T=8192", d=d, T=T, n_hc=4, sinkhorn_iters=20,
                    schedule=a.schedule),
        roofline=dict(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=gbs / HBM_PEAK_GBS, traffic=None,
                      bytes_per_call=b, kernel="mhc_boundary (whole call)"),
    )
    if not a.no_decode:
        print("[bench] decode T=32", file=sys.stderr, flush=True)
        line["decode_t32"] = decode_numbers(200, a.schedule)
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w.inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
