"""The debug aids: the LDS-poison build and MHC_SYNC_DEBUG.

libmhc_lds_poison.so is libmhc.so built with every kernel filling its LDS
with NaN before use: if any kernel read an LDS word it had not written, its
outputs would change.  Every kernel family that uses LDS runs here under both
libraries and the outputs must be bit-identical.  MHC_SYNC_DEBUG=1 makes every
entry point wait for its kernels; a child process with it set must give the
same bits as this one."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from mhc_hyper_connection_boundary_amd import api, build
from mhc_hyper_connection_boundary_amd import workloads as WL

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def say(msg):
    print(f"[debug-builds] {msg}", flush=True)


def bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy().view(np.uint32)


class Inputs:
    def __init__(self, T, d, seed):
        inp = WL.make_inputs(WL.Config("dbg", d=d, T=T, seed=seed, scale=(0.31, 0.047, 0.83),
                                       comb_family="routed"))
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
        self.inp = inp
        self.x, self.X = bf(inp.x), bf(inp.X)
        self.post, self.comb, self.pre_lag = f(inp.post_prev), f(inp.comb_prev), f(inp.pre_lag)
        self.W, self.scale, self.base = f(inp.W), f(inp.scale), f(inp.base)
        self.norm_w = bf(inp.norm_w)


# (label, T, d, call) for every kernel family that uses LDS
def cases():
    def boundary(schedule):
        def run(v, wp):
            r = api.boundary(v.x, v.X, v.post, v.comb, v.pre_lag, wp, v.scale, v.base, v.norm_w,
                             prm=api.params(**v.inp.params(), schedule=schedule), debug=True)
            return [bits(t) for t in r]
        return run

    def pre(schedule):
        def run(v, wp):
            r = api.pre(v.X, wp, v.scale, v.base, v.norm_w,
                        prm=api.params(**v.inp.params(), schedule=schedule), debug=True)
            return [bits(t) for t in r]
        return run

    def pre_mixes(v, wp):
        dm, sq = (torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
                  for a in WL.make_partials(v.inp.T, v.inp.d, 3, seed=v.inp.T))
        r = api.pre_mixes(v.X, dm, sq, v.scale, v.base, v.norm_w,
                          prm=api.params(**v.inp.params()))
        return [bits(t) for t in r]

    return [
        ("boundary split (k_partial, k_finish)", 37, 1024, boundary("split")),
        ("boundary split, several steps per wave (k_partial, k_finish)", 2000, 7168, boundary("split")),
        ("boundary invariant", 33, 2048, boundary("invariant")),
        ("boundary fused 16-token tiles (k_fused)", 300, 1024, boundary("fused")),
        ("boundary fused 32-token tiles (k_fused_w4)", 8192 + 7, 1024, boundary("fused")),
        ("boundary fused 32-token tiles, rotated sweeps (k_fused_w4)", 8192 + 7, 2048, boundary("fused")),
        ("boundary fused 16-token tiles, rotated sweeps (k_fused)", 700, 2048, boundary("fused")),
        ("boundary auto 19-token tiles, rotated sweeps (k_fused_w4)", 4096 + 600, 2048, boundary("auto")),
        ("boundary stream (k_stream)", 200, 2048, boundary("stream")),
        ("pre split (k_partial, k_pre_finish)", 50, 4096, pre("split")),
        ("pre split, several steps per wave (k_partial, k_pre_finish)", 1000, 4096, pre("split")),
        ("pre split, four groups (k_partial_pre_wide)", 2400, 7168, pre("split")),
        ("pre fused 16-token tiles (k_fused_pre)", 100, 1024, pre("fused")),
        ("pre fused 32-token tiles (k_fused_pre_w4)", 8192 + 3, 1024, pre("fused")),
        ("pre fused 32-token tiles, rotated sweeps (k_fused_pre_w4)", 8192 + 3, 2048, pre("fused")),
        ("pre onepass (k_pre_one)", 40, 2048, pre("onepass")),
        ("pre_mixes (k_pre_finish)", 45, 1024, pre_mixes),
    ]


def use_library(path):
    api._lib = None
    api.LIB_PATH = path
    return api.lib()


@pytest.fixture
def product_after():
    yield
    use_library(build.LIB)


def test_lds_poison_build_changes_no_bit(product_after):
    assert os.path.exists(build.POISON_LIB), "build() makes libmhc_lds_poison.so"
    for k, (label, T, d, run) in enumerate(cases()):
        say(f"{label}: T={T} d={d}")
        v = Inputs(T, d, seed=100 + k)
        use_library(build.LIB)
        ref = run(v, api.prepare_weight(v.W))
        torch.cuda.synchronize()
        use_library(build.POISON_LIB)
        got = run(v, api.prepare_weight(v.W))
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, got)):
            assert np.array_equal(a, b), f"{label}: output {i} differs under the LDS poison"


CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, {root!r})
from mhc_hyper_connection_boundary_amd import api
from mhc_hyper_connection_boundary_amd import workloads as WL
inp = WL.make_inputs(WL.Config("sync", d=1024, T=21, seed=9))
bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
wp = api.prepare_weight(f(inp.W))
out = []
for sched in ("split", "fused", "stream"):
    r = api.boundary(bf(inp.x), bf(inp.X), f(inp.post_prev), f(inp.comb_prev), f(inp.pre_lag), wp,
                     f(inp.scale), f(inp.base), bf(inp.norm_w), prm=api.params(**inp.params(), schedule=sched))
    out += [t.float().cpu().numpy().ravel() for t in r]
r = api.pre(bf(inp.X), wp, f(inp.scale), f(inp.base), bf(inp.norm_w), prm=api.params(**inp.params()))
out += [t.float().cpu().numpy().ravel() for t in r]
np.save(sys.argv[1], np.concatenate(out))
"""


def test_sync_debug_gives_the_same_bits(tmp_path):
    script = tmp_path / "child.py"
    script.write_text(CHILD.format(root=ROOT))
    outs = {}
    for flag in ("0", "1"):
        path = tmp_path / f"out{flag}.npy"
        env = dict(os.environ, MHC_SYNC_DEBUG=flag)
        say(f"child process, MHC_SYNC_DEBUG={flag}")
        r = subprocess.run([sys.executable, str(script), str(path)], env=env, capture_output=True,
                           text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        outs[flag] = np.load(path)
    assert np.array_equal(outs["0"], outs["1"])
