"""mhc_boundary_noalloc (no workspace, the library's own device scratch) against
mhc_boundary with a workspace, through the C ABI: two calls in a row on every
case, the second with a smaller batch; the outputs must be bit-identical (the
same kernels and plan run on both), which is within every parity bar."""
import numpy as np
import pytest
import torch

from mhc_hyper_connection_boundary_amd import api
from mhc_hyper_connection_boundary_amd import workloads as WL

pytestmark = pytest.mark.gpu


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def outputs(T, d):
    return dict(residual_out=torch.empty(T, 4, d, dtype=torch.bfloat16, device="cuda"),
                layer_input=torch.empty(T, d, dtype=torch.bfloat16, device="cuda"),
                pre=torch.empty(T, 4, device="cuda"), post=torch.empty(T, 4, 1, device="cuda"),
                comb=torch.empty(T, 4, 4, device="cuda"))


def same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("schedule,d,T1,T2", [
    ("split", 1024, 300, 37),        # partial records in the scratch, several tiles
    ("auto", 7168, 32, 9),           # the decode split
    ("invariant", 2048, 200, 50),    # finest split: the most records per token
    ("fused", 2048, 40, 17),         # no records: the scratch is not touched
    ("stream", 2048, 700, 65),       # queue and tile counters at the start of the scratch
])
def test_noalloc_matches_workspace_entry_point(schedule, d, T1, T2):
    print(f"[noalloc] schedule={schedule} d={d} T={T1} then T={T2}", flush=True)
    inp = WL.make_inputs(WL.Config("na", d=d, T=T1, seed=d + T1, scale=(0.3, 0.05, 0.7),
                                   comb_family="routed"))
    dev = dict(x=bf(inp.x), X=bf(inp.X), post=f32(inp.post_prev), comb=f32(inp.comb_prev),
               pre_lag=f32(inp.pre_lag))
    wp = api.prepare_weight(f32(inp.W))
    scale, base, nw = f32(inp.scale), f32(inp.base), bf(inp.norm_w)
    prm = api.params(**inp.params(), schedule=schedule)
    for T in (T1, T2):
        sl = {k: v[:T].contiguous() for k, v in dev.items()}
        ref, got = outputs(T, d), outputs(T, d)
        api.boundary(sl["x"], sl["X"], sl["post"], sl["comb"], sl["pre_lag"], wp, scale, base,
                     nw, prm=prm, out=ref)
        api.boundary_noalloc(sl["x"], sl["X"], sl["post"], sl["comb"], sl["pre_lag"], wp, scale,
                             base, nw, prm=prm, out=got)
        torch.cuda.synchronize()
        for k in ref:
            assert same(ref[k], got[k]), f"T={T}: {k} differs from mhc_boundary"


def test_noalloc_refuses_beyond_its_scratch():
    T, d = 8192, 16384
    x = torch.zeros(T, d, dtype=torch.bfloat16, device="cuda")
    X = torch.zeros(T, 4, d, dtype=torch.bfloat16, device="cuda")
    post, pre = torch.zeros(T, 4, device="cuda"), torch.zeros(T, 4, device="cuda")
    comb = torch.zeros(T, 4, 4, device="cuda")
    wp = torch.zeros(384 * d, dtype=torch.uint8, device="cuda")
    with pytest.raises(api.MhcError) as e:
        api.boundary_noalloc(x, X, post, comb, pre, wp, torch.zeros(3, device="cuda"),
                             torch.zeros(24, device="cuda"), prm=api.params(schedule="invariant"))
    assert e.value.status == 7
