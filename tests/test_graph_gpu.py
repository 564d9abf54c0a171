"""The boundary captured in a HIP graph: every replay, with eager work and
synchronisations in between, reproduces the eager result bit for bit."""
import numpy as np
import pytest
import torch

from mhc_hyper_connection_boundary_amd import api
from mhc_hyper_connection_boundary_amd import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("schedule,d,T", [("split", 7168, 32), ("fused", 2048, 40), ("fused", 1024, 8192 + 5),
                                          ("invariant", 1024, 300), ("stream", 7168, 32),
                                          ("stream", 2048, 3000 + 7)])
def test_graph_replay_matches_eager(schedule, d, T):
    print(f"[graph] schedule={schedule} d={d} T={T}", flush=True)
    inp = WL.make_inputs(WL.Config("g", d=d, T=T, seed=d + T))
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    args = (bf(inp.x), bf(inp.X), f(inp.post_prev), f(inp.comb_prev), f(inp.pre_lag))
    wp = api.prepare_weight(f(inp.W))
    rest = (f(inp.scale), f(inp.base), bf(inp.norm_w))
    prm = api.params(**inp.params(), schedule=schedule)
    ws = api.workspace(T, d)
    out = dict(residual_out=torch.empty_like(args[1]),
               layer_input=torch.empty(T, d, dtype=torch.bfloat16, device="cuda"),
               pre=torch.empty(T, 4, device="cuda"), post=torch.empty(T, 4, 1, device="cuda"),
               comb=torch.empty(T, 4, 4, device="cuda"))

    def call():
        api.boundary(*args, wp, *rest, prm=prm, ws=ws, out=out)

    call()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for v in out.values():
            v.zero_()                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k].view(torch.uint8) if out[k].dtype == torch.bfloat16 else out[k],
                               eager[k].view(torch.uint8) if eager[k].dtype == torch.bfloat16 else eager[k]), \
                f"replay {rep}: {k} differs"
