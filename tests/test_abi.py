"""The C ABI on the host: the library loads, exports every entry point that
include/mhc.h declares, and refuses bad arguments before any HIP call (these
tests pass fake, never-dereferenced device addresses and run without a GPU)."""
import ctypes
import os
import re

import pytest

from mhc_hyper_connection_boundary_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")

OK, INVALID, SHAPE, MISALIGNED, ALIASING, WORKSPACE = 0, 1, 2, 3, 4, 5
T, D = 32, 1024
GB = 1 << 30


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return api.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"mhc_prepare_weight", "mhc_pre", "mhc_boundary"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.mhc_abi_version() == 1
    assert L.mhc_status_string(3) == b"pointer not 16-byte aligned"


def test_boundary_kernels_query(L):
    """The kernel names follow the schedule; shapes mhc_boundary refuses, and
    empty batches, name nothing.  (AUTO depends on the device, so only the
    explicit schedules are pinned here.)"""
    split, fused, invariant, stream = (api.SCHEDULES[k] for k in ("split", "fused", "invariant", "stream"))
    assert L.mhc_boundary_kernels(8192, 7168, split) == b"k_partial+k_finish"
    assert L.mhc_boundary_kernels(32, 7168, invariant) == b"k_partial+k_finish"
    assert L.mhc_boundary_kernels(8192, 7168, stream) == b"k_stream"
    assert L.mhc_boundary_kernels(8192, 7168, fused) == b"k_fused_w4"
    assert L.mhc_boundary_kernels(100, 7168, fused) == b"k_fused"
    assert L.mhc_boundary_kernels(0, 7168, split) == b""
    assert L.mhc_boundary_kernels(32, 7000, split) == b""
    assert L.mhc_boundary_kernels(32, 7168, 5) == b""
    assert L.mhc_boundary_kernels(32, 7168, -1) == b""
    assert api.boundary_kernels(8192, 7168, "stream") == "k_stream"


COUNTERS = 196864   # the streaming schedule's counters: 4 * (3 + 3 * 2^20 / 64), rounded to 256


def stream_data(T, d):
    return -(-4 * T // 256) * 256 + T * (d // 256) * 128


def test_size_queries(L):
    assert L.mhc_prepared_weight_bytes(7168) == 384 * 7168 == 2752512
    assert L.mhc_prepared_weight_bytes(7000) == 0
    # every schedule fits: the counters, then the larger of the finest split's
    # records (128 B per token per 128 of hidden) and the streaming data
    for T, d in ((32, 7168), (8192, 7168), (3, 1280), (1, 256), (5, 256)):
        assert L.mhc_workspace_bytes(T, d) == COUNTERS + max(T * d, stream_data(T, d)), (T, d)
    # the limits: no 32-bit overflow in the size queries
    assert L.mhc_workspace_bytes(1 << 20, 16384) == COUNTERS + (1 << 20) * 16384
    assert L.mhc_workspace_bytes((1 << 20) + 1, 16384) == 0
    assert L.mhc_prepared_weight_bytes(16384) == 384 * 16384
    assert L.mhc_prepared_weight_bytes(16640) == 0
    assert L.mhc_workspace_bytes(0, 7168) == 0
    assert L.mhc_workspace_bytes(32, 100) == 0


class Buffers:
    """Disjoint fake device addresses, 16-byte aligned, for one boundary call."""

    def __init__(self, L, T=T, d=D):
        self.T, self.d = T, d
        sizes = dict(x=T * d * 2, residual=T * 4 * d * 2, post=T * 16, comb=T * 64, pre_lag=T * 16,
                     w=384 * d, scale=16, base=96, norm_w=d * 2, res_out=T * 4 * d * 2,
                     li=T * d * 2, pre_out=T * 16, post_out=T * 16, comb_out=T * 64,
                     mixes=T * 96, rstd=T * 4, ws=max(L.mhc_workspace_bytes(T, d), 16))
        self.addr = {}
        a = GB
        for k, n in sizes.items():
            self.addr[k] = a
            a += (n + 4095) // 4096 * 4096 + 4096
        self.ws_bytes = sizes["ws"]

    def args(self, **over):
        a = dict(self.addr)
        a.update(over)
        P = lambda k: ctypes.c_void_p(a[k]) if a[k] else None
        return [a.get("T", self.T), a.get("d", self.d), P("x"), P("residual"), P("post"),
                P("comb"), P("pre_lag"), P("w"), P("scale"), P("base"), P("norm_w"),
                a.get("prm", ctypes.byref(api.params())), P("res_out"), P("li"), P("pre_out"),
                P("post_out"), P("comb_out"), P("mixes"), P("rstd"), P("ws"),
                a.get("ws_bytes", self.ws_bytes), None]


def call(L, b, **over):
    return L.mhc_boundary(*b.args(**over))


def test_boundary_refusals(L):
    b = Buffers(L)
    assert call(L, b, T=-3) == INVALID
    assert call(L, b, x=0) == INVALID
    assert call(L, b, li=0) == INVALID
    assert call(L, b, prm=None) == INVALID
    assert call(L, b, prm=ctypes.byref(api.params(sinkhorn_iters=0))) == INVALID
    assert call(L, b, prm=ctypes.byref(api.params(rms_eps=-1.0))) == INVALID
    assert call(L, b, prm=ctypes.byref(api.params(norm_eps=float("nan")))) == INVALID
    bad_schedule = api.params()
    bad_schedule.schedule = 6
    assert call(L, b, prm=ctypes.byref(bad_schedule)) == INVALID
    # the single-pass schedule belongs to mhc_pre; the boundary refuses it
    assert call(L, b, prm=ctypes.byref(api.params(schedule="onepass"))) == INVALID
    assert call(L, b, d=1000) == SHAPE
    assert call(L, b, d=128) == SHAPE
    assert call(L, b, T=(1 << 20) + 1) == SHAPE
    assert call(L, b, residual=b.addr["residual"] + 2) == MISALIGNED
    assert call(L, b, comb_out=b.addr["comb_out"] + 8) == MISALIGNED
    assert call(L, b, li=b.addr["res_out"] + 64) == ALIASING            # output in output
    assert call(L, b, res_out=b.addr["residual"]) == ALIASING           # in place is refused
    assert call(L, b, ws=b.addr["x"]) == ALIASING                       # workspace over input
    assert call(L, b, ws=0) == WORKSPACE
    assert call(L, b, ws_bytes=b.ws_bytes - 16) == WORKSPACE


def test_pre_refusals(L):
    b = Buffers(L)
    a = b.addr
    P = ctypes.c_void_p
    prm = ctypes.byref(api.params())

    def pre(T=T, d=D, residual=a["residual"], li=a["li"], ws=a["ws"], wsb=b.ws_bytes, prm=prm):
        return L.mhc_pre(T, d, P(residual) if residual else None, P(a["w"]), P(a["scale"]),
                         P(a["base"]), None, prm, P(li) if li else None, P(a["pre_out"]),
                         P(a["post_out"]), P(a["comb_out"]), None, None,
                         P(ws) if ws else None, wsb, None)
    assert pre(residual=0) == INVALID
    assert pre(d=300) == SHAPE
    assert pre(li=a["li"] + 4) == MISALIGNED
    assert pre(li=a["residual"]) == ALIASING
    assert pre(ws=0) == WORKSPACE
    assert pre(prm=ctypes.byref(api.params(sinkhorn_iters=0))) == INVALID
    # the single pass holds at most 64 tokens (one 16-token group per wave)
    onepass = ctypes.byref(api.params(schedule="onepass"))
    assert pre(T=65, prm=onepass) == SHAPE
    assert pre(T=0, prm=onepass) == OK


def test_prepare_weight_refusals(L):
    P = ctypes.c_void_p
    assert L.mhc_prepare_weight(None, 1024, P(GB), None) == INVALID
    assert L.mhc_prepare_weight(P(GB), 1000, P(2 * GB), None) == SHAPE
    assert L.mhc_prepare_weight(P(GB + 4), 1024, P(2 * GB), None) == MISALIGNED
    assert L.mhc_prepare_weight(P(GB), 1024, P(GB + 4096), None) == ALIASING


def test_post_refusals(L):
    P = ctypes.c_void_p
    b = Buffers(L)
    a = b.addr

    def post(T=T, d=D, x=a["x"], res=a["residual"], out=a["res_out"]):
        return L.mhc_post(T, d, P(x) if x else None, P(res), P(a["post"]), P(a["comb"]),
                          P(out) if out else None, None)
    assert post(x=0) == INVALID
    assert post(out=0) == INVALID
    assert post(d=1000) == SHAPE
    assert post(x=a["x"] + 8) == MISALIGNED
    assert post(out=a["residual"] + 4096) == ALIASING


def test_pre_mixes_refusals(L):
    P = ctypes.c_void_p
    b = Buffers(L)
    a = b.addr
    S = 4
    dm, sq = a["ws"], a["ws"] + S * T * 96 + 4096   # fake partial buffers past the others
    prm = ctypes.byref(api.params())

    def pm(T=T, d=D, S=S, res=a["residual"], dm=dm, sq=sq, li=a["li"], prm=prm):
        return L.mhc_pre_mixes(T, d, S, P(res) if res else None, P(dm) if dm else None, P(sq),
                               P(a["scale"]), P(a["base"]), None, prm, P(li), P(a["pre_out"]),
                               P(a["post_out"]), P(a["comb_out"]), None)
    assert pm(S=0) == INVALID
    assert pm(S=65) == INVALID
    assert pm(dm=0) == INVALID
    assert pm(prm=ctypes.byref(api.params(sinkhorn_iters=0))) == INVALID
    assert pm(d=1000) == SHAPE
    assert pm(dm=dm + 4) == MISALIGNED
    assert pm(li=dm + 16) == ALIASING                     # output over the partials
    assert pm(li=sq + (S - 1) * T * 4) == ALIASING       # ... over the last split of sqrsum


def test_prefetch_weight_refusals(L):
    P = ctypes.c_void_p
    assert L.mhc_prefetch_weight(None, 1024, None) == INVALID
    assert L.mhc_prefetch_weight(P(GB), 1000, None) == SHAPE
    assert L.mhc_prefetch_weight(P(GB + 8), 1024, None) == MISALIGNED


def test_empty_batch_is_a_noop(L):
    """tokens == 0 returns OK once the parameters and hidden pass their checks,
    reading no pointer (all NULL here) and enqueueing nothing."""
    prm = ctypes.byref(api.params())
    bad = ctypes.byref(api.params(sinkhorn_iters=0))
    N = None

    def boundary(d=D, p=prm):
        return L.mhc_boundary(0, d, *([N] * 9), p, *([N] * 8), 0, N)

    def pre(d=D, p=prm):
        return L.mhc_pre(0, d, *([N] * 5), p, *([N] * 7), 0, N)

    assert boundary() == OK
    assert pre() == OK
    assert L.mhc_post(0, D, *([N] * 6)) == OK
    assert L.mhc_pre_mixes(0, D, 1, *([N] * 6), prm, *([N] * 5)) == OK
    # the checks that do not depend on the batch still apply
    assert boundary(d=300) == SHAPE and pre(d=300) == SHAPE
    assert L.mhc_post(0, 300, *([N] * 6)) == SHAPE
    assert boundary(p=bad) == INVALID and pre(p=bad) == INVALID
    assert L.mhc_pre_mixes(0, D, 0, *([N] * 6), prm, *([N] * 5)) == INVALID
    assert boundary(p=N) == INVALID
    fused = ctypes.byref(api.params(schedule="fused"))
    assert boundary(d=1280, p=fused) == SHAPE and pre(d=1280, p=fused) == SHAPE
    assert boundary(d=1024, p=fused) == OK


def test_boundary_noalloc_refusals(L):
    """The no-allocation entry point validates like mhc_boundary, and refuses a
    batch whose schedule needs more record space than its device array holds
    (here INVARIANT: tokens * hidden bytes of records) before any HIP call."""
    assert L.mhc_status_string(7) == b"batch needs more than the no-allocation entry point's scratch"
    b = Buffers(L)

    def noalloc(**over):
        return L.mhc_boundary_noalloc(*b.args(**over)[:-3], None)
    assert noalloc(T=-1) == INVALID
    assert noalloc(x=0) == INVALID
    assert noalloc(d=1000) == SHAPE
    assert noalloc(residual=b.addr["residual"] + 2) == MISALIGNED
    assert noalloc(li=b.addr["res_out"] + 64) == ALIASING
    assert noalloc(T=0) == OK
    inv = ctypes.byref(api.params(schedule="invariant"))
    big = Buffers(L, T=8192, d=16384)         # 8192 * 16384 bytes of records > 64 MiB
    assert L.mhc_boundary_noalloc(*big.args(prm=inv)[:-3], None) == 7
