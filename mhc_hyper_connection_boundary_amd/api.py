"""Python binding of libmhc.so (ctypes).  Argument marshalling only: every step
of the boundary runs in the HIP kernels behind the C ABI.  torch supplies
device memory and the current stream.  There is no fallback: if the library is
missing, loading raises."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmhc.so")
ABI_VERSION = 1

SCHEDULES = {"auto": 0, "split": 1, "fused": 2, "invariant": 3, "stream": 4, "onepass": 5}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "misaligned",
          4: "aliasing", 5: "workspace", 6: "device", 7: "scratch limit"}


class MhcError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: status {status} ({STATUS.get(status, '?')})")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("rms_eps", ctypes.c_float), ("pre_eps", ctypes.c_float),
                ("post_mult", ctypes.c_float), ("sinkhorn_eps", ctypes.c_float),
                ("sinkhorn_iters", ctypes.c_int), ("norm_eps", ctypes.c_float),
                ("schedule", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C ABI.  Raises if libmhc.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m mhc_hyper_connection_boundary_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.mhc_abi_version.restype = I
        L.mhc_abi_version.argtypes = []
        L.mhc_status_string.restype = ctypes.c_char_p
        L.mhc_status_string.argtypes = [I]
        L.mhc_boundary_kernels.restype = ctypes.c_char_p
        L.mhc_boundary_kernels.argtypes = [I, I, I]
        L.mhc_prepared_weight_bytes.restype = Z
        L.mhc_prepared_weight_bytes.argtypes = [I]
        L.mhc_workspace_bytes.restype = Z
        L.mhc_workspace_bytes.argtypes = [I, I]
        L.mhc_prepare_weight.restype = I
        L.mhc_prepare_weight.argtypes = [P, I, P, P]
        L.mhc_pre.restype = I
        L.mhc_pre.argtypes = [I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        L.mhc_pre_mixes.restype = I
        L.mhc_pre_mixes.argtypes = [I, I, I, P, P, P, P, P, P, P, P, P, P, P, P]
        L.mhc_prefetch_weight.restype = I
        L.mhc_prefetch_weight.argtypes = [P, I, P]
        L.mhc_post.restype = I
        L.mhc_post.argtypes = [I, I, P, P, P, P, P, P]
        L.mhc_boundary.restype = I
        L.mhc_boundary.argtypes = [I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        L.mhc_boundary_noalloc.restype = I
        L.mhc_boundary_noalloc.argtypes = [I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
        if L.mhc_abi_version() != ABI_VERSION:
            raise RuntimeError("libmhc.so ABI version mismatch")
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(name, t, dtype, shape, device, optional=False):
    """Refuses, with ValueError, a tensor that the C ABI would read or write out
    of bounds or misread: wrong dtype, shape or device, or not contiguous."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_post(post_prev, T, device):
    """post_prev is [T, 4], or [T, 4, 1] as the boundary returns it."""
    three = isinstance(post_prev, torch.Tensor) and post_prev.dim() == 3
    _check("post_prev", post_prev, torch.float32, (T, 4, 1) if three else (T, 4), device)


def _check_device(device):
    """The kernels run on a GPU: every tensor must live on one."""
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU (cuda device), got {device}")
    if device.index is not None and device.index != torch.cuda.current_device():
        raise ValueError(f"tensors are on {device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()} (the library works on the current one)")


def _shape_of_residual(residual):
    if not isinstance(residual, torch.Tensor) or residual.dim() != 3 or residual.shape[1] != 4:
        raise ValueError("residual must be a [T, 4, hidden] tensor")
    return residual.shape[0], residual.shape[2], residual.device


def _check_workspace(ws, T, hidden, device):
    need = workspace_bytes(T, hidden)
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous() or ws.device != device:
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor on the residual's device")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def params(rms_eps=1e-6, pre_eps=1e-6, post_mult=2.0, sinkhorn_eps=1e-6, sinkhorn_iters=20,
           norm_eps=1e-6, schedule="auto") -> Params:
    return Params(rms_eps, pre_eps, post_mult, sinkhorn_eps, sinkhorn_iters, norm_eps,
                  SCHEDULES[schedule])


def _status(fn, status):
    if status != 0:
        raise MhcError(fn, status)


def _check_common(w_prepared, scale, base, norm_w, hidden, dev):
    _check("w_prepared", w_prepared, torch.uint8, (384 * hidden,), dev)
    _check("scale", scale, torch.float32, (3,), dev)
    _check("base", base, torch.float32, (24,), dev)
    _check("norm_w", norm_w, torch.bfloat16, (hidden,), dev, optional=True)


def prepared_weight_bytes(hidden: int) -> int:
    return lib().mhc_prepared_weight_bytes(hidden)


def boundary_kernels(tokens: int, hidden: int, schedule: str = "auto") -> str:
    """The kernels mhc_boundary launches for this shape and schedule, as the
    library decides them ("" where it would refuse or launch nothing)."""
    return lib().mhc_boundary_kernels(int(tokens), int(hidden), SCHEDULES[schedule]).decode()


def workspace_bytes(tokens: int, hidden: int) -> int:
    return lib().mhc_workspace_bytes(tokens, hidden)


def workspace(tokens: int, hidden: int, device=None) -> torch.Tensor:
    """A workspace for batches up to `tokens` tokens of `hidden`: zero-filled, as
    the library requires before first use (every call leaves it ready for the
    next)."""
    n = max(workspace_bytes(tokens, hidden), 16)
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def prepare_weight(w: torch.Tensor) -> torch.Tensor:
    """W [24, 4*hidden] FP32 (device) -> prepared uint8 tensor (384*hidden bytes)."""
    if not isinstance(w, torch.Tensor) or w.dim() != 2 or w.shape[0] != 24 or w.shape[1] % 4:
        raise ValueError("w must be a [24, 4*hidden] tensor")
    hidden = w.shape[1] // 4
    _check("w", w, torch.float32, (24, 4 * hidden), w.device)
    _check_device(w.device)
    out = torch.empty(prepared_weight_bytes(hidden), dtype=torch.uint8, device=w.device)
    _status("mhc_prepare_weight", lib().mhc_prepare_weight(_ptr(w), hidden, _ptr(out), _stream()))
    return out


def boundary(x, residual, post_prev, comb_prev, pre_lag, w_prepared, scale, base, norm_w=None,
             *, prm: Params | None = None, debug: bool = False, ws: torch.Tensor | None = None,
             out: dict | None = None):
    """Shifted mHC boundary.  Returns (new_residual, new_post [T,4,1], new_comb [T,4,4],
    layer_input, new_pre), plus (mixes, rstd) when debug=True."""
    return _boundary(False, x, residual, post_prev, comb_prev, pre_lag, w_prepared, scale, base,
                     norm_w, prm, debug, ws, out)


def boundary_noalloc(x, residual, post_prev, comb_prev, pre_lag, w_prepared, scale, base,
                     norm_w=None, *, prm: Params | None = None, debug: bool = False,
                     out: dict | None = None):
    """mhc_boundary_noalloc: the boundary without a workspace (the library's own
    device scratch holds the partial records).  Same returns as boundary()."""
    return _boundary(True, x, residual, post_prev, comb_prev, pre_lag, w_prepared, scale, base,
                     norm_w, prm, debug, None, out)


def _boundary(noalloc, x, residual, post_prev, comb_prev, pre_lag, w_prepared, scale, base,
              norm_w, prm, debug, ws, out):
    T, hidden, dev = _shape_of_residual(residual)
    f32, bf16 = torch.float32, torch.bfloat16
    _check("x", x, bf16, (T, hidden), dev)
    _check("residual", residual, bf16, (T, 4, hidden), dev)
    _check_post(post_prev, T, dev)
    _check("comb_prev", comb_prev, f32, (T, 4, 4), dev)
    _check("pre_lag", pre_lag, f32, (T, 4), dev)
    _check_common(w_prepared, scale, base, norm_w, hidden, dev)
    prm = prm or params()
    o = out if out is not None else {}
    for k, shape, dt in (("residual_out", (T, 4, hidden), bf16), ("layer_input", (T, hidden), bf16),
                         ("pre", (T, 4), f32), ("post", (T, 4, 1), f32), ("comb", (T, 4, 4), f32)):
        if k in o:
            _check(f"out['{k}']", o[k], dt, shape, dev)
    _check_device(dev)
    nres = o.get("residual_out")
    if nres is None:
        nres = torch.empty_like(residual)
    li = o.get("layer_input")
    if li is None:
        li = torch.empty(T, hidden, dtype=torch.bfloat16, device=dev)
    pre = torch.empty(T, 4, dtype=torch.float32, device=dev) if "pre" not in o else o["pre"]
    post = torch.empty(T, 4, 1, dtype=torch.float32, device=dev) if "post" not in o else o["post"]
    comb = torch.empty(T, 4, 4, dtype=torch.float32, device=dev) if "comb" not in o else o["comb"]
    mixes = torch.empty(T, 24, dtype=torch.float32, device=dev) if debug else None
    rstd = torch.empty(T, dtype=torch.float32, device=dev) if debug else None
    args = (T, hidden, _ptr(x), _ptr(residual), _ptr(post_prev), _ptr(comb_prev), _ptr(pre_lag),
            _ptr(w_prepared), _ptr(scale), _ptr(base), _ptr(norm_w), ctypes.byref(prm),
            _ptr(nres), _ptr(li), _ptr(pre), _ptr(post), _ptr(comb), _ptr(mixes), _ptr(rstd))
    if noalloc:
        _status("mhc_boundary_noalloc", lib().mhc_boundary_noalloc(*args, _stream()))
    else:
        if ws is None:
            ws = workspace(T, hidden, dev)
        _check_workspace(ws, T, hidden, dev)
        _status("mhc_boundary", lib().mhc_boundary(*args, _ptr(ws), ws.numel(), _stream()))
    res = (nres, post, comb, li, pre)
    return res + (mixes, rstd) if debug else res


def prefetch_weight(w_prepared: torch.Tensor, hidden: int, stream=None):
    """Enqueue a read of the prepared weight (warms the last-level cache)."""
    _check("w_prepared", w_prepared, torch.uint8, (384 * hidden,), w_prepared.device)
    _check_device(w_prepared.device)
    st = ctypes.c_void_p((stream or torch.cuda.current_stream()).cuda_stream)
    _status("mhc_prefetch_weight", lib().mhc_prefetch_weight(_ptr(w_prepared), hidden, st))


def post(x, residual, post_prev, comb_prev, out: torch.Tensor | None = None):
    """Residual update alone: returns X' [T, 4, hidden] (the bits of boundary's
    new_residual)."""
    T, hidden, dev = _shape_of_residual(residual)
    f32, bf16 = torch.float32, torch.bfloat16
    _check("x", x, bf16, (T, hidden), dev)
    _check("residual", residual, bf16, (T, 4, hidden), dev)
    _check_post(post_prev, T, dev)
    _check("comb_prev", comb_prev, f32, (T, 4, 4), dev)
    _check("out", out, bf16, (T, 4, hidden), dev, optional=True)
    _check_device(dev)
    nres = torch.empty_like(residual) if out is None else out
    _status("mhc_post", lib().mhc_post(T, hidden, _ptr(x), _ptr(residual), _ptr(post_prev),
                                      _ptr(comb_prev), _ptr(nres), _stream()))
    return nres


def pre(residual, w_prepared, scale, base, norm_w=None, *, prm: Params | None = None,
        debug: bool = False, ws: torch.Tensor | None = None):
    """Non-shifted mHC pre.  Returns (layer_input, pre, post [T,4,1], comb [T,4,4]),
    plus (mixes, rstd) when debug=True."""
    T, hidden, dev = _shape_of_residual(residual)
    _check("residual", residual, torch.bfloat16, (T, 4, hidden), dev)
    _check_common(w_prepared, scale, base, norm_w, hidden, dev)
    _check_device(dev)
    prm = prm or params()
    li = torch.empty(T, hidden, dtype=torch.bfloat16, device=dev)
    pr = torch.empty(T, 4, dtype=torch.float32, device=dev)
    post = torch.empty(T, 4, 1, dtype=torch.float32, device=dev)
    comb = torch.empty(T, 4, 4, dtype=torch.float32, device=dev)
    mixes = torch.empty(T, 24, dtype=torch.float32, device=dev) if debug else None
    rstd = torch.empty(T, dtype=torch.float32, device=dev) if debug else None
    if ws is None:
        ws = workspace(T, hidden, dev)
    _check_workspace(ws, T, hidden, dev)
    _status("mhc_pre", lib().mhc_pre(
        T, hidden, _ptr(residual), _ptr(w_prepared), _ptr(scale), _ptr(base), _ptr(norm_w),
        ctypes.byref(prm), _ptr(li), _ptr(pr), _ptr(post), _ptr(comb), _ptr(mixes), _ptr(rstd),
        _ptr(ws), ws.numel(), _stream()))
    res = (li, pr, post, comb)
    return res + (mixes, rstd) if debug else res


def pre_mixes(residual, dot_mix, sqrsum, scale, base, norm_w=None, *, prm: Params | None = None):
    """Non-shifted pre from projection partials made elsewhere: dot_mix
    [splits, T, 24] and sqrsum [splits, T] FP32.  Returns (layer_input, pre,
    post [T,4,1], comb [T,4,4])."""
    T, hidden, dev = _shape_of_residual(residual)
    if not isinstance(dot_mix, torch.Tensor) or dot_mix.dim() != 3:
        raise ValueError("dot_mix must be a [splits, T, 24] tensor")
    splits = dot_mix.shape[0]
    _check("residual", residual, torch.bfloat16, (T, 4, hidden), dev)
    _check("dot_mix", dot_mix, torch.float32, (splits, T, 24), dev)
    _check("sqrsum", sqrsum, torch.float32, (splits, T), dev)
    _check("scale", scale, torch.float32, (3,), dev)
    _check("base", base, torch.float32, (24,), dev)
    _check("norm_w", norm_w, torch.bfloat16, (hidden,), dev, optional=True)
    _check_device(dev)
    prm = prm or params()
    li = torch.empty(T, hidden, dtype=torch.bfloat16, device=dev)
    pr = torch.empty(T, 4, dtype=torch.float32, device=dev)
    post = torch.empty(T, 4, 1, dtype=torch.float32, device=dev)
    comb = torch.empty(T, 4, 4, dtype=torch.float32, device=dev)
    _status("mhc_pre_mixes", lib().mhc_pre_mixes(
        T, hidden, splits, _ptr(residual), _ptr(dot_mix), _ptr(sqrsum), _ptr(scale), _ptr(base),
        _ptr(norm_w), ctypes.byref(prm), _ptr(li), _ptr(pr), _ptr(post), _ptr(comb), _stream()))
    return li, pr, post, comb
