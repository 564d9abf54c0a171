"""ctypes front end of the CPU oracle (``mhc_oracle.c``).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the GPU library never
does, and the two share no code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mhc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmhc_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP over tokens, no FP contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Params(ctypes.Structure):
    _fields_ = [("rms_eps", ctypes.c_float), ("pre_eps", ctypes.c_float),
                ("post_mult", ctypes.c_float), ("sinkhorn_eps", ctypes.c_float),
                ("sinkhorn_iters", ctypes.c_int), ("norm_eps", ctypes.c_float)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        L.oracle_tf32_bits.restype = ctypes.c_uint32
        L.oracle_tf32_bits.argtypes = [ctypes.c_uint32]
        L.oracle_bf16_from_f32.restype = ctypes.c_uint16
        L.oracle_bf16_from_f32.argtypes = [ctypes.c_float]
        L.oracle_bf16_from_f64.restype = ctypes.c_uint16
        L.oracle_bf16_from_f64.argtypes = [ctypes.c_double]
        L.oracle_split_weight.restype = None
        L.oracle_split_weight.argtypes = [P, ctypes.c_size_t, P, P, P]
        L.oracle_prepare_weight.restype = ctypes.c_int
        L.oracle_prepare_weight.argtypes = [P, ctypes.c_int, P]
        L.oracle_sinkhorn.restype = None
        L.oracle_sinkhorn.argtypes = [P, ctypes.c_double, ctypes.c_int, P]
        L.oracle_run.restype = ctypes.c_int
        L.oracle_run.argtypes = [ctypes.c_int] * 3 + [P, ctypes.c_int] + [P] * 10 + [P] * 11
        L.oracle_pre_from_mixes.restype = ctypes.c_int
        L.oracle_pre_from_mixes.argtypes = [ctypes.c_int] * 3 + [P, ctypes.c_int] + [P] * 7 + [P] * 9
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return lib().oracle_max_threads()


def tf32_bits(u: int) -> int:
    return lib().oracle_tf32_bits(u)


def bf16_from_f32(v: float) -> int:
    return lib().oracle_bf16_from_f32(v)


def bf16_from_f64(v: float) -> int:
    return lib().oracle_bf16_from_f64(v)


def split_weight(w: np.ndarray):
    """Returns (tf32(w) as float32, hi bf16 bits, lo bf16 bits)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    t = np.empty_like(w)
    hi = np.empty(w.shape, np.uint16)
    lo = np.empty(w.shape, np.uint16)
    lib().oracle_split_weight(_p(w), w.size, _p(t), _p(hi), _p(lo))
    return t, hi, lo


def prepare_weight(W: np.ndarray) -> np.ndarray:
    """Prepared-weight bytes (uint8, 384*d) rebuilt from the documented layout."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    d = W.shape[1] // 4
    out = np.zeros(192 * d, np.uint16)
    rc = lib().oracle_prepare_weight(_p(W), d, _p(out))
    if rc:
        raise ValueError(f"oracle_prepare_weight: status {rc}")
    return out.view(np.uint8)


def sinkhorn(logits: np.ndarray, eps: float, iters: int) -> np.ndarray:
    lg = np.ascontiguousarray(logits, dtype=np.float64).reshape(16)
    out = np.empty(16, np.float64)
    lib().oracle_sinkhorn(_p(lg), eps, iters, _p(out))
    return out.reshape(4, 4)


def _params(p: dict) -> _Params:
    return _Params(p["rms_eps"], p["pre_eps"], p["post_mult"], p["sinkhorn_eps"],
                   p["sinkhorn_iters"], p["norm_eps"])


def run(shifted: bool, X, x, post_prev, comb_prev, pre_lag, W, scale, base, norm_w,
        params: dict, tokens=None) -> dict:
    """Run the oracle on the listed tokens (all by default); see oracle_run."""
    X = np.ascontiguousarray(X, np.uint16)
    T, _, d = X.shape
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, np.int32)
    n = len(tok)
    if shifted:
        x = np.ascontiguousarray(x, np.uint16)
        post_prev = np.ascontiguousarray(post_prev, np.float32)
        comb_prev = np.ascontiguousarray(comb_prev, np.float32)
        pre_lag = np.ascontiguousarray(pre_lag, np.float32)
    else:
        x = post_prev = comb_prev = pre_lag = None
    tf32w, _, _ = split_weight(W)
    scale = np.ascontiguousarray(scale, np.float32)
    base = np.ascontiguousarray(base, np.float32)
    norm_w = None if norm_w is None else np.ascontiguousarray(norm_w, np.uint16)
    out = dict(
        xn=np.empty((n, 4, d), np.uint16), li=np.empty((n, d), np.uint16),
        layer_input=np.empty((n, d), np.uint16), mixes=np.empty((n, 24)),
        ssq=np.empty(n), rstd=np.empty(n), ssq_li=np.empty(n), rstd_li=np.empty(n),
        pre=np.empty((n, 4)), post=np.empty((n, 4)), comb=np.empty((n, 4, 4)))
    prm = _params(params)
    rc = lib().oracle_run(
        int(shifted), T, d, _p(tok), n, _p(X), _p(x), _p(post_prev), _p(comb_prev),
        _p(pre_lag), _p(tf32w), _p(scale), _p(base), _p(norm_w), ctypes.addressof(prm),
        _p(out["xn"]), _p(out["li"]), _p(out["layer_input"]), _p(out["mixes"]),
        _p(out["ssq"]), _p(out["rstd"]), _p(out["ssq_li"]), _p(out["rstd_li"]),
        _p(out["pre"]), _p(out["post"]), _p(out["comb"]))
    if rc:
        raise ValueError(f"oracle_run: status {rc}")
    return out


def boundary(inp, tokens=None, use_norm: bool = True) -> dict:
    """Shifted boundary on a ``workloads.Inputs`` set."""
    return run(True, inp.X, inp.x, inp.post_prev, inp.comb_prev, inp.pre_lag, inp.W,
               inp.scale, inp.base, inp.norm_w if use_norm else None, inp.params(), tokens)


def pre(inp, tokens=None, use_norm: bool = False) -> dict:
    """Non-shifted pre on a ``workloads.Inputs`` set (X as the residual)."""
    return run(False, inp.X, None, None, None, None, inp.W, inp.scale, inp.base,
               inp.norm_w if use_norm else None, inp.params(), tokens)


def pre_from_mixes(X, dot_mix, sqrsum, scale, base, norm_w, params: dict, tokens=None) -> dict:
    """Non-shifted pre from precomputed projection partials dot_mix [S,T,24] and
    sqrsum [S,T] (summed over S in order)."""
    X = np.ascontiguousarray(X, np.uint16)
    T, _, d = X.shape
    dot_mix = np.ascontiguousarray(dot_mix, np.float32)
    sqrsum = np.ascontiguousarray(sqrsum, np.float32)
    S = dot_mix.shape[0]
    assert dot_mix.shape == (S, T, 24) and sqrsum.shape == (S, T)
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, np.int32)
    n = len(tok)
    scale = np.ascontiguousarray(scale, np.float32)
    base = np.ascontiguousarray(base, np.float32)
    norm_w = None if norm_w is None else np.ascontiguousarray(norm_w, np.uint16)
    out = dict(layer_input=np.empty((n, d), np.uint16), li=np.empty((n, d), np.uint16),
               mixes=np.empty((n, 24)), ssq=np.empty(n), rstd=np.empty(n),
               rstd_li=np.empty(n), pre=np.empty((n, 4)), post=np.empty((n, 4)),
               comb=np.empty((n, 4, 4)))
    prm = _params(params)
    rc = lib().oracle_pre_from_mixes(
        T, d, S, _p(tok), n, _p(X), _p(dot_mix), _p(sqrsum), _p(scale), _p(base), _p(norm_w),
        ctypes.addressof(prm), _p(out["layer_input"]), _p(out["li"]), _p(out["mixes"]),
        _p(out["ssq"]), _p(out["rstd"]), _p(out["rstd_li"]), _p(out["pre"]), _p(out["post"]),
        _p(out["comb"]))
    if rc:
        raise ValueError(f"oracle_pre_from_mixes: status {rc}")
    return out
