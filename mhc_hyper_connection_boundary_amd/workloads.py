"""Seeded synthetic inputs for the mHC layer boundary.

This module draws random numbers and nothing else: it holds none of the
boundary's arithmetic (no residual update, no projection, no sigmoid, no
Sinkhorn).  Both the CPU oracle and the GPU path read the arrays it returns,
so a draw here can never hide a difference between them.

Shapes follow the shifted boundary's interface (vLLM DeepSeek-V4.1
"mhc_boundary" page, API function ``mhc_shifted_post_pre_boundary``):

    residual X  [T, 4, d]  bf16      block output x  [T, d]   bf16
    post_prev   [T, 4]     fp32      comb_prev       [T, 4, 4] fp32 (row j = source stream)
    pre_lag     [T, 4]     fp32      weight W        [24, 4d] fp32 (rows: 4 pre | 4 post | 16 comb)
    scale       [3]        fp32      base            [24]     fp32
    norm_w      [d]        bf16

BF16 arrays are returned as their uint16 bit patterns.

Draw order (fixed, one ``numpy.random.default_rng(seed)`` stream):
X, x, post_prev, comb_prev mixture weights, pre_lag, W, base, norm_w noise,
then the stress permutation, then (routed comb_prev family only) the dominant
permutation of every token.
"""
from __future__ import annotations

import dataclasses
import itertools

import numpy as np

N_HC = 4
MIXES = 24

# The 24 permutation matrices of order 4, used to draw doubly stochastic
# matrices as convex combinations (Birkhoff-von Neumann).
_PERMS = np.array(list(itertools.permutations(range(N_HC))), dtype=np.int64)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    d: int
    T: int
    seed: int
    norm: str = "noisy"       # "ones": norm_w = 1; "noisy": bf16(1 + N(0, 0.05))
    stress: bool = False      # 1% of tokens x1e3, 1% x1e-3, comb bases N(0, 3)
    sinkhorn_iters: int = 20
    eps: float = 1e-6         # pre eps and Sinkhorn eps
    rms_eps: float = 1e-6     # mix RMS eps and layer-input RMSNorm eps
    post_mult: float = 2.0
    scale: tuple = (0.01, 0.01, 0.01)  # per-group scales: pre, post, comb
    comb_family: str = "mixture"  # "mixture": Dirichlet(1) weights over the 24
                                  # permutations; "routed": 0.9 on one permutation
                                  # per token plus 0.1 of such a mixture


CONFIGS = {
    c.name: c
    for c in (
        Config("tiny", d=256, T=8, seed=0, norm="ones"),
        Config("decode", d=7168, T=32, seed=1),
        Config("decode_wave", d=7168, T=256, seed=2),
        Config("prefill", d=7168, T=8192, seed=3),
        Config("stress", d=4096, T=16384, seed=4, stress=True),
    )
}


@dataclasses.dataclass
class Inputs:
    cfg: Config
    X: np.ndarray          # uint16 [T, 4, d]
    x: np.ndarray          # uint16 [T, d]
    post_prev: np.ndarray  # float32 [T, 4]
    comb_prev: np.ndarray  # float32 [T, 4, 4]
    pre_lag: np.ndarray    # float32 [T, 4]
    W: np.ndarray          # float32 [24, 4d]
    scale: np.ndarray      # float32 [3]
    base: np.ndarray       # float32 [24]
    norm_w: np.ndarray     # uint16 [d]

    @property
    def T(self) -> int:
        return self.X.shape[0]

    @property
    def d(self) -> int:
        return self.X.shape[2]

    def params(self) -> dict:
        c = self.cfg
        return dict(rms_eps=c.rms_eps, pre_eps=c.eps, post_mult=c.post_mult,
                    sinkhorn_eps=c.eps, sinkhorn_iters=c.sinkhorn_iters,
                    norm_eps=c.rms_eps)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (torch's CPU cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _doubly_stochastic(rng: np.random.Generator, T: int) -> np.ndarray:
    """[T,4,4] positive doubly stochastic matrices: Dirichlet(1) weights over
    the 24 permutation matrices."""
    w = rng.dirichlet(np.ones(len(_PERMS)), size=T)          # [T, 24]
    m = np.zeros((T, N_HC, N_HC), dtype=np.float64)
    rows = np.arange(N_HC)
    for p, perm in enumerate(_PERMS):
        m[:, rows, perm] += w[:, p:p + 1]
    return m.astype(np.float32)


def _routed(rng: np.random.Generator, mixture: np.ndarray) -> np.ndarray:
    """Strongly routed doubly stochastic matrices: 0.9 of one permutation
    matrix (drawn per token) plus 0.1 of the given mixture, so most of each
    destination stream comes from one source stream."""
    T = mixture.shape[0]
    pick = rng.integers(0, len(_PERMS), size=T)
    m = np.zeros((T, N_HC, N_HC), dtype=np.float64)
    m[np.arange(T)[:, None], np.arange(N_HC)[None, :], _PERMS[pick]] = 1.0
    return (0.9 * m + 0.1 * mixture.astype(np.float64)).astype(np.float32)


def make_inputs(cfg: Config | str, T: int | None = None) -> Inputs:
    """Draw one input set.  ``T`` overrides the token count (same recipe)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if T is not None:
        cfg = dataclasses.replace(cfg, T=T)
    T, d = cfg.T, cfg.d
    rng = np.random.default_rng(cfg.seed)
    X = rng.standard_normal((T, N_HC, d), dtype=np.float32)
    x = rng.standard_normal((T, d), dtype=np.float32)
    post_prev = rng.uniform(0.0, 2.0, size=(T, N_HC)).astype(np.float32)
    comb_prev = _doubly_stochastic(rng, T)
    pre_lag = rng.uniform(0.0, 1.0, size=(T, N_HC)).astype(np.float32)
    W = (rng.standard_normal((MIXES, N_HC * d)) / np.sqrt(N_HC * d)).astype(np.float32)
    scale = np.array(cfg.scale, dtype=np.float32)
    assert scale.shape == (3,)
    base = (rng.standard_normal(MIXES) * 0.1).astype(np.float32)
    if cfg.norm == "ones":
        norm_w = np.ones(d, dtype=np.float32)
    else:
        norm_w = (1.0 + rng.standard_normal(d) * 0.05).astype(np.float32)
    if cfg.stress:
        base[8:] = (rng.standard_normal(MIXES - 8) * 3.0).astype(np.float32)
        perm = rng.permutation(T)
        k = -(-T // 100)  # ceil(1% of T)
        X[perm[:k]] *= np.float32(1e3)
        X[perm[k:2 * k]] *= np.float32(1e-3)
    if cfg.comb_family == "routed":
        comb_prev = _routed(rng, comb_prev)
    else:
        assert cfg.comb_family == "mixture", cfg.comb_family
    inp = Inputs(cfg, to_bf16_bits(X), to_bf16_bits(x), post_prev, comb_prev,
                 pre_lag, W, scale, base, to_bf16_bits(norm_w))
    _check_no_subnormals(inp)
    return inp


def make_partials(T: int, d: int, splits: int, seed: int):
    """Projection partials as a split-K GEMM hands them over, drawn at random:
    dot_mix [splits, T, 24] FP32 with N(0, 1/splits) entries (their sum has the
    unit spread of the fused projection of unit-variance activations with the
    1/sqrt(4d) weights above) and sqrsum [splits, T] FP32, each split's share of
    a total near 4d (4d/splits times U(0.5, 1.5)).  A separate stream so that
    the residual draws stay as they are."""
    rng = np.random.default_rng(10_000 + seed)
    dot_mix = (rng.standard_normal((splits, T, MIXES)) / np.sqrt(splits)).astype(np.float32)
    sqrsum = (N_HC * d / splits * rng.uniform(0.5, 1.5, (splits, T))).astype(np.float32)
    return dot_mix, sqrsum


def _check_no_subnormals(inp: Inputs) -> None:
    """No input holds a nonzero value below 2^-126, so flush-to-zero and IEEE
    subnormal handling cannot differ on them."""
    tiny = np.float32(2.0 ** -126)
    for name in ("post_prev", "comb_prev", "pre_lag", "W", "scale", "base"):
        a = np.abs(getattr(inp, name))
        assert not np.any((a > 0) & (a < tiny)), name
    for name in ("X", "x", "norm_w"):
        a = np.abs(bf16_bits_to_f32(getattr(inp, name)))
        assert not np.any((a > 0) & (a < tiny)), name
