"""Seeded synthetic inputs for the ReLU-gated FFN workloads.

The pages measure trained 0.5B-2B models at context 2048 (intellectnews.ru
TwELL article, section "Результаты тестов") and report activation statistics
(fewer than 2% of FFN neurons active at 1.5B, and fewer non-zeros at 2B than
at 0.5B: gate.com/es post 20977915, paragraph 4; gate.com/id post 20978418,
paragraphs 6-7).  No trained weights or text are available, so every tensor is
drawn here with the shapes and activation structure of those workloads:

* every draw comes from ``Generator(PCG64(SeedSequence([seed, tensor_id])))``
  in float32 and, for bf16 workloads, is rounded to bf16 with
  round-to-nearest-even; the arrays returned are float32 arrays whose values
  are exactly representable in the workload dtype;
* weights are N(0, std = 1/sqrt(fan_in)); x is N(0, 1) except in the tiny
  float32 workload, where it is N(0, 1/sqrt(d));
* each alive neuron n gets a gate bias b_n = sigma_x * ||w_n|| * Phi^-1(p_n)
  (w_n the rounded gate row), so that over Gaussian x the pre-activation
  x.w_n + b_n is positive with probability p_n; dead neurons get b_n = -1e4
  and never fire;
* p_n follows a Zipf law over a seeded random ranking of the alive neurons,
  p_n = min(0.99, c * rank^-s), with c found by bisection so that the mean
  over all neurons (dead included) equals the target density.

Nothing in this module computes the FFN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
from scipy.special import ndtri

# Tensor ids of the seeded streams.
_ID_X, _ID_WG, _ID_WU, _ID_WD, _ID_DY, _ID_RANK, _ID_ROWS, _ID_XDEC = range(8)


@dataclass(frozen=True)
class FFNConfig:
    name: str
    T: int
    d: int
    f: int
    dtype: str                      # "f32" or "bf16": dtype of x, weights, bias, dY
    density: float                  # target mean P(gate > 0) over all f neurons
    zipf_s: Optional[float] = None  # None: every alive neuron has p_n = density
    dead_frac: float = 0.0
    x_std: float = 1.0
    hybrid_rows_frac: float = 0.0   # fraction of token rows with scaled-up x
    hybrid_rows_density: float = 0.0
    tau_frac: Optional[float] = None  # dense-row threshold as a fraction of f
    decode_T: Optional[int] = None
    R: int = 16
    C: int = 64
    description: str = ""


CONFIGS = {
    "tiny_f32": FFNConfig(
        "tiny_f32", T=64, d=128, f=512, dtype="f32", density=0.05,
        x_std=1.0 / math.sqrt(128),
        description="tiny fp32 gated FFN fwd, T=64 d=128 f=512, uniform 5% gate density"),
    "0.5b": FFNConfig(
        "0.5b", T=8 * 2048, d=1024, f=4096, dtype="bf16", density=0.03,
        zipf_s=1.1, dead_frac=0.10,
        description="0.5B-scale layer fwd, 3% density, Zipf(1.1), 10% dead"),
    "1.5b": FFNConfig(
        "1.5b", T=16 * 2048, d=2048, f=5632, dtype="bf16", density=0.015,
        zipf_s=1.1, dead_frac=0.15,
        description="1.5B-scale layer fwd, 1.5% density, Zipf(1.1), 15% dead"),
    "2b": FFNConfig(
        "2b", T=16 * 2048, d=2304, f=9216, dtype="bf16", density=0.0093,
        zipf_s=1.2, dead_frac=0.20, decode_T=64,
        description="2B-scale layer fwd, 0.93% density, Zipf(1.2), 20% dead, plus T=64 decode"),
    "hybrid": FFNConfig(
        "hybrid", T=8 * 2048, d=2048, f=5632, dtype="bf16", density=0.01,
        hybrid_rows_frac=0.05, hybrid_rows_density=0.30, tau_frac=0.10,
        description="hybrid training fwd+bwd: 95% rows at 1%, 5% rows at 30%, fp32 grads"),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float32 values that are exactly bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id])))


def _normal(seed, tid, shape, std, dtype):
    a = _rng(seed, tid).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_bf16(a) if dtype == "bf16" else a


def zipf_probs(f: int, density: float, s: Optional[float], dead_frac: float,
               rng: np.random.Generator):
    """Per-neuron activation probabilities p_n and the dead-neuron mask."""
    n_dead = int(round(dead_frac * f))
    alive = f - n_dead
    perm = rng.permutation(f)
    p = np.zeros(f, dtype=np.float64)
    dead = np.zeros(f, dtype=bool)
    dead[perm[alive:]] = True
    if s is None:
        p[perm[:alive]] = density * f / alive
        return p, dead
    r = np.arange(1, alive + 1, dtype=np.float64)
    lo, hi = 0.0, 1.0
    while np.minimum(0.99, hi * r ** (-s)).sum() / f < density:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(0.99, mid * r ** (-s)).sum() / f < density:
            lo = mid
        else:
            hi = mid
    p[perm[:alive]] = np.minimum(0.99, hi * r ** (-s))
    return p, dead


@dataclass
class Workload:
    cfg: FFNConfig
    seed: int
    T: int
    d: int
    f: int
    x: np.ndarray          # [T, d]
    WgT: np.ndarray        # [f, d]  gate weights, neuron-major
    bg: np.ndarray         # [f]     gate bias
    WuT: np.ndarray        # [f, d]  up weights, neuron-major
    Wd: np.ndarray         # [f, d]  down weights, neuron-major
    p: np.ndarray          # [f]     target activation probability per neuron
    dead: np.ndarray       # [f]     bool
    dY: Optional[np.ndarray] = None        # [T, d] output gradient (training workload)
    tau: Optional[int] = None              # dense-row threshold (training workload)
    dense_rows: Optional[np.ndarray] = None  # rows drawn at the higher density
    extra: dict = field(default_factory=dict)

    @property
    def dtype(self) -> str:
        return self.cfg.dtype


def make_workload(name: str, seed: int = 0, T: Optional[int] = None,
                  d: Optional[int] = None, f: Optional[int] = None,
                  decode: bool = False, grad: bool = False) -> Workload:
    """Draw the inputs of workload ``name``; T, d, f may be overridden (smaller
    parity cases keep the same value distributions and activation structure).
    grad=True also draws an output gradient dY ~ N(0, 1) and a dense-row
    threshold tau = floor(0.10 * f) for workloads that do not define them."""
    cfg = CONFIGS[name]
    d = cfg.d if d is None else d
    f = cfg.f if f is None else f
    if decode:
        if cfg.decode_T is None:
            raise ValueError(f"workload {name} has no decode pass")
        T = cfg.decode_T if T is None else T
    T = cfg.T if T is None else T
    dt = cfg.dtype
    w_in = 1.0 / math.sqrt(d)
    WgT = _normal(seed, _ID_WG, (f, d), w_in, dt)
    WuT = _normal(seed, _ID_WU, (f, d), w_in, dt)
    Wd = _normal(seed, _ID_WD, (f, d), 1.0 / math.sqrt(f), dt)
    x = _normal(seed, _ID_XDEC if decode else _ID_X, (T, d), 1.0, "f32")
    if cfg.x_std != 1.0:
        x *= np.float32(cfg.x_std)

    p, dead = zipf_probs(f, cfg.density, cfg.zipf_s, cfg.dead_frac, _rng(seed, _ID_RANK))
    wnorm = np.sqrt((WgT.astype(np.float64) ** 2).sum(axis=1))
    sigma = cfg.x_std * wnorm
    b = np.where(dead, -1.0e4, sigma * ndtri(np.clip(p, 1e-12, 1 - 1e-12)))
    bg = b.astype(np.float32)

    dense_rows = None
    if cfg.hybrid_rows_frac > 0:
        n_rows = int(round(cfg.hybrid_rows_frac * T))
        dense_rows = np.sort(_rng(seed, _ID_ROWS).choice(T, size=n_rows, replace=False))
        alpha = ndtri(cfg.density) / ndtri(cfg.hybrid_rows_density)
        x[dense_rows] *= np.float32(alpha)
    if dt == "bf16":
        x = round_bf16(x)
        bg = round_bf16(bg)

    dY = None
    tau = None
    if cfg.tau_frac is not None or grad:
        dY = _normal(seed, _ID_DY, (T, d), 1.0, dt)
        tau = int(math.floor((cfg.tau_frac if cfg.tau_frac is not None else 0.10) * f))
    return Workload(cfg=cfg, seed=seed, T=T, d=d, f=f, x=x, WgT=WgT, bg=bg, WuT=WuT,
                    Wd=Wd, p=p, dead=dead, dY=dY, tau=tau, dense_rows=dense_rows)
