"""Seeded generators (numpy PCG64).  Draw order per configuration:
per-token mean m_t, then the base values z, then the outlier channel set, then
the factor parameters [nb][5][(l, log u, v)], then log s_c of the SmoothQuant
multipliers.  "N(0, s)" means standard deviation s.

Value model: x[t, c] = (z[t, c] + m_t) * (k if c is an outlier channel else 1),
z ~ N(0, 1) (or Student-t with nu degrees of freedom and no mean), m_t ~ N(0, mean_std).
Factors: l, v ~ N(0, 0.5), u = exp(N(0, 0.3)).  SmoothQuant: s_c = exp(N(0, 0.5)),
passed to the quantizer as the fp32 multiplier 1/s_c.
bf16 activations are the fp32 draws rounded to nearest even, held as uint16 bits.
"""
from __future__ import annotations

import numpy as np

from .configs import Config, WeightConfig


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(a, np.float32).view(np.uint32)
    lsb = (b >> 16) & 1
    r = (b + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def f32_from_bf16_bits(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_activations(cfg: Config, rng: np.random.Generator, rows: int | None = None) -> np.ndarray:
    """Activations X[rows, d]: uint16 bf16 bits or float32, per cfg.dtype."""
    rows = cfg.rows if rows is None else rows
    d = cfg.d
    if cfg.dist == "gauss_mean":
        m = rng.normal(0.0, cfg.mean_std, size=(rows, 1)).astype(np.float32)
        z = rng.standard_normal(size=(rows, d), dtype=np.float32)
        x = z + m
    elif cfg.dist == "student_t":
        x = rng.standard_t(cfg.t_nu, size=(rows, d)).astype(np.float32)
    else:
        raise ValueError(cfg.dist)
    out_ch = rng.choice(d, size=cfg.n_outliers, replace=False)
    x[:, out_ch] *= np.float32(cfg.outlier_scale)
    if cfg.dtype == "bf16":
        return bf16_bits_from_f32(x)
    return np.ascontiguousarray(x, np.float32)


def make_params(nb: int, rng: np.random.Generator) -> np.ndarray:
    """Factor parameters [nb][5][3] float32 holding (l, u, v)."""
    g = rng.standard_normal(size=(nb, 5, 3))
    p = np.empty((nb, 5, 3), np.float32)
    p[..., 0] = 0.5 * g[..., 0]
    p[..., 1] = np.exp(0.3 * g[..., 1])
    p[..., 2] = 0.5 * g[..., 2]
    return p


def make_identity_params(nb: int) -> np.ndarray:
    p = np.zeros((nb, 5, 3), np.float32)
    p[..., 1] = 1.0
    return p


def make_rotation_params(nb: int, rng: np.random.Generator | None = None,
                         angle: float = np.pi / 4) -> np.ndarray:
    """Factor parameters [nb][5][3] (l, u, v) whose factors are plane rotations
    [[c, s], [-s, c]] (orthogonal, unit determinant): u = c, v = s, l = -s / c.
    Every factor at `angle`, or (with rng) angles uniform in (-pi/3, pi/3), so c >= 1/2."""
    th = (np.full((nb, 5), angle) if rng is None else rng.uniform(-np.pi / 3, np.pi / 3, size=(nb, 5)))
    c, s = np.cos(th), np.sin(th)
    p = np.empty((nb, 5, 3), np.float32)
    p[..., 0] = -s / c
    p[..., 1] = c
    p[..., 2] = s
    return p


def make_sq_mult(d: int, rng: np.random.Generator) -> np.ndarray:
    s = np.exp(rng.normal(0.0, 0.5, size=d))
    return (1.0 / s).astype(np.float32)


def make_inputs(cfg: Config, rows: int | None = None, seed: int | None = None):
    """(x, params, sq_mult) for a configuration, all from one seeded stream."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    x = make_activations(cfg, rng, rows)
    params = make_params(cfg.nb, rng)
    mult = make_sq_mult(cfg.d, rng)
    return x, params, mult


def make_activations_device(cfg: Config, seed: int, device="cuda"):
    """Same value model drawn on the GPU with torch's seeded generator (for the
    multi-gigabyte batched sweep, where host generation would dominate).  Returns a
    torch tensor: bfloat16 (cfg.dtype == "bf16") or float32."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    rows, d = cfg.rows, cfg.d
    if cfg.dist == "gauss_mean":
        m = torch.randn((rows, 1), generator=g, device=device) * cfg.mean_std
        x = torch.randn((rows, d), generator=g, device=device)
        x += m
    else:
        raise ValueError("device generation supports the gaussian-mean model only")
    out_ch = torch.randperm(d, generator=g, device=device)[: cfg.n_outliers]
    x[:, out_ch] *= cfg.outlier_scale
    return x.to(torch.bfloat16) if cfg.dtype == "bf16" else x


def make_weights(cfg: WeightConfig, seed: int | None = None):
    """(w, params): weights W[rows, d] (uint16 bf16 bits or float32) drawn as
    N(0, std * exp(N(0, row_spread))) per output row, then the factor parameters of
    the d/32 input blocks, from one seeded stream."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    rs = np.exp(rng.normal(0.0, cfg.row_spread, size=(cfg.rows, 1))).astype(np.float32)
    w = rng.standard_normal(size=(cfg.rows, cfg.d), dtype=np.float32) * np.float32(cfg.std) * rs
    params = make_params(cfg.nb, rng)
    if cfg.dtype == "bf16":
        return bf16_bits_from_f32(w), params
    return np.ascontiguousarray(w, np.float32), params


def make_modulation(n_samples: int, d: int, rng: np.random.Generator):
    """(shift, scale) float32 [n_samples, d] of the adaptive-norm modulation:
    scale ~ N(0, 0.3), shift ~ N(0, 0.5), drawn in that order."""
    scale = rng.normal(0.0, 0.3, size=(n_samples, d)).astype(np.float32)
    shift = rng.normal(0.0, 0.5, size=(n_samples, d)).astype(np.float32)
    return shift, scale
