"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module only draws numbers and lays them out. It holds none of the
method's arithmetic (no differences, scores, levels, schedules or attention),
so both the HIP path and the CPU oracle can consume its output without
sharing any computation.

Seeds are 20260000 + 100*cfg_id + role, with roles
  1 x0 background, 2 eps, 3 texture mask, 4/5/6 Q/K/V, 7 active-block mask,
  8 moving-texture field, 9/10/11 Q/K/V drift directions (schedule run),
  12 random block scores (random-masking index source).

The pages evaluate on real Flux-1-dev / Wan2.1 generations; these inputs stand
in for them with the same token grids, following the configuration recipe:
x_t = (1 - t) * x0 + t * eps with t linear from 1.0 to 0.84 over the K warm-up
latents, x0 smooth in background blocks and textured in the rest.
"""
from __future__ import annotations

import numpy as np

ROLE_X0, ROLE_EPS, ROLE_TEX, ROLE_Q, ROLE_K, ROLE_V = 1, 2, 3, 4, 5, 6
ROLE_ACTIVE, ROLE_FIELD, ROLE_DQ, ROLE_DK, ROLE_DV = 7, 8, 9, 10, 11
ROLE_RANDOM_SCORES = 12


def rng(cfg_id: int, role: int, extra: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(20260000 + 100 * cfg_id + role + 1000000 * extra))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding here expects finite inputs")
    # finite inputs never carry past bit 31 here
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _pixel_block_mask(block_flags: np.ndarray, F, H, W, block) -> np.ndarray:
    """Expand a [nBF, nBH, nBW] boolean block map to an [F, H, W] pixel map."""
    bF, bH, bW = block
    m = np.repeat(np.repeat(np.repeat(block_flags, bF, 0), bH, 1), bW, 2)
    return m[:F, :H, :W]


def texture_blocks(cfg) -> np.ndarray:
    """Boolean [nBF, nBH, nBW]: blocks whose x0 carries high-frequency texture."""
    nBF, nBH, nBW = cfg.block_grid
    B = nBF * nBH * nBW
    n_tex = int(round(cfg.texture_frac * B))
    perm = rng(cfg.cfg_id, ROLE_TEX).permutation(B)
    flags = np.zeros(B, dtype=bool)
    flags[perm[:n_tex]] = True
    return flags.reshape(nBF, nBH, nBW)


def latent_parts(cfg):
    """Returns (smooth, texture, texmask, eps) as fp64/bool arrays [C,F,H,W]."""
    C, F, H, W = cfg.C, cfg.F, cfg.H, cfg.W
    g = rng(cfg.cfg_id, ROLE_X0)
    alpha = g.uniform(0.25, 1.0, C)
    beta = g.uniform(0.25, 1.0, C)
    phi = g.uniform(0.0, 2.0 * np.pi, C)
    lo, hi = cfg.omega
    omega = np.full(C, lo) if lo == hi else g.uniform(lo, hi, C)
    f = np.arange(F, dtype=np.float64)[None, :, None, None]
    h = np.arange(H, dtype=np.float64)[None, None, :, None]
    w = np.arange(W, dtype=np.float64)[None, None, None, :]
    smooth = np.sin(2.0 * np.pi * (alpha[:, None, None, None] * h / H
                                   + beta[:, None, None, None] * w / W)
                    + phi[:, None, None, None] + omega[:, None, None, None] * f)
    if cfg.texture_kind == "white":
        texture = rng(cfg.cfg_id, ROLE_FIELD).standard_normal((C, F, H, W))
    else:
        # one field per channel, moved by (+1, +1) latent pixels per frame
        field = rng(cfg.cfg_id, ROLE_FIELD).standard_normal((C, H, W))
        texture = np.stack([np.roll(field, shift=(fr, fr), axis=(1, 2))
                            for fr in range(F)], axis=1)
    texmask = _pixel_block_mask(texture_blocks(cfg), F, H, W, cfg.block)[None]
    eps = rng(cfg.cfg_id, ROLE_EPS).standard_normal((C, F, H, W))
    return smooth, texture, np.broadcast_to(texmask, (C, F, H, W)), eps


def warmup_t(K: int) -> np.ndarray:
    return np.linspace(1.0, 0.84, K)


def latents(cfg, signal: bool = False) -> np.ndarray:
    """Warm-up latent history, fp32 [K, C, F, H, W], C-contiguous.

    signal=False is the literal recipe: x_k is affine in k, so every exact
    second step-difference vanishes and only fp32 storage rounding remains.
    signal=True multiplies the texture term by (1 - t_k) / (1 - t_{K-1}), which
    makes textured blocks genuinely non-affine in k (quadratic)."""
    smooth, texture, texmask, eps = latent_parts(cfg)
    t = warmup_t(cfg.K)
    out = np.empty(cfg.latent_shape, dtype=np.float32)
    for k in range(cfg.K):
        s = (1.0 - t[k]) / (1.0 - t[-1]) if signal else 1.0
        x0 = np.where(texmask, s * texture, smooth)
        out[k] = ((1.0 - t[k]) * x0 + t[k] * eps).astype(np.float32)
    return out


def qkv_bits(cfg, n_tokens: int | None = None, extra: int = 0, which: str = "qkv"):
    """bf16 bit patterns (uint16) of Q, K, V, each [N, heads, d], N(0,1)*scale.
    `which` selects a subset (e.g. "q"); each tensor has its own seed."""
    N = cfg.N if n_tokens is None else n_tokens
    shape = (N, cfg.heads, cfg.d)
    out = []
    for role in [{"q": ROLE_Q, "k": ROLE_K, "v": ROLE_V}[c] for c in which]:
        x = rng(cfg.cfg_id, role, extra).standard_normal(shape, dtype=np.float32)
        out.append(f32_to_bf16_bits(x * np.float32(cfg.qkv_scale)))
    return tuple(out)


def active_level_map(cfg, frac: float) -> np.ndarray:
    """uint8 [B] level map with round(frac*B) seeded-random blocks at level 3
    (Active) and the rest at level 1 (Static). At an interleaved step where only
    Active tokens are due, the schedule then selects exactly those blocks'
    tokens; this is how the attention-only workloads pick their active set."""
    B = cfg.B
    n = int(round(frac * B))
    perm = rng(cfg.cfg_id, ROLE_ACTIVE, int(round(frac * 1000))).permutation(B)
    lv = np.ones(B, dtype=np.uint8)
    lv[perm[:n]] = 3
    return lv


def random_block_scores(cfg, extra: int = 0) -> np.ndarray:
    """fp32 [B] uniform draws in [0, 1): ranking blocks by them instead of by
    the analyzer's complexity gives the random-masking index source (the
    pages' ablation); the level bucketing and schedule stay the same."""
    return rng(cfg.cfg_id, ROLE_RANDOM_SCORES, extra).random(cfg.B, dtype=np.float32)


def drift_qkv_f32(cfg, seed_extra: int = 0):
    """fp32 base and direction tensors for the multi-step run (see
    step_qkv_bits)."""
    shape = (cfg.N, cfg.heads, cfg.d)
    base = [rng(cfg.cfg_id, r, seed_extra).standard_normal(shape, dtype=np.float32)
            for r in (ROLE_Q, ROLE_K, ROLE_V)]
    dirs = [rng(cfg.cfg_id, r, seed_extra).standard_normal(shape, dtype=np.float32)
            for r in (ROLE_DQ, ROLE_DK, ROLE_DV)]
    return base, dirs


def step_coeffs(s: int):
    """fp32 (cos, sin) of 0.05 s: step-s tensors rotate from base towards dir,
    so every step's rows differ while each element stays N(0, 1), the scale
    of normalised activations."""
    return np.float32(np.cos(0.05 * s)), np.float32(np.sin(0.05 * s))


def step_qkv_bits(base, dirs, s: int):
    """Step-s Q/K/V bits: bf16(cos(0.05 s) base + sin(0.05 s) dir), fp32
    multiplies then add, rounded to nearest even."""
    c, sn = step_coeffs(s)
    return tuple(f32_to_bf16_bits(c * b + sn * d) for b, d in zip(base, dirs))
