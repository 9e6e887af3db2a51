"""Workload presets for the Jano hot path.

Shapes follow the model token grids the Jano pages evaluate on (Flux-1-dev
images, Wan2.1 480p and 720p video, the latter "75k tokens"; Jano pages,
technical summary, results section). Numbers the pages leave open (block
size, warm-up latent count, update periods, phase lengths) are fixed here.

Notation:
  latent      [C, F, H, W] fp32 per step, K warm-up latents stacked in front
  patch       (pF, pH, pW) latent pixels per token along each axis
  block       (bF, bH, bW) analyzer block in latent pixels (1x4x4 tokens)
  tokens      (F/pF) x (H/pH) x (W/pW), token n = (f*Ht + h)*Wt + w
  heads, d    attention heads and head dimension, Q/K/V laid out [N, H, d]
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Schedule:
    """Interleaved-pipeline phases (Jano pages, technical summary, §2
    "adaptive generation": warm-up, interleaved, cool-down)."""
    T: int = 50            # denoising steps
    W: int = 5             # dense warm-up steps (they feed the analyzer)
    Cd: int = 5            # dense cool-down steps
    periods: tuple = (4, 2, 1)  # update period of Static, Moderate, Active


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    K: int
    C: int
    F: int
    H: int
    W: int
    patch: tuple
    block: tuple
    heads: int
    d: int
    texture_frac: float
    texture_kind: str          # "white" (image-like) or "moving" (video-like)
    qkv_scale: float = 1.0     # Q/K/V ~ N(0,1) * qkv_scale, rounded to bf16
    active_fracs: tuple = (0.3,)
    static_permille: int = 400
    moderate_permille: int = 300
    omega: tuple = (0.05, 0.15)  # temporal drift of the smooth background
    schedule: Schedule = field(default_factory=Schedule)

    @property
    def token_grid(self):
        pF, pH, pW = self.patch
        return (self.F // pF, self.H // pH, self.W // pW)

    @property
    def N(self):
        Ft, Ht, Wt = self.token_grid
        return Ft * Ht * Wt

    @property
    def block_grid(self):
        bF, bH, bW = self.block
        return (-(-self.F // bF), -(-self.H // bH), -(-self.W // bW))

    @property
    def B(self):
        a, b, c = self.block_grid
        return a * b * c

    @property
    def latent_shape(self):
        return (self.K, self.C, self.F, self.H, self.W)

    @property
    def latent_bytes(self):
        K, C, F, H, W = self.latent_shape
        return K * C * F * H * W * 4


TINY = Config("tiny", 1, K=8, C=16, F=3, H=16, W=16, patch=(1, 1, 1),
              block=(1, 4, 4), heads=2, d=64, texture_frac=0.30,
              texture_kind="white", qkv_scale=1.0 / 8.0, active_fracs=(0.3,),
              omega=(0.2, 0.2))
IMAGE = Config("image", 2, K=5, C=16, F=1, H=128, W=128, patch=(1, 2, 2),
               block=(1, 8, 8), heads=24, d=128, texture_frac=0.30,
               texture_kind="white", active_fracs=(0.3, 1.0))
V480 = Config("480p", 3, K=5, C=16, F=21, H=60, W=104, patch=(1, 2, 2),
              block=(1, 8, 8), heads=12, d=128, texture_frac=0.25,
              texture_kind="moving", active_fracs=(0.25,))
V720 = Config("720p", 4, K=5, C=16, F=21, H=90, W=160, patch=(1, 2, 2),
              block=(1, 8, 8), heads=40, d=128, texture_frac=0.25,
              texture_kind="moving", active_fracs=(0.10, 0.25, 0.50, 1.0))
# 50-step interleaved run on the 480p grid.
SCHED480 = Config("sched480p", 5, K=5, C=16, F=21, H=60, W=104,
                  patch=(1, 2, 2), block=(1, 8, 8), heads=12, d=128,
                  texture_frac=0.25, texture_kind="moving",
                  active_fracs=(), schedule=Schedule(T=50, W=5, Cd=5,
                                                     periods=(4, 2, 1)))

CONFIGS = {c.cfg_id: c for c in (TINY, IMAGE, V480, V720, SCHED480)}
BY_NAME = {c.name: c for c in CONFIGS.values()}
