"""The attention workloads of the Stable Diffusion 1.x UNet used for tests and
benchmarks, as seeded synthetic inputs (no trained weights or activations are
needed: the kernels' cost and correctness depend only on shapes and value
ranges).

Seeds: 1000 * config_index + {0: Q, 1: K, 2: V}.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import synth


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str          # 'f32', 'f16', 'bf16'
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    what: str = ""

    @property
    def scale(self) -> float:
        # the scale handed to the kernels is a float32 value
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> int:
        """Useful attention FLOPs: 2*Nq*Nk*d for Q K^T plus the same for P V."""
        return 4 * self.B * self.H * self.Nq * self.Nk * self.d

    def inputs(self, dtype: str | None = None):
        """Seeded (q, k, v) as numpy arrays of the element type (bf16 as uint16)."""
        dt = dtype or self.dtype
        s = 1000 * self.index
        q = synth.tensor(s + 0, (self.B, self.H, self.Nq, self.d), dt, self.sigma_qk)
        k = synth.tensor(s + 1, (self.B, self.H, self.Nk, self.d), dt, self.sigma_qk)
        v = synth.tensor(s + 2, (self.B, self.H, self.Nk, self.d), dt, self.sigma_v)
        return q, k, v

    def with_dtype(self, dtype: str) -> "Config":
        return Config(self.name, self.index, self.B, self.H, self.Nq, self.Nk, self.d, dtype,
                      self.sigma_qk, self.sigma_v, self.what)


CONFIGS = {
    "tiny": Config("tiny", 0, 1, 1, 64, 64, 40, "f32", what="tiny self-attention, fp32"),
    "tiny8": Config("tiny8", 1, 1, 1, 8, 8, 40, "f32", what="tiny self-attention at N=8, fp32"),
    "sd512_self": Config("sd512_self", 2, 2, 8, 4096, 4096, 40, "f16",
                         what="SD 512x512 UNet top-level self-attention (64x64 latent)"),
    "sd512_cross": Config("sd512_cross", 3, 2, 8, 4096, 77, 40, "f16",
                          what="SD top-level cross-attention over 77 text tokens"),
    "level2_self": Config("level2_self", 4, 2, 8, 1024, 1024, 80, "f16",
                          what="UNet level-2 self-attention"),
    "level3_self": Config("level3_self", 5, 2, 8, 256, 256, 160, "f16",
                          what="UNet level-3 self-attention"),
    "level4_self": Config("level4_self", 6, 2, 8, 64, 64, 160, "f16",
                          what="UNet level-4 self-attention"),
    "sd1024_self": Config("sd1024_self", 7, 2, 8, 16384, 16384, 40, "f16", sigma_qk=1.5,
                          what="1024x1024-image self-attention stress (128x128 latent), "
                               "Q, K with sigma 1.5"),
}
