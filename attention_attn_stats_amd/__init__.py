"""MI355X (gfx950) attention for the Stable Diffusion UNet: the partially fused
softmax (row statistics + fused softmax-times-V) and the FlashAttention single
pass, as HIP kernels behind a C ABI (include/attn.h, libattn.so).

This Python layer only marshals arguments: tensors are PyTorch device tensors
(PyTorch supplies memory and streams), every arithmetic step runs in the HIP
kernels.  See api.py for the entry points.
"""
from .api import (AttnError, default_variant, flash, forward, pv, select, select_reset,  # noqa: F401
                  stats)

__all__ = ["stats", "pv", "flash", "forward", "select", "select_reset", "default_variant", "AttnError"]
