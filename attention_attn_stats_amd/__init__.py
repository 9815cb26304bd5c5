"""MI355X (gfx950) attention for the Stable Diffusion UNet: the partially fused
softmax (row statistics + fused softmax-times-V) and the FlashAttention single
pass, as HIP kernels behind a C ABI (include/attn.h, libattn.so); plus the
partially fused form over a stored logit matrix (scores, scores_stats,
scores_pv), strided [B, N, H*d] views, and the UNet's two other specialised
kernels: group normalisation in one launch (group_norm) and the GELU-gated
product (geglu).

This Python layer only marshals arguments: tensors are PyTorch device tensors
(PyTorch supplies memory and streams), every arithmetic step runs in the HIP
kernels.  See api.py for the entry points.
"""
from .api import (AttnError, default_variant, flash, forward, geglu, group_norm, pv, scores,  # noqa: F401
                  scores_pv, scores_stats, select, select_reset, stats)

__all__ = ["stats", "pv", "flash", "forward", "select", "select_reset", "default_variant",
           "scores", "scores_stats", "scores_pv", "group_norm", "geglu", "AttnError"]
