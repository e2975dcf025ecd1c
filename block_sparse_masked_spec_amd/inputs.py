"""Seeded synthetic inputs for masked sparse attention.

This module is shared by the GPU path's tests and bench and by the oracle's
tests.  It holds no part of the attention arithmetic: it only draws numbers.

Recipe: one ``torch.Generator`` seeded with ``seed`` draws Q, then K, then V
as fp32 standard-normal tensors of shape [B, H, T, d] on the CPU; for bf16
they are then rounded to bf16 (round-to-nearest-even).  The oracle consumes
the stored values exactly, so parity never depends on the generator.
"""
from __future__ import annotations

import torch

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def qkv(B: int, H: int, T: int, d: int, dtype: str = "bf16", seed: int = 0):
    """Return CPU tensors (Q, K, V), each [B, H, T, d], iid N(0, 1)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shape = (B, H, T, d)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        out.append(x.to(DTYPES[dtype]).contiguous())
    return tuple(out)


def scaled(x: torch.Tensor, s: float) -> torch.Tensor:
    """x * s rounded back to x's dtype (used to make sharper attention rows)."""
    return (x.to(torch.float32) * s).to(x.dtype).contiguous()
