"""Seeded synthetic inputs for the compressed-attention layer.

This module only draws random numbers. It holds none of the layer's
arithmetic, so the GPU path (tests, smoke, bench) and the CPU oracle may
both consume what it produces: tensors are drawn on the GPU with torch's
seeded Philox generator, one stream per (seed, name), and the tests copy
the rows they check back to the host for the oracle, which therefore sees
exactly the values the kernels read.
"""
from __future__ import annotations

import zlib


def _generator(seed: int, name: str, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + zlib.crc32(name.encode())) & 0x7FFFFFFFFFFFFFFF)
    return g


def normal_device(seed: int, name: str, shape, std: float = 1.0, dtype: str = "bf16", device="cuda"):
    """Seeded N(0, std^2) values drawn as float32, rounded to bf16 (nearest even) for dtype "bf16"."""
    import torch

    x = torch.randn(shape, generator=_generator(seed, name, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def uniform_device(seed: int, name: str, shape, device="cuda"):
    """Seeded U(0, 1) float32 values (head weights are always fp32)."""
    import torch

    return torch.rand(shape, generator=_generator(seed, name, device), device=device, dtype=torch.float32)
