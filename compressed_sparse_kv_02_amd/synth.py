"""Seeded synthetic inputs for the compressed-attention layer.

This module only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic, so both the GPU path (tests,
bench) and the CPU oracle may consume what it produces.

Every tensor is drawn from its own stream,
``np.random.Generator(PCG64(SeedSequence([seed, crc32(name)])))``, as
float32, then rounded to bfloat16 (round to nearest even) when the workload
is bf16. The arrays returned are float32 whose values are exactly
representable in the storage type, so the GPU copy and the oracle see
identical numbers.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, Optional

import numpy as np


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, zlib.crc32(name.encode())])))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even); return float32."""
    out = np.array(x, dtype=np.float32, copy=True)
    u = out.view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    lsb += 0x7FFF
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return out


def normal(seed: int, name: str, shape, std: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    x = (_rng(seed, name).standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    return to_bf16_values(x) if dtype == "bf16" else x


def uniform(seed: int, name: str, shape, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """Uniform fp32 values (head weights and the like are always fp32)."""
    return _rng(seed, name).uniform(lo, hi, size=shape).astype(np.float32)


def low_rank_queries(seed: int, name: str, T: int, H: int, D: int, rank: int, dtype: str = "bf16") -> np.ndarray:
    """Indexer queries built from a shared latent: c [T, r] times W [r, H*D], scaled by 1/sqrt(r).

    The product is an input recipe (the shared-latent projection sits outside
    the layer kernels), computed here in float32 and rounded to the storage type.
    """
    c = _rng(seed, name + ".latent").standard_normal(size=(T, rank), dtype=np.float32)
    W = _rng(seed, name + ".proj").standard_normal(size=(rank, H * D), dtype=np.float32)
    q = (c @ W) * np.float32(1.0 / np.sqrt(rank))
    q = q.reshape(T, H, D).astype(np.float32)
    return to_bf16_values(q) if dtype == "bf16" else q


@dataclasses.dataclass
class LayerShape:
    """Shape of one compressed-attention layer call (one sequence batch)."""

    kind: str  # "csa" or "hca"
    batch: int
    T: int  # new tokens in this call (queries and raw rows)
    pos0: int  # absolute position of the first new token
    d: int  # KV / head dim
    rope_dims: int
    H: int  # query heads
    m: int  # compression ratio
    w: int  # sliding window
    k: int = 0  # top-k (CSA)
    HI: int = 0  # indexer heads (CSA)
    dI: int = 0  # indexer dim (CSA)
    qi_rank: int = 0  # 0: indexer queries drawn directly; else low-rank recipe
    bias_std: float = 1.0
    dtype: str = "bf16"
    seed: int = 0
    cached: int = 0  # compressed entries already in the cache before this call


def csa_compress_inputs(s: LayerShape, prefix: str = "") -> Dict[str, np.ndarray]:
    """Streams for the overlapped compressor: KV streams (dim d) and indexer-key streams (dim dI)."""
    B, T, d, m = s.batch, s.T, s.d, s.m
    out = {}
    for tag, c in (("kv", d), ("ik", s.dI)):
        for nm in ("Ca", "Cb", "Za", "Zb"):
            out[f"{tag}.{nm}"] = normal(s.seed, prefix + f"{tag}.{nm}", (B, T, c), dtype=s.dtype)
        out[f"{tag}.B"] = normal(s.seed, prefix + f"{tag}.B", (2 * m, c), std=s.bias_std, dtype=s.dtype)
        if s.pos0 > 0:
            out[f"{tag}.prevCb"] = normal(s.seed, prefix + f"{tag}.prevCb", (B, m, c), dtype=s.dtype)
            out[f"{tag}.prevZb"] = normal(s.seed, prefix + f"{tag}.prevZb", (B, m, c), dtype=s.dtype)
    return out


def hca_compress_inputs(s: LayerShape, prefix: str = "") -> Dict[str, np.ndarray]:
    B, T, d, m = s.batch, s.T, s.d, s.m
    return {
        "C": normal(s.seed, prefix + "hca.C", (B, T, d), dtype=s.dtype),
        "Z": normal(s.seed, prefix + "hca.Z", (B, T, d), dtype=s.dtype),
        "B": normal(s.seed, prefix + "hca.B", (m, d), std=s.bias_std, dtype=s.dtype),
    }


def attention_inputs(s: LayerShape, prefix: str = "") -> Dict[str, np.ndarray]:
    """Queries, raw window rows (positions pos0-w+1 .. pos0+T-1, clipped at 0), sinks, indexer queries."""
    B, T, d = s.batch, s.T, s.d
    win_pos0 = max(0, s.pos0 - s.w + 1)
    W = s.pos0 + T - win_pos0
    out = {
        "q": normal(s.seed, prefix + "q", (B, T, s.H, d), dtype=s.dtype),
        "win_raw": normal(s.seed, prefix + "win_raw", (B, W, d), dtype=s.dtype),
        "sink": normal(s.seed, prefix + "sink", (s.H,), dtype="f32"),
        "win_pos0": np.array(win_pos0, dtype=np.int64),
    }
    if s.kind == "csa":
        if s.qi_rank:
            q = np.stack([low_rank_queries(s.seed, prefix + f"qI{b}", T, s.HI, s.dI, s.qi_rank, s.dtype) for b in range(B)])
        else:
            q = normal(s.seed, prefix + "qI", (B, T, s.HI, s.dI), dtype=s.dtype)
        out["qI"] = q
        out["wI"] = uniform(s.seed, prefix + "wI", (B, T, s.HI))
    return out


def cache_inputs(s: LayerShape, n_entries: int, prefix: str = "") -> Dict[str, np.ndarray]:
    """A stored compressed cache (values as stored: N(0,1)), plus indexer keys for CSA."""
    out = {"kv": normal(s.seed, prefix + "cache.kv", (s.batch, n_entries, s.d), dtype=s.dtype)}
    if s.kind == "csa":
        out["ik"] = normal(s.seed, prefix + "cache.ik", (s.batch, n_entries, s.dI), dtype=s.dtype)
    return out


def normal_device(seed: int, name: str, shape, std: float = 1.0, dtype: str = "bf16", device="cuda"):
    """Large seeded N(0, std^2) tensors drawn on the GPU with torch's Philox generator.

    Used for the full-size workloads, whose inputs are too large to draw on the
    host; tests copy the rows they check back to the host for the oracle.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + zlib.crc32(name.encode())) & 0x7FFFFFFFFFFFFFFF)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def uniform_device(seed: int, name: str, shape, device="cuda"):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + zlib.crc32(name.encode())) & 0x7FFFFFFFFFFFFFFF)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def sample_rows(seed: int, T: int, n: int, must: Optional[list] = None) -> np.ndarray:
    """A seeded, sorted sample of query rows that always includes the listed rows."""
    must = [r for r in (must or []) if 0 <= r < T]
    rest = _rng(seed, "sample_rows").choice(T, size=min(T, n), replace=False)
    return np.unique(np.concatenate([np.array(must, dtype=np.int64), rest.astype(np.int64)]))
