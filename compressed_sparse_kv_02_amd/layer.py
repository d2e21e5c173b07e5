"""One compressed-attention layer call, composed from the C-ABI entry points.

A call appends T new tokens at absolute positions pos0 .. pos0+T-1 to a
sequence batch whose caches already hold `n_cached` compressed entries and
the last w-1 prepared window rows ("Paper Breakdown: DeepSeek-V4", §2.3.1
and §2.3.2; "Inside DeepSeek V4", "Local window"). Prefill from scratch is
n_cached = 0, pos0 = 0; chunked prefill appends a chunk to a long cache;
decode is T = 1 with the split-K attention entry point.

CSA layer, in order:
  1. csa_compress  KV streams -> new compressed entries (RMSNorm + RoPE),
                   appended in place to the KV cache;
  2. csa_compress  indexer-key streams -> new indexer keys, appended;
  3. hca_compress  (m' = 1) raw rows of the new tokens -> window rows;
  4. indexer_scores + topk_select (the two halves of indexer_topk, kept
                   apart so the scoring kernel can be timed on its own; the
                   scorer's block maxima let long rows skip a score pass);
  5. compressed_attn_prefill / _decode (CSA mode).
HCA layer: hca_compress (m') -> append, window rows, attention (HCA mode).

Inputs are drawn on the GPU by the seeded generator in `synth`; nothing
here computes any part of the layer outside the library.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

from . import binding as B
from .synth import normal_device, uniform_device


@dataclasses.dataclass
class LayerCall:
    kind: str          # "csa" | "hca"
    batch: int
    T: int             # new tokens
    pos0: int          # absolute position of the first new token
    n_cached: int      # compressed entries already cached
    d: int = 512
    rope_dims: int = 64
    H: int = 64
    m: int = 4
    w: int = 128
    k: int = 1024
    HI: int = 64
    dI: int = 128
    qi_rank: int = 0   # >0: indexer queries from a shared rank-r latent
    bias_std: float = 1.0
    dtype: str = "bf16"
    seed: int = 0
    name: str = "layer"
    decode: bool = False
    n_splits: int = 0

    @property
    def n_new(self) -> int:
        return self.T // self.m

    @property
    def N(self) -> int:
        return self.n_cached + self.n_new

    @property
    def win_cached(self) -> int:
        return min(self.w - 1, self.pos0)

    @property
    def win_pos0(self) -> int:
        return self.pos0 - self.win_cached

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


def make_inputs(L: LayerCall, device="cuda") -> Dict[str, torch.Tensor]:
    """Seeded device inputs and cache/output buffers for one layer call."""
    g = lambda nm, shape, std=1.0: normal_device(L.seed, f"{L.name}.{nm}", shape, std, L.dtype, device)
    Bt, T, d, m = L.batch, L.T, L.d, L.m
    t: Dict[str, torch.Tensor] = {}
    t["q"] = g("q", (Bt, T, L.H, d))
    t["sink"] = normal_device(L.seed, f"{L.name}.sink", (L.H,), 1.0, "f32", device)
    t["win_raw"] = g("win_raw", (Bt, T, d))
    win = torch.empty(Bt, L.win_cached + T, d, dtype=L.torch_dtype, device=device)
    if L.win_cached:
        win[:, :L.win_cached] = g("win_cached", (Bt, L.win_cached, d))
    t["win"] = win
    streams = [("kv", d)] + ([("ik", L.dI)] if L.kind == "csa" else [])
    for tag, c in streams:
        cache = torch.empty(Bt, L.N, c, dtype=L.torch_dtype, device=device)
        if L.n_cached:
            cache[:, :L.n_cached] = g(f"cache.{tag}", (Bt, L.n_cached, c))
        t[f"cache.{tag}"] = cache
        if L.n_new:
            if L.kind == "csa":
                for nm in ("Ca", "Cb", "Za", "Zb"):
                    t[f"{tag}.{nm}"] = g(f"{tag}.{nm}", (Bt, T, c))
                t[f"{tag}.B"] = g(f"{tag}.B", (2 * m, c), L.bias_std)
                if L.pos0 > 0:
                    t[f"{tag}.prevCb"] = g(f"{tag}.prevCb", (Bt, m, c))
                    t[f"{tag}.prevZb"] = g(f"{tag}.prevZb", (Bt, m, c))
            else:
                t[f"{tag}.C"] = g(f"{tag}.C", (Bt, T, c))
                t[f"{tag}.Z"] = g(f"{tag}.Z", (Bt, T, c))
                t[f"{tag}.B"] = g(f"{tag}.B", (m, c), L.bias_std)
    if L.kind == "csa":
        if L.qi_rank:
            lat = normal_device(L.seed, f"{L.name}.qI.latent", (Bt * T, L.qi_rank), 1.0, "f32", device)
            proj = normal_device(L.seed, f"{L.name}.qI.proj", (L.qi_rank, L.HI * L.dI), 1.0, "f32", device)
            qI = (lat @ proj) * (1.0 / L.qi_rank ** 0.5)
            t["qI"] = qI.reshape(Bt, T, L.HI, L.dI).to(L.torch_dtype).contiguous()
        else:
            t["qI"] = g("qI", (Bt, T, L.HI, L.dI))
        t["wI"] = uniform_device(L.seed, f"{L.name}.wI", (Bt, T, L.HI), device)
        t["idx"] = torch.empty(Bt, T, L.k, dtype=torch.int32, device=device)
        t["ws.scores"] = torch.empty(Bt, T, B.score_ld(L.N), dtype=torch.float32, device=device)
        if L.dtype == "bf16":  # block maxima beside the scores, for the selection of long rows
            t["ws.bm"] = torch.empty(Bt, T, B.block_max_ld(L.N), dtype=torch.int32, device=device)
        nsel = B.topk_workspace_bytes(Bt, T, L.N, L.k)
        if nsel:
            t["ws.topk"] = torch.empty(nsel, dtype=torch.uint8, device=device)
    t["out"] = torch.empty(Bt, T, L.H, d, dtype=L.torch_dtype, device=device)
    t["lse"] = torch.empty(Bt, T, L.H, dtype=torch.float32, device=device)
    if L.decode:
        t["ws.dec"] = torch.empty(max(16, B.decode_workspace_bytes(Bt, T, L.H, d, L.n_splits)),
                                  dtype=torch.uint8, device=device)
    return t


def compress_step(L: LayerCall, t: Dict[str, torch.Tensor]) -> None:
    """Steps 1-3: append new compressed entries (and indexer keys) and prepare window rows."""
    entries_step(L, t)
    window_step(L, t)


def entries_step(L: LayerCall, t: Dict[str, torch.Tensor]) -> None:
    """Steps 1-2: append the entries (and CSA indexer keys) of the blocks the call completes."""
    if L.n_new:
        if L.kind == "csa":
            B.csa_compress(t["kv.Ca"], t["kv.Cb"], t["kv.Za"], t["kv.Zb"], t["kv.B"], L.m, L.pos0,
                           t.get("kv.prevCb"), t.get("kv.prevZb"), apply_norm=True,
                           rope_dims=L.rope_dims, out=t["cache.kv"], out_row0=L.n_cached)
            B.csa_compress(t["ik.Ca"], t["ik.Cb"], t["ik.Za"], t["ik.Zb"], t["ik.B"], L.m, L.pos0,
                           t.get("ik.prevCb"), t.get("ik.prevZb"), apply_norm=False, rope_dims=0,
                           out=t["cache.ik"], out_row0=L.n_cached)
        else:
            B.hca_compress(t["kv.C"], t["kv.Z"], t["kv.B"], L.m, L.pos0, apply_norm=True,
                           rope_dims=L.rope_dims, out=t["cache.kv"], out_row0=L.n_cached)


def window_step(L: LayerCall, t: Dict[str, torch.Tensor]) -> None:
    """Step 3: prepare the call's window rows (RMSNorm + RoPE of the raw rows)."""
    B.hca_compress(t["win_raw"], None, None, 1, L.pos0, apply_norm=True, rope_dims=L.rope_dims,
                   out=t["win"], out_row0=L.win_cached)


def score_step(L: LayerCall, t: Dict[str, torch.Tensor]) -> None:
    """Step 4a (CSA only): lightning-indexer scores of every query over the whole cache."""
    if L.kind == "csa":
        B.indexer_scores(t["qI"], t["wI"], t["cache.ik"], L.pos0, L.m, scores=t["ws.scores"],
                         block_max=t.get("ws.bm"))


def topk_step(L: LayerCall, t: Dict[str, torch.Tensor]) -> None:
    """Step 4b (CSA only): per-query top-k of the scores (indexer_topk's second half)."""
    if L.kind == "csa":
        B.topk_select(t["ws.scores"], L.N, L.pos0, L.m, L.k, out=t["idx"], workspace=t.get("ws.topk"),
                      block_max=t.get("ws.bm"))


def select_step(L: LayerCall, t: Dict[str, torch.Tensor]) -> None:
    score_step(L, t)
    topk_step(L, t)


def attend_step(L: LayerCall, t: Dict[str, torch.Tensor]) -> None:
    mode = B.CSA if L.kind == "csa" else B.HCA
    kw = dict(apply_q_norm=True, rope_dims=L.rope_dims, rope_on_output=True, out=t["out"], lse=t["lse"])
    idx = t.get("idx") if L.kind == "csa" else None
    if L.decode:
        B.compressed_attn_decode(mode, t["q"], t["cache.kv"], idx, t["win"], L.win_pos0, t["sink"], L.pos0,
                                 L.m, L.w, k=L.k, n_splits=L.n_splits, workspace=t["ws.dec"], **kw)
    else:
        B.compressed_attn_prefill(mode, t["q"], t["cache.kv"], idx, t["win"], L.win_pos0, t["sink"],
                                  L.pos0, L.m, L.w, k=L.k, **kw)


def run_layer(L: LayerCall, t: Dict[str, torch.Tensor]) -> torch.Tensor:
    """The whole hot path of one layer call; returns the attention output."""
    compress_step(L, t)
    select_step(L, t)
    attend_step(L, t)
    return t["out"]


# --------------------------------------------------------------------------- streaming decode

class DecodeStream:
    """Token-by-token decode of one layer whose caches grow as tokens arrive.

    A compressed entry exists once its block is complete ("Paper Breakdown:
    DeepSeek-V4", §2.3.1 and §2.3.2): CSA entry i pools the a-rows of block i
    and the b-rows of block i-1, HCA entry i the m' rows of block i. The raw
    rows of the producer (C^a, C^b, Z^a, Z^b per stream for CSA; C, Z for HCA)
    go into rings that the producer writes directly (`slot`):

      * CSA: [2, batch, m, c] -- block i in half i % 2, so the completed block
        and the b-rows of the block before it are each one contiguous
        [batch, m, c] argument of csa_compress;
      * HCA: [batch, m', c] -- the block being filled;
      * window: a ring of w prepared rows, position p in row p mod w, read by
        the attention entry points with win_pos0 = 0.

    `step(t, ...)` prepares token t's window row in place, appends a cache
    entry (KV, and indexer key for CSA) when t completes a block, then runs the
    indexer, top-k and split-K attention against the caches. The caches are
    allocated for `capacity` entries and passed whole: the kernels read only
    entries visible at t, i.e. complete blocks, so rows not yet written are
    never read. All arithmetic is the library's; this class only keeps state.
    """

    def __init__(self, L: LayerCall, capacity: int, device="cuda"):
        self.L = L
        self.capacity = capacity
        td = L.torch_dtype
        Bt, d, m = L.batch, L.d, L.m
        self.streams = [("kv", d)] + ([("ik", L.dI)] if L.kind == "csa" else [])
        self.ring: Dict[str, torch.Tensor] = {}
        self.cache: Dict[str, torch.Tensor] = {}
        for tag, c in self.streams:
            names = ("Ca", "Cb", "Za", "Zb") if L.kind == "csa" else ("C", "Z")
            for nm in names:
                shape = (2, Bt, m, c) if L.kind == "csa" else (Bt, m, c)
                self.ring[f"{tag}.{nm}"] = torch.zeros(shape, dtype=td, device=device)
            self.cache[tag] = torch.zeros(Bt, capacity, c, dtype=td, device=device)
        self.win = torch.zeros(Bt, L.w, d, dtype=td, device=device)
        self.out = torch.empty(Bt, 1, L.H, d, dtype=td, device=device)
        self.lse = torch.empty(Bt, 1, L.H, dtype=torch.float32, device=device)
        self.ws_dec = torch.empty(max(16, B.decode_workspace_bytes(Bt, 1, L.H, d, L.n_splits)),
                                  dtype=torch.uint8, device=device)
        if L.kind == "csa":
            self.idx = torch.empty(Bt, 1, L.k, dtype=torch.int32, device=device)
            self.scores = torch.empty(Bt, 1, B.score_ld(capacity), dtype=torch.float32, device=device)
            self.bm = (torch.empty(Bt, 1, B.block_max_ld(capacity), dtype=torch.int32, device=device)
                       if L.dtype == "bf16" else None)
            nsel = B.topk_workspace_bytes(Bt, 1, capacity, L.k)
            self.ws_topk = torch.empty(nsel, dtype=torch.uint8, device=device) if nsel else None
        self.n_entries = 0

    def slot(self, name: str, t: int) -> torch.Tensor:
        """[batch, c] view where the producer writes raw row `name` (e.g. "kv.Ca") of token t."""
        m = self.L.m
        if self.L.kind == "csa":
            return self.ring[name][(t // m) % 2, :, t % m]
        return self.ring[name][:, t % m]

    def _compress(self, i: int, biases: Dict[str, torch.Tensor]) -> None:
        """Cache entry i from the ring (block i complete)."""
        L, m = self.L, self.L.m
        if i >= self.capacity:
            raise ValueError("DecodeStream capacity exceeded")
        for tag, _ in self.streams:
            r = lambda nm, h: self.ring[f"{tag}.{nm}"][h]
            if L.kind == "csa":
                cur, prev = i % 2, (i - 1) % 2
                pb = (r("Cb", prev), r("Zb", prev)) if i > 0 else (None, None)
                kv = tag == "kv"
                B.csa_compress(r("Ca", cur), r("Cb", cur), r("Za", cur), r("Zb", cur), biases[f"{tag}.B"], m,
                               m * i, pb[0], pb[1], apply_norm=kv, rope_dims=L.rope_dims if kv else 0,
                               out=self.cache[tag], out_row0=i)
            else:
                B.hca_compress(self.ring["kv.C"], self.ring["kv.Z"], biases["kv.B"], m, m * i, apply_norm=True,
                               rope_dims=L.rope_dims, out=self.cache["kv"], out_row0=i)
        self.n_entries = i + 1

    def step(self, t: int, q, win_raw, sink, biases: Dict[str, torch.Tensor], qI=None, wI=None) -> torch.Tensor:
        """Decode token t (its raw rows already in their slots); returns its attention output [batch, 1, H, d]."""
        L = self.L
        B.hca_compress(win_raw, None, None, 1, t, apply_norm=True, rope_dims=L.rope_dims, out=self.win,
                       out_row0=t % L.w)
        if (t + 1) % L.m == 0:
            self._compress((t + 1) // L.m - 1, biases)
        mode = B.CSA if L.kind == "csa" else B.HCA
        idx = None
        if L.kind == "csa":
            B.indexer_scores(qI, wI, self.cache["ik"], t, L.m, scores=self.scores, block_max=self.bm)
            B.topk_select(self.scores, self.capacity, t, L.m, L.k, out=self.idx, workspace=self.ws_topk,
                          block_max=self.bm)
            idx = self.idx
        return B.compressed_attn_decode(mode, q, self.cache["kv"], idx, self.win, 0, sink, t, L.m, L.w, k=L.k,
                                        apply_q_norm=True, rope_dims=L.rope_dims, rope_on_output=True,
                                        n_splits=L.n_splits, workspace=self.ws_dec, out=self.out, lse=self.lse)


# --------------------------------------------------------------------------- workloads

def tiny_csa(dtype="f32", seed=0) -> LayerCall:
    """Tiny CSA layer: T 512, d 64 (RoPE 16), 4 heads, indexer 2 x 32, k 16, window 16."""
    return LayerCall("csa", 1, 512, 0, 0, d=64, rope_dims=16, H=4, m=4, w=16, k=16, HI=2, dI=32,
                     dtype=dtype, seed=seed, name="tiny")


def hca_prefill_16k(seed=3) -> LayerCall:
    """HCA prefill: T 16384, m' 128, 32 heads x 512 (RoPE 64), window 128, bias std 0.1."""
    return LayerCall("hca", 1, 16384, 0, 0, d=512, rope_dims=64, H=32, m=128, w=128, bias_std=0.1,
                     seed=seed, name="hca16k")


def csa_prefill_64k(seed=1) -> LayerCall:
    """CSA prefill: T 65536, m 4, 64 heads x 512, indexer 64 x 128 (rank-256 queries), k 1024."""
    return LayerCall("csa", 1, 65536, 0, 0, d=512, rope_dims=64, H=64, m=4, w=128, k=1024, HI=64,
                     dI=128, qi_rank=256, seed=seed, name="csa64k")


def decode_1m(seed=4, n_splits=0):
    """Decode at 1M context, batch 8: one CSA layer (262144 entries, k 1024) + one HCA layer (8192)."""
    t = 1 << 20
    return [LayerCall("csa", 8, 1, t, t // 4, m=4, seed=seed, name="dec.csa", decode=True, n_splits=n_splits),
            LayerCall("hca", 8, 1, t, t // 128, m=128, seed=seed, name="dec.hca", decode=True,
                      n_splits=n_splits)]


def chunked_prefill_512k(seed=2):
    """4-layer CSA/HCA/CSA/HCA stack: a 4096-token chunk on a 524288-token context, batch 2."""
    p = 524288
    out = []
    for i, kind in enumerate(("csa", "hca", "csa", "hca")):
        m = 4 if kind == "csa" else 128
        out.append(LayerCall(kind, 2, 4096, p, p // m, m=m, seed=seed, name=f"chunk.l{i}"))
    return out
