"""The allocation-free decode entry point against compressed_attn_decode, through the C ABI:
two calls in a row on the same GPU (the second smaller, so it reuses the static scratch the
first one filled), each bit-identical to the workspace entry point at the same split count."""
import numpy as np
import pytest
import torch

from compressed_sparse_kv_02_amd import binding as B
from compressed_sparse_kv_02_amd.synth import normal_device, uniform_device

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(kind, bt, N, H, seed):
    m, k, w, d = (4, 256, 128, 512) if kind == "csa" else (128, 0, 128, 512)
    pos0 = N * m + 3
    g = lambda nm, sh: normal_device(seed, f"na.{nm}", sh, 1.0, "bf16", DEV)
    q = g("q", (bt, 1, H, d))
    kv = g("kv", (bt, N, d))
    win = g("win", (bt, w, d))
    sink = normal_device(seed, "na.sink", (H,), 1.0, "f32", DEV)
    idx = None
    if kind == "csa":
        r = np.random.default_rng(seed)
        V = min(N, (pos0 + 1) // m)
        sel = np.stack([np.sort(r.choice(V, k, replace=False)) for _ in range(bt)]).astype(np.int32)
        idx = torch.from_numpy(sel).to(DEV).reshape(bt, 1, k)
    mode = B.CSA if kind == "csa" else B.HCA
    return mode, q, kv, idx, win, pos0 - w + 1, sink, pos0, m, w, k


@pytest.mark.parametrize("order", ["large_then_small"])
def test_decode_noalloc_matches_workspace_entry_point(order):
    print("decode noalloc: HCA batch 8 x 8192 entries (32 splits), then CSA batch 2 x 4096 entries", flush=True)
    cases = [("hca", 8, 8192, 64, 32, 101), ("csa", 2, 4096, 64, 0, 102)]
    for kind, bt, N, H, ns, seed in cases:
        mode, q, kv, idx, win, wp0, sink, pos0, m, w, k = _case(kind, bt, N, H, seed)
        kw = dict(k=k, rope_dims=64, n_splits=ns)
        ref, ref_lse = B.compressed_attn_decode(mode, q, kv, idx, win, wp0, sink, pos0, m, w, return_lse=True, **kw)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((bt, 1, H), float("nan"), dtype=torch.float32, device=DEV)
        B.compressed_attn_decode_noalloc(mode, q, kv, idx, win, wp0, sink, pos0, m, w, out=out, lse=lse, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (kind, (out.float() - ref.float()).abs().max().item())
        assert torch.equal(lse, ref_lse), kind
    # an explicit split count whose partials exceed the scratch is refused, with nothing launched
    mode, q, kv, idx, win, wp0, sink, pos0, m, w, k = _case("hca", 8, 8192, 64, 101)
    out = torch.empty_like(q)
    with pytest.raises(B.CskvError, match="workspace"):
        B.compressed_attn_decode_noalloc(mode, q, kv, idx, win, wp0, sink, pos0, m, w, out=out, n_splits=256,
                                         rope_dims=64)
