"""ctypes binding of libcskv.so (include/cskv.h).

Argument marshalling only: every step of the layer runs in the library's
HIP kernels. Tensors must already be on the GPU and contiguous; outputs and
workspaces are allocated with torch (device memory and streams are the only
things torch provides). There is no CPU fallback: a missing library or a CPU
tensor raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcskv.so")

BF16, F32, FP8, FP4, MXFP4, MXFP8 = 0, 1, 2, 3, 4, 5
CSA, HCA = 0, 1
EXPORTS = ("cskv_version", "cskv_status_string", "csa_compress", "hca_compress",
           "cskv_indexer_workspace_size", "indexer_topk", "indexer_scores", "topk_select",
           "cskv_topk_workspace_size", "cskv_quantize_fp8", "indexer_scores_fp8", "indexer_topk_fp8",
           "cskv_quantize_fp4", "indexer_scores_fp4", "indexer_topk_fp4",
           "cskv_quantize_mxfp4", "indexer_scores_mxfp4", "indexer_topk_mxfp4",
           "cskv_quantize_mxfp8", "indexer_scores_mxfp8", "indexer_topk_mxfp8",
           "cskv_quantize_kv_fp8", "compressed_attn_prefill_kv8", "cskv_prefill_kv8_workspace_size",
           "compressed_attn_decode_kv8",
           "compressed_attn_prefill",
           "cskv_decode_workspace_size", "compressed_attn_decode", "compressed_attn_decode_noalloc",
           "cskv_lowrank_proj", "cskv_grouped_out_proj")

_lib = None

_P, _I, _L, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "cskv_version": (_I, []),
    "cskv_status_string": (ctypes.c_char_p, [_I]),
    "csa_compress": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _L, _I, _I, _L, _I, _P, _F, _I, _F, _P, _L, _I, _P]),
    "hca_compress": (_I, [_P, _P, _P, _I, _L, _I, _I, _L, _I, _P, _F, _I, _F, _P, _L, _I, _P]),
    "cskv_indexer_workspace_size": (_Z, [_I, _L, _L, _I, _I, _I]),
    "indexer_topk": (_I, [_P, _P, _P, _I, _L, _L, _I, _I, _L, _I, _I, _P, _P, _Z, _I, _P]),
    "indexer_scores": (_I, [_P, _P, _P, _I, _L, _L, _I, _I, _L, _I, _P, _L, _P, _L, _I, _P]),
    "topk_select": (_I, [_P, _L, _P, _L, _I, _L, _L, _L, _I, _I, _P, _P, _Z, _P]),
    "cskv_topk_workspace_size": (_Z, [_I, _L, _L, _I]),
    "cskv_quantize_fp8": (_I, [_P, _L, _I, _I, _P, _P, _P]),
    "indexer_scores_fp8": (_I, [_P, _P, _P, _P, _P, _I, _L, _L, _I, _I, _L, _I, _P, _L, _P]),
    "indexer_topk_fp8": (_I, [_P, _P, _P, _P, _P, _I, _L, _L, _I, _I, _L, _I, _I, _P, _P, _Z, _P]),
    "cskv_quantize_fp4": (_I, [_P, _L, _I, _I, _P, _P, _P]),
    "indexer_scores_fp4": (_I, [_P, _P, _P, _P, _P, _I, _L, _L, _I, _I, _L, _I, _P, _L, _P]),
    "indexer_topk_fp4": (_I, [_P, _P, _P, _P, _P, _I, _L, _L, _I, _I, _L, _I, _I, _P, _P, _Z, _P]),
    "cskv_quantize_mxfp4": (_I, [_P, _L, _I, _I, _P, _P, _P]),
    "indexer_scores_mxfp4": (_I, [_P, _P, _P, _P, _P, _I, _L, _L, _I, _I, _L, _I, _P, _L, _P]),
    "indexer_topk_mxfp4": (_I, [_P, _P, _P, _P, _P, _I, _L, _L, _I, _I, _L, _I, _I, _P, _P, _Z, _P]),
    "cskv_quantize_mxfp8": (_I, [_P, _L, _I, _I, _P, _P, _P]),
    "indexer_scores_mxfp8": (_I, [_P, _P, _P, _P, _P, _I, _L, _L, _I, _I, _L, _I, _P, _L, _P]),
    "indexer_topk_mxfp8": (_I, [_P, _P, _P, _P, _P, _I, _L, _L, _I, _I, _L, _I, _I, _P, _P, _Z, _P]),
    "cskv_quantize_kv_fp8": (_I, [_P, _I, _L, _I, _I, _I, _P, _P, _L, _P]),
    "compressed_attn_prefill_kv8": (_I, [_I, _P, _P, _P, _P, _P, _L, _L, _P, _I, _L, _L, _L, _I, _I, _I, _I, _I,
                                         _I, _P, _F, _I, _F, _F, _I, _P, _Z, _P, _P, _P]),
    "cskv_prefill_kv8_workspace_size": (_Z, [_I, _I, _L, _I]),
    "compressed_attn_decode_kv8": (_I, [_I, _P, _P, _P, _P, _P, _L, _L, _P, _I, _L, _L, _L, _I, _I, _I, _I, _I,
                                        _I, _P, _F, _I, _F, _F, _I, _I, _P, _Z, _P, _P, _P]),
    "compressed_attn_prefill": (_I, [_I, _P, _P, _P, _P, _L, _L, _P, _I, _L, _L, _L, _I, _I, _I, _I, _I,
                                     _I, _P, _F, _I, _F, _F, _I, _P, _P, _I, _P]),
    "cskv_decode_workspace_size": (_Z, [_I, _L, _I, _I, _I]),
    "compressed_attn_decode_noalloc": (_I, [_I, _P, _P, _P, _P, _L, _L, _P, _I, _L, _L, _L, _I, _I, _I, _I, _I,
                                            _I, _P, _F, _I, _F, _F, _I, _I, _P, _P, _I, _P]),
    "cskv_lowrank_proj": (_I, [_P, _P, _P, _L, _L, _L, _I, _P]),
    "cskv_grouped_out_proj": (_I, [_P, _P, _P, _P, _P, _L, _I, _I, _I, _L, _L, _I, _P]),
    "compressed_attn_decode": (_I, [_I, _P, _P, _P, _P, _L, _L, _P, _I, _L, _L, _L, _I, _I, _I, _I, _I,
                                    _I, _P, _F, _I, _F, _F, _I, _I, _P, _Z, _P, _P, _I, _P]),
}


class CskvError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libcskv.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CskvError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().cskv_status_string(code).decode()


def _check(name: str, code: int) -> None:
    if code != 0:
        raise CskvError(f"{name} failed: {status_string(code)} ({code})")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise CskvError("tensor is not on the GPU (the layer has no CPU path)")
    if not t.is_contiguous():
        raise CskvError("tensor must be contiguous")
    return t.data_ptr()


def _need(cond: bool, msg: str) -> None:
    """Raise before any library call when a caller buffer cannot hold what the call writes."""
    if not cond:
        raise CskvError(msg)


def _check_append(name: str, out: torch.Tensor, batch: int, width: int, out_row0: int, n_new: int) -> None:
    """out [batch, cap, width]: rows out_row0 .. out_row0 + n_new - 1 of every sequence must exist."""
    _need(out.dim() == 3 and out.shape[0] == batch and out.shape[2] == width,
          f"{name}: out must be [batch={batch}, cap, {width}], got {tuple(out.shape)}")
    _need(0 <= out_row0 and out_row0 + n_new <= out.shape[1],
          f"{name}: rows {out_row0} .. {out_row0 + n_new - 1} do not fit a cache of {out.shape[1]} rows")


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise CskvError(f"unsupported dtype {t.dtype}")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def csa_compress(Ca, Cb, Za, Zb, B, m: int, pos0: int = 0, prev_Cb=None, prev_Zb=None,
                 apply_norm: bool = False, norm_w=None, eps: float = 1e-6, rope_dims: int = 0,
                 rope_base: float = 10000.0, out=None, out_row0: int = 0) -> torch.Tensor:
    """Overlapped 1/m compression of [batch, T, c] streams -> [batch, T // m, c].

    With `out` given as a [batch, cap, c] cache, the entries land in rows
    out_row0 .. out_row0 + T // m - 1 of each sequence (an in-place append).
    """
    batch, T, c = Ca.shape
    if out is None:
        out = torch.empty(batch, T // m, c, dtype=Ca.dtype, device=Ca.device)
    _need(out.dtype == Ca.dtype, "csa_compress: out must have the streams' dtype")
    _check_append("csa_compress", out, batch, c, out_row0, T // m if m > 0 else 0)
    _ptr(out)
    ptr = out.data_ptr() + out_row0 * c * out.element_size()
    _check("csa_compress", lib().csa_compress(
        _ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), _ptr(B), _ptr(prev_Cb), _ptr(prev_Zb), batch, T, c, m,
        pos0, int(apply_norm), _ptr(norm_w), eps, rope_dims, rope_base, ptr, out.shape[1], _dtype(Ca),
        _stream(Ca)))
    return out


def hca_compress(C, Z=None, B=None, m: int = 128, pos0: int = 0, apply_norm: bool = False,
                 norm_w=None, eps: float = 1e-6, rope_dims: int = 0, rope_base: float = 10000.0,
                 out=None, out_row0: int = 0) -> torch.Tensor:
    """Non-overlapped 1/m' compression of [batch, T, c] -> [batch, T // m', c] (m' = 1: window rows).

    `out` / `out_row0` append in place into a [batch, cap, c] buffer, as in csa_compress.
    """
    batch, T, c = C.shape
    if out is None:
        out = torch.empty(batch, T // m, c, dtype=C.dtype, device=C.device)
    _need(out.dtype == C.dtype, "hca_compress: out must have the stream's dtype")
    _check_append("hca_compress", out, batch, c, out_row0, T // m if m > 0 else 0)
    _ptr(out)
    ptr = out.data_ptr() + out_row0 * c * out.element_size()
    _check("hca_compress", lib().hca_compress(
        _ptr(C), _ptr(Z), _ptr(B), batch, T, c, m, pos0, int(apply_norm), _ptr(norm_w), eps,
        rope_dims, rope_base, ptr, out.shape[1], _dtype(C), _stream(C)))
    return out


def indexer_workspace_bytes(batch: int, Tq: int, N: int, HI: int, k: int, dtype: int) -> int:
    return int(lib().cskv_indexer_workspace_size(batch, Tq, N, HI, k, dtype))


def indexer_topk(qI, wI, KI, pos0: int, m: int, k: int, out=None, workspace=None) -> torch.Tensor:
    """Top-k compressed entries per query: [batch, Tq, k] int32, ascending, -1 padded."""
    batch, Tq, HI, dI = qI.shape
    N = KI.shape[1]
    dt = _dtype(qI)
    if out is None:
        out = torch.empty(batch, Tq, k, dtype=torch.int32, device=qI.device)
    _check_idx("indexer_topk", out, batch, Tq, k)
    need = indexer_workspace_bytes(batch, Tq, N, HI, k, dt)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=qI.device)
    _check("indexer_topk", lib().indexer_topk(
        _ptr(qI), _ptr(wI), _ptr(KI), batch, Tq, N, HI, dI, pos0, m, k, _ptr(out), _ptr(workspace),
        workspace.numel(), dt, _stream(qI)))
    return out


def _check_scores(name: str, scores: torch.Tensor, batch: int, Tq: int, N: int) -> None:
    _need(scores.dtype == torch.float32 and scores.dim() == 3 and tuple(scores.shape[:2]) == (batch, Tq)
          and scores.shape[2] >= N, f"{name}: scores must be fp32 [{batch}, {Tq}, >= {N}], got "
          f"{scores.dtype} {tuple(scores.shape)}")


def _check_idx(name: str, out: torch.Tensor, batch: int, Tq: int, k: int) -> None:
    _need(out.dtype == torch.int32 and tuple(out.shape) == (batch, Tq, k),
          f"{name}: out must be int32 [{batch}, {Tq}, {k}], got {out.dtype} {tuple(out.shape)}")


def score_ld(N: int) -> int:
    """Row stride used for score matrices: N rounded up to 64 entries."""
    return max(64, (N + 63) // 64 * 64)


def block_max_ld(N: int) -> int:
    """Row stride used for block-maximum matrices: ceil(N / 32) rounded up to 4 blocks."""
    return max(4, ((N + 31) // 32 + 3) // 4 * 4)


def _check_bm(name: str, bm: torch.Tensor, batch: int, Tq: int, N: int) -> None:
    _need(bm.dtype == torch.int32 and bm.dim() == 3 and tuple(bm.shape[:2]) == (batch, Tq)
          and bm.shape[2] >= (N + 31) // 32 and bm.is_contiguous(),
          f"{name}: block_max must be contiguous int32 [{batch}, {Tq}, >= {(N + 31) // 32}], got "
          f"{bm.dtype} {tuple(bm.shape)}")


def indexer_scores(qI, wI, KI, pos0: int, m: int, scores=None, block_max=None) -> torch.Tensor:
    """Lightning-indexer scores [batch, Tq, ld] fp32 (valid for s < V_t).

    `block_max` (optional, int32 [batch, Tq, >= ceil(N/32)] holding uint32 bit patterns) also
    receives each 32-entry block's largest order key, for topk_select.
    """
    batch, Tq, HI, dI = qI.shape
    N = KI.shape[1]
    if scores is None:
        scores = torch.empty(batch, Tq, score_ld(N), dtype=torch.float32, device=qI.device)
    _check_scores("indexer_scores", scores, batch, Tq, N)
    bm, bm_ld = None, 0
    if block_max is not None:
        _check_bm("indexer_scores", block_max, batch, Tq, N)
        bm, bm_ld = _ptr(block_max), block_max.shape[-1]
    _check("indexer_scores", lib().indexer_scores(
        _ptr(qI), _ptr(wI), _ptr(KI), batch, Tq, N, HI, dI, pos0, m, _ptr(scores), scores.shape[-1], bm,
        bm_ld, _dtype(qI), _stream(qI)))
    return scores


def topk_workspace_bytes(batch: int, Tq: int, N: int, k: int) -> int:
    return int(lib().cskv_topk_workspace_size(batch, Tq, N, k))


def topk_select(scores, N: int, pos0: int, m: int, k: int, out=None, workspace=None, block_max=None) -> torch.Tensor:
    """Top-k selection from a score matrix written by indexer_scores.

    `workspace` (optional, cskv_topk_workspace_size bytes) lets few long rows be
    selected with several workgroups per row; `block_max` (optional) are the
    block maxima indexer_scores wrote beside these scores. The result is the
    same with or without either.
    """
    batch, Tq, ld = scores.shape
    if out is None:
        out = torch.empty(batch, Tq, k, dtype=torch.int32, device=scores.device)
    _check_scores("topk_select", scores, batch, Tq, N)
    _check_idx("topk_select", out, batch, Tq, k)
    ws, nbytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
    bm, bm_ld = None, 0
    if block_max is not None:
        _check_bm("topk_select", block_max, batch, Tq, N)
        bm, bm_ld = _ptr(block_max), block_max.shape[-1]
    _check("topk_select", lib().topk_select(_ptr(scores), ld, bm, bm_ld, batch, Tq, N, pos0, m, k, _ptr(out), ws,
                                            nbytes, _stream(scores)))
    return out


_LOWP = {FP8: ("fp8", 1), FP4: ("fp4", 2), MXFP4: ("mxfp4", 2), MXFP8: ("mxfp8", 1)}  # name suffix, values per byte


def _quantize(x, fmt):
    suffix, per_byte = _LOWP[fmt]
    dim = x.shape[-1]
    rows = x.numel() // dim if dim else 0
    codes = torch.empty(*x.shape[:-1], dim // per_byte, dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    name = f"cskv_quantize_{suffix}"
    _check(name, getattr(lib(), name)(_ptr(x), rows, dim, _dtype(x), _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def quantize_fp8(x) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-row E4M3 codes (uint8, x's shape) and fp32 scales (x.shape[:-1]) of x (bf16 or fp32)."""
    return _quantize(x, FP8)


def quantize_fp4(x) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-row E2M1 codes, two per byte ([..., dim / 2] uint8), and fp32 scales of x (bf16 or fp32)."""
    return _quantize(x, FP4)


def _quantize_mx(x, fmt):
    suffix, per_byte = _LOWP[fmt]
    dim = x.shape[-1]
    rows = x.numel() // dim if dim else 0
    codes = torch.empty(*x.shape[:-1], dim // per_byte, dtype=torch.uint8, device=x.device)
    scales = torch.empty(*x.shape[:-1], dim // 32, dtype=torch.uint8, device=x.device)
    name = f"cskv_quantize_{suffix}"
    _check(name, getattr(lib(), name)(_ptr(x), rows, dim, _dtype(x), _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def quantize_mxfp4(x) -> Tuple[torch.Tensor, torch.Tensor]:
    """MX-FP4 rows of x (bf16 or fp32): E2M1 codes, two per byte ([..., dim / 2] uint8), and one
    E8M0 scale byte per 32 values ([..., dim / 32] uint8)."""
    return _quantize_mx(x, MXFP4)


def quantize_mxfp8(x) -> Tuple[torch.Tensor, torch.Tensor]:
    """MX-FP8 rows of x (bf16 or fp32): E4M3 codes ([..., dim] uint8) and one E8M0 scale byte per
    32 values ([..., dim / 32] uint8)."""
    return _quantize_mx(x, MXFP8)


def _scores_lowp(fmt, q_codes, q_scales, wI, k_codes, k_scales, pos0, m, scores):
    suffix, per_byte = _LOWP[fmt]
    batch, Tq, HI, db = q_codes.shape
    N = k_codes.shape[1]
    if scores is None:
        scores = torch.empty(batch, Tq, score_ld(N), dtype=torch.float32, device=q_codes.device)
    name = f"indexer_scores_{suffix}"
    _check_scores(name, scores, batch, Tq, N)
    _check(name, getattr(lib(), name)(
        _ptr(q_codes), _ptr(q_scales), _ptr(wI), _ptr(k_codes), _ptr(k_scales), batch, Tq, N, HI, db * per_byte,
        pos0, m, _ptr(scores), scores.shape[-1], _stream(q_codes)))
    return scores


def _topk_lowp(fmt, q_codes, q_scales, wI, k_codes, k_scales, pos0, m, k, out, workspace):
    suffix, per_byte = _LOWP[fmt]
    batch, Tq, HI, db = q_codes.shape
    N = k_codes.shape[1]
    if out is None:
        out = torch.empty(batch, Tq, k, dtype=torch.int32, device=q_codes.device)
    _check_idx(f"indexer_topk_{suffix}", out, batch, Tq, k)
    need = indexer_workspace_bytes(batch, Tq, N, HI, k, fmt)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_codes.device)
    name = f"indexer_topk_{suffix}"
    _check(name, getattr(lib(), name)(
        _ptr(q_codes), _ptr(q_scales), _ptr(wI), _ptr(k_codes), _ptr(k_scales), batch, Tq, N, HI, db * per_byte,
        pos0, m, k, _ptr(out), _ptr(workspace), workspace.numel(), _stream(q_codes)))
    return out


def indexer_scores_fp8(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int, scores=None) -> torch.Tensor:
    """Indexer scores on E4M3 rows: [batch, Tq, ld] fp32 (valid for s < V_t)."""
    return _scores_lowp(FP8, q_codes, q_scales, wI, k_codes, k_scales, pos0, m, scores)


def indexer_scores_fp4(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int, scores=None) -> torch.Tensor:
    """Indexer scores on E2M1 rows (two codes per byte): [batch, Tq, ld] fp32 (valid for s < V_t)."""
    return _scores_lowp(FP4, q_codes, q_scales, wI, k_codes, k_scales, pos0, m, scores)


def indexer_topk_fp8(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int, k: int, out=None,
                     workspace=None) -> torch.Tensor:
    """Top-k compressed entries per query from E4M3 rows: [batch, Tq, k] int32, ascending, -1 padded."""
    return _topk_lowp(FP8, q_codes, q_scales, wI, k_codes, k_scales, pos0, m, k, out, workspace)


def indexer_topk_fp4(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int, k: int, out=None,
                     workspace=None) -> torch.Tensor:
    """Top-k compressed entries per query from E2M1 rows: [batch, Tq, k] int32, ascending, -1 padded."""
    return _topk_lowp(FP4, q_codes, q_scales, wI, k_codes, k_scales, pos0, m, k, out, workspace)


def kv_fp8_row_bytes(d: int, rope_dims: int) -> int:
    return d - rope_dims + 2 * rope_dims


def quantize_kv_fp8(x, rope_dims: int, out=None, scales=None, out_row0: int = 0):
    """FP8 (non-RoPE dims) + BF16 (RoPE dims) storage of entries x [batch, n, d] (bf16 or fp32).

    Returns (rows [batch, cap, row bytes] uint8, scales [batch, cap] fp32); `out` / `scales` /
    `out_row0` append in place into a cache of capacity cap.
    """
    batch, n, d = x.shape
    rb = kv_fp8_row_bytes(d, rope_dims)
    if out is None:
        _need(scales is None, "quantize_kv_fp8: scales given without out")
        out = torch.empty(batch, n, rb, dtype=torch.uint8, device=x.device)
        scales = torch.empty(batch, n, dtype=torch.float32, device=x.device)
    _need(scales is not None, "quantize_kv_fp8: out given without scales")
    _need(out.dtype == torch.uint8 and scales.dtype == torch.float32, "quantize_kv_fp8: out uint8, scales fp32")
    _check_append("quantize_kv_fp8", out, batch, rb, out_row0, n)
    _need(scales.dim() == 2 and tuple(scales.shape) == (batch, out.shape[1]),
          f"quantize_kv_fp8: scales must be [{batch}, {out.shape[1]}], got {tuple(scales.shape)}")
    _ptr(out), _ptr(scales)
    cap = out.shape[1]
    _check("cskv_quantize_kv_fp8", lib().cskv_quantize_kv_fp8(
        _ptr(x), batch, n, d, rope_dims, _dtype(x), out.data_ptr() + out_row0 * rb,
        scales.data_ptr() + out_row0 * 4, cap, _stream(x)))
    return out, scales


def _attn_common(mode, q, kv, idx, win, win_pos0, sink, pos0, m, k, w, apply_q_norm, q_norm_w, eps,
                 rope_dims, rope_base, scale, rope_on_output, out, lse, return_lse, kv_scale=None):
    batch, Tq, H, d = q.shape
    N = kv.shape[1]
    W = win.shape[1]
    # the entries' row width and the per-entry scales bound every gathered row
    if kv_scale is None:
        _need(kv.dim() == 3 and kv.shape[2] == d and kv.dtype == q.dtype,
              f"attention: kv must be {q.dtype} [batch, N, {d}]")
    else:
        rb = kv_fp8_row_bytes(d, rope_dims)
        _need(kv.dim() == 3 and kv.shape[2] == rb and kv.dtype == torch.uint8,
              f"attention (FP8 cache): kv must be uint8 [batch, N, {rb}]")
        _need(kv_scale.dtype == torch.float32 and tuple(kv_scale.shape) == (batch, N),
              f"attention (FP8 cache): kv_scale must be fp32 [{batch}, {N}]")
    _need(sink is None or (sink.dtype == torch.float32 and sink.numel() == H), f"attention: sink must be fp32 [{H}]")
    _need(q_norm_w is None or (q_norm_w.dtype == torch.float32 and q_norm_w.numel() == d),
          f"attention: q_norm_w must be fp32 [{d}]")
    _need(win.dtype == q.dtype, "attention: win must have q's dtype")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty(batch, Tq, H, dtype=torch.float32, device=q.device)
    _need(out.shape == q.shape and out.dtype == q.dtype, f"attention: out must match q {tuple(q.shape)} {q.dtype}")
    _need(lse is None or (lse.dtype == torch.float32 and tuple(lse.shape) == (batch, Tq, H)),
          f"attention: lse must be fp32 [{batch}, {Tq}, {H}]")
    _need(kv.dim() == 3 and kv.shape[0] == batch and win.dim() == 3 and win.shape[0] == batch
          and win.shape[2] == d, "attention: kv [batch, N, .] and win [batch, W, d] expected")
    if mode == CSA:
        _need(idx is not None and idx.dim() == 3 and tuple(idx.shape[:2]) == (batch, Tq)
              and idx.dtype == torch.int32, f"attention (CSA): idx must be int32 [{batch}, {Tq}, k]")
        k = idx.shape[2]
    args = (mode, _ptr(q), _ptr(kv), _ptr(idx), _ptr(win), win_pos0, W, _ptr(sink), batch, Tq, N, pos0,
            m, k, w, H, d, int(apply_q_norm), _ptr(q_norm_w), eps, rope_dims, rope_base, scale,
            int(rope_on_output))
    return args, out, lse


def compressed_attn_prefill(mode: int, q, kv, idx, win, win_pos0: int, sink, pos0: int, m: int,
                            w: int, k: int = 0, apply_q_norm: bool = True, q_norm_w=None,
                            eps: float = 1e-6, rope_dims: int = 0, rope_base: float = 10000.0,
                            scale: float = 0.0, rope_on_output: bool = True, out=None, lse=None,
                            return_lse: bool = False, kv_scale=None, workspace=None):
    """CSA / HCA attention for a chunk of queries: out [batch, Tq, H, d] (and lse [batch, Tq, H]).

    With kv_scale, kv is an FP8 KV cache written by quantize_kv_fp8 ([batch, N, row bytes] uint8).
    HCA over such a cache widens the entries once into `workspace` (allocated here when None;
    an empty tensor selects the route that widens each gathered tile instead).
    """
    args, out, lse = _attn_common(mode, q, kv, idx, win, win_pos0, sink, pos0, m, k, w, apply_q_norm,
                                  q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output, out, lse,
                                  return_lse, kv_scale)
    if kv_scale is not None:  # FP8 KV storage: kv holds the stored entries (uint8 rows)
        batch, N = kv.shape[0], kv.shape[1]
        need = int(lib().cskv_prefill_kv8_workspace_size(mode, batch, N, q.shape[-1]))
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
        ws, ws_bytes = (None, 0) if workspace is None or workspace.numel() == 0 else (workspace, workspace.numel())
        _check("compressed_attn_prefill_kv8", lib().compressed_attn_prefill_kv8(
            *args[:3], _ptr(kv_scale), *args[3:], _ptr(ws), ws_bytes, _ptr(out), _ptr(lse), _stream(q)))
    else:
        _check("compressed_attn_prefill", lib().compressed_attn_prefill(
            *args, _ptr(out), _ptr(lse), _dtype(q), _stream(q)))
    return (out, lse) if return_lse else out


def decode_workspace_bytes(batch: int, Tq: int, H: int, d: int, n_splits: int) -> int:
    return int(lib().cskv_decode_workspace_size(batch, Tq, H, d, n_splits))


def compressed_attn_decode(mode: int, q, kv, idx, win, win_pos0: int, sink, pos0: int, m: int,
                           w: int, k: int = 0, apply_q_norm: bool = True, q_norm_w=None,
                           eps: float = 1e-6, rope_dims: int = 0, rope_base: float = 10000.0,
                           scale: float = 0.0, rope_on_output: bool = True, n_splits: int = 0,
                           workspace=None, out=None, lse=None, return_lse: bool = False, kv_scale=None):
    """Split-K attention of a few new tokens against a long cache (same result as prefill)."""
    args, out, lse = _attn_common(mode, q, kv, idx, win, win_pos0, sink, pos0, m, k, w, apply_q_norm,
                                  q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output, out, lse,
                                  return_lse, kv_scale)
    batch, Tq, H, d = q.shape
    need = decode_workspace_bytes(batch, Tq, H, d, n_splits)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if kv_scale is not None:
        _check("compressed_attn_decode_kv8", lib().compressed_attn_decode_kv8(
            *args[:3], _ptr(kv_scale), *args[3:], n_splits, _ptr(workspace), workspace.numel(), _ptr(out),
            _ptr(lse), _stream(q)))
    else:
        _check("compressed_attn_decode", lib().compressed_attn_decode(
            *args, n_splits, _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _dtype(q), _stream(q)))
    return (out, lse) if return_lse else out


NOALLOC_SCRATCH_BYTES = 64 << 20


def compressed_attn_decode_noalloc(mode: int, q, kv, idx, win, win_pos0: int, sink, pos0: int, m: int, w: int,
                                   out, lse=None, k: int = 0, apply_q_norm: bool = True, q_norm_w=None,
                                   eps: float = 1e-6, rope_dims: int = 0, rope_base: float = 10000.0,
                                   scale: float = 0.0, rope_on_output: bool = True, n_splits: int = 0):
    """compressed_attn_decode without a workspace: the split partials use the library's static
    per-GPU scratch (NOALLOC_SCRATCH_BYTES, held from the library's first use on a GPU to the end of
    the process), so the call allocates no device memory; `out` (and `lse`, if wanted) are the
    caller's. Calls that overlap on one GPU race on the shared scratch."""
    _need(out is not None, "compressed_attn_decode_noalloc: out must be given (the call allocates nothing)")
    args, out, lse = _attn_common(mode, q, kv, idx, win, win_pos0, sink, pos0, m, k, w, apply_q_norm,
                                  q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output, out, lse, False)
    _check("compressed_attn_decode_noalloc", lib().compressed_attn_decode_noalloc(
        *args, n_splits, _ptr(out), _ptr(lse), _dtype(q), _stream(q)))
    return out


def lowrank_proj(cq, W, out=None):
    """out [..., n_out] = cq [..., r] @ W [r, n_out] (bf16; the leading dims of cq are the tokens)."""
    r, n_out = W.shape
    T = cq.numel() // r
    if out is None:
        out = torch.empty(*cq.shape[:-1], n_out, dtype=cq.dtype, device=cq.device)
    _check("cskv_lowrank_proj", lib().cskv_lowrank_proj(_ptr(cq), _ptr(W), _ptr(out), T, r, n_out,
                                                        _dtype(cq), _stream(cq)))
    return out


def grouped_out_proj(o, Wg, Wo, mid=None, out=None, return_mid: bool = False):
    """Grouped output projection of attention outputs o [..., H, d] with Wg [G, (H/G) d, dg] and
    Wo [G dg, D] -> y [..., D] (and the bf16 intermediate mid [..., G, dg])."""
    H, d = o.shape[-2], o.shape[-1]
    G, _, dg = Wg.shape
    D = Wo.shape[1]
    T = o.numel() // (H * d)
    lead = o.shape[:-2]
    if mid is None:
        mid = torch.empty(*lead, G, dg, dtype=o.dtype, device=o.device)
    if out is None:
        out = torch.empty(*lead, D, dtype=o.dtype, device=o.device)
    _check("cskv_grouped_out_proj", lib().cskv_grouped_out_proj(
        _ptr(o), _ptr(Wg), _ptr(Wo), _ptr(mid), _ptr(out), T, H, d, G, dg, D, _dtype(o), _stream(o)))
    return (out, mid) if return_mid else out


def indexer_scores_mxfp4(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int, scores=None) -> torch.Tensor:
    """Indexer scores on MX-FP4 rows (dI = 128): [batch, Tq, ld] fp32 (valid for s < V_t)."""
    return _scores_lowp(MXFP4, q_codes, q_scales, wI, k_codes, k_scales, pos0, m, scores)


def indexer_topk_mxfp4(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int, k: int, out=None,
                       workspace=None) -> torch.Tensor:
    """Top-k compressed entries per query from MX-FP4 rows: [batch, Tq, k] int32, ascending, -1 padded."""
    return _topk_lowp(MXFP4, q_codes, q_scales, wI, k_codes, k_scales, pos0, m, k, out, workspace)


def indexer_scores_mxfp8(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int, scores=None) -> torch.Tensor:
    """Indexer scores on MX-FP8 rows (dI = 128): [batch, Tq, ld] fp32 (valid for s < V_t)."""
    return _scores_lowp(MXFP8, q_codes, q_scales, wI, k_codes, k_scales, pos0, m, scores)


def indexer_topk_mxfp8(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int, k: int, out=None,
                       workspace=None) -> torch.Tensor:
    """Top-k compressed entries per query from MX-FP8 rows: [batch, Tq, k] int32, ascending, -1 padded."""
    return _topk_lowp(MXFP8, q_codes, q_scales, wI, k_codes, k_scales, pos0, m, k, out, workspace)
