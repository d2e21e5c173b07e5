"""MI355X (gfx950) implementation of DeepSeek-V4's hybrid compressed attention layer.

The compute path is libcskv.so (hand-written HIP kernels behind a C ABI,
include/cskv.h); `binding` marshals torch tensors into it. Importing the
package does not load the library; the first binding call does, and fails
loudly if it has not been built. The attention entry points take an FP8 + BF16
KV cache through their `kv_scale` argument (compressed_attn_prefill_kv8 /
compressed_attn_decode_kv8 of the C ABI).
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    csa_compress,
    hca_compress,
    indexer_topk,
    indexer_scores,
    topk_select,
    quantize_fp8,
    indexer_scores_fp8,
    indexer_topk_fp8,
    quantize_fp4,
    indexer_scores_fp4,
    indexer_topk_fp4,
    quantize_mxfp4,
    indexer_scores_mxfp4,
    indexer_topk_mxfp4,
    quantize_mxfp8,
    indexer_scores_mxfp8,
    indexer_topk_mxfp8,
    quantize_kv_fp8,
    compressed_attn_prefill,
    compressed_attn_decode,
    compressed_attn_decode_noalloc,
    lowrank_proj,
    grouped_out_proj,
)
