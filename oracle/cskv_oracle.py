"""CPU oracle for the DeepSeek-V4 hybrid compressed attention layer (CSA / HCA).

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library never
calls it and shares no code with it.

Plain NumPy, float64 arithmetic on the given input values, written for a
reader to check against the pages by eye; no blocking, fusion or reordering.
Sources, cited by page title and section:

* "Paper Breakdown: DeepSeek-V4", section 4 "Hybrid Attention: CSA + HCA
  (§2.3)": the CSA compressor (§2.3.1, two streams, overlapped blocks of 2m
  entries, softmax with positional biases), the lightning indexer and top-k
  over compressed keys, MQA core attention plus the uncompressed sliding
  window; HCA (§2.3.2, one stream, ratio 1/m', no overlap, dense attention);
  "Additional Techniques (§2.3.3)": query/KV RMSNorm, partial RoPE on the
  last 64 dims, sliding window, per-head attention sink logits.
* "How DeepSeek-V4 architecture and training work together", section "Two
  compressed views of one history": 4-to-1 pooling, 1024 selected entries
  per query, 128-token local window.
* "Inside DeepSeek V4", "Two compression regimes" and "Local window":
  4x overlapping vs 128x non-overlapping blocks; every CSA and HCA layer
  adds 128 recent uncompressed entries.

Where the pages leave a step open, the plainest reading is taken; each such
reading is named at the function that uses it.

Conventions: t is an absolute token position; compressed entry i (absolute)
covers block [m*i, m*i + m - 1]; query t sees entry i iff its block is
complete, i.e. i < V_t = floor((t + 1) / m) (capped by the entries present).
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# Storage rounding (the cache stores bf16 in bf16 mode)
# ---------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), kept as float64.

    bfloat16 carries 8 significant bits and float32's exponent range; below
    2**-126 its quantum is fixed at 2**-133.
    """
    x = np.asarray(x, dtype=F64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    big = np.ldexp(2.0 - 2.0 ** -8, 127)  # halfway between bf16 max and 2**128
    r = np.where(np.abs(x) >= big, np.copysign(np.inf, x), r)
    return np.where(np.isnan(x), np.nan, r)


# ---------------------------------------------------------------------------
# Query / KV RMSNorm and partial RoPE ("Additional Techniques (§2.3.3)")
# ---------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, gamma: Optional[np.ndarray] = None, eps: float = 1e-6) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * gamma over the last axis.

    Reading: eps = 1e-6 and gamma = 1 unless given (the pages name the norm only).
    """
    x = np.asarray(x, dtype=F64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x / r
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=F64)
    return y


def rope(x: np.ndarray, pos, rope_dims: int, base: float = 10000.0) -> np.ndarray:
    """Rotate the last `rope_dims` dims of x by position `pos` (RoFormer rotary form).

    Reading of "Partial RoPE (last 64 dims)": pairs (2j, 2j+1), counted from
    the first rotated dim, turn by angle pos * base**(-2j/rope_dims). `pos`
    broadcasts against x's leading axes.
    """
    x = np.array(x, dtype=F64, copy=True)
    if rope_dims == 0:
        return x
    d = x.shape[-1]
    j = np.arange(rope_dims // 2, dtype=F64)
    theta = base ** (-2.0 * j / rope_dims)
    ang = np.asarray(pos, dtype=F64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x0 = x[..., d - rope_dims + 0::2].copy()
    x1 = x[..., d - rope_dims + 1::2].copy()
    x[..., d - rope_dims + 0::2] = x0 * c - x1 * s
    x[..., d - rope_dims + 1::2] = x0 * s + x1 * c
    return x


def _epilogue(chat, positions, apply_norm, norm_w, eps, rope_dims, rope_base):
    e = rmsnorm(chat, norm_w, eps) if apply_norm else chat
    return rope(e, positions, rope_dims, rope_base)


# ---------------------------------------------------------------------------
# KV compression ("Paper Breakdown: DeepSeek-V4", CSA §2.3.1 and HCA §2.3.2)
# ---------------------------------------------------------------------------

def csa_compress(Ca, Cb, Za, Zb, B, m: int, pos0: int = 0, prev_Cb=None, prev_Zb=None,
                 apply_norm: bool = False, norm_w=None, eps: float = 1e-6,
                 rope_dims: int = 0, rope_base: float = 10000.0) -> np.ndarray:
    """Overlapped 1/m compression with two softmax-weighted streams (one sequence).

    Ca, Cb, Za, Zb: [T, c]; B: [2m, c] holding B^b (rows 0..m-1) above B^a
    (rows m..2m-1); prev_Cb / prev_Zb: [m, c], the b-stream rows of the block
    just before row 0 (positions pos0-m .. pos0-1), or None.

    Readings (the sums' ranges are lost in the pages' formula): entry i pools
    2m entries, the m a-stream rows of its own block and the m b-stream rows
    of the block before it, under ONE softmax per channel over the 2m logits
    Z + B; when no preceding block exists the b-half is left out of the
    softmax. Output entry i has absolute index pos0/m + i; its RoPE position
    is the first token of its own block, pos0 + m*i.
    """
    Ca, Cb, Za, Zb, B = (np.asarray(a, dtype=F64) for a in (Ca, Cb, Za, Zb, B))
    T, c = Ca.shape
    assert B.shape == (2 * m, c) and pos0 % m == 0
    n = T // m
    out = np.zeros((n, c), dtype=F64)
    for i in range(n):
        a_rows = slice(m * i, m * i + m)
        logits = [Za[a_rows] + B[m:]]
        values = [Ca[a_rows]]
        if i > 0:
            b_rows = slice(m * (i - 1), m * i)
            logits.insert(0, Zb[b_rows] + B[:m])
            values.insert(0, Cb[b_rows])
        elif prev_Cb is not None:
            logits.insert(0, np.asarray(prev_Zb, dtype=F64) + B[:m])
            values.insert(0, np.asarray(prev_Cb, dtype=F64))
        L = np.concatenate(logits, axis=0)  # [2m or m, c]
        Vv = np.concatenate(values, axis=0)
        S = np.exp(L - L.max(axis=0, keepdims=True))
        S = S / S.sum(axis=0, keepdims=True)
        out[i] = (S * Vv).sum(axis=0)
    pos = pos0 + m * np.arange(n)
    return _epilogue(out, pos, apply_norm, norm_w, eps, rope_dims, rope_base)


def csa_weights(Za, Zb, B, m: int, i: int) -> np.ndarray:
    """The 2m (or m) softmax weights per channel used for entry i (for pins)."""
    Za, Zb, B = (np.asarray(a, dtype=F64) for a in (Za, Zb, B))
    L = Za[m * i:m * i + m] + B[m:]
    if i > 0:
        L = np.concatenate([Zb[m * (i - 1):m * i] + B[:m], L], axis=0)
    S = np.exp(L - L.max(axis=0, keepdims=True))
    return S / S.sum(axis=0, keepdims=True)


def hca_compress(C, Z=None, B=None, m: int = 128, pos0: int = 0, apply_norm: bool = False,
                 norm_w=None, eps: float = 1e-6, rope_dims: int = 0,
                 rope_base: float = 10000.0) -> np.ndarray:
    """Non-overlapped 1/m' compression of one stream (one sequence).

    C, Z: [T, c] (Z None: uniform weights); B: [m', c] positional bias (None: 0).
    Entry i = sum over the m' rows of block i of softmax_p(Z + B) * C, per
    channel; RoPE position pos0 + m'*i. With m' = 1 this prepares raw
    sliding-window rows (norm + RoPE at their own position).
    """
    C = np.asarray(C, dtype=F64)
    T, c = C.shape
    Z = np.zeros_like(C) if Z is None else np.asarray(Z, dtype=F64)
    B = np.zeros((m, c)) if B is None else np.asarray(B, dtype=F64)
    n = T // m
    out = np.zeros((n, c), dtype=F64)
    for i in range(n):
        L = Z[m * i:m * i + m] + B
        S = np.exp(L - L.max(axis=0, keepdims=True))
        S = S / S.sum(axis=0, keepdims=True)
        out[i] = (S * C[m * i:m * i + m]).sum(axis=0)
    pos = pos0 + m * np.arange(n)
    return _epilogue(out, pos, apply_norm, norm_w, eps, rope_dims, rope_base)


# ---------------------------------------------------------------------------
# Lightning indexer and top-k ("Paper Breakdown: DeepSeek-V4", CSA §2.3.1,
# "DSA on Compressed KV (lightning indexer + top-k)")
# ---------------------------------------------------------------------------

def visible(t: int, m: int, N: int) -> int:
    """Number of compressed entries query t may see: complete blocks only, capped at N."""
    return min(N, (t + 1) // m)


def indexer_scores(qI, wI, KI, pos0: int, m: int) -> np.ndarray:
    """I[j, s] = sum_h w[j,h] * max(0, qI[j,h,:] . KI[s,:]) for s < V_t, -inf elsewhere.

    qI: [Tq, HI, dI]; wI: [Tq, HI]; KI: [N, dI]; query j sits at t = pos0 + j.
    Reading: the scoring form is a head-weighted sum of ReLU'd dot products
    (the V3.2 lightning indexer the page names); no scale, norm or RoPE on
    this path, since a positive scale does not change a top-k.
    """
    qI, wI, KI = (np.asarray(a, dtype=F64) for a in (qI, wI, KI))
    Tq = qI.shape[0]
    N = KI.shape[0]
    out = np.full((Tq, N), -np.inf)
    for j in range(Tq):
        V = visible(pos0 + j, m, N)
        dots = KI[:V] @ qI[j].T  # [V, HI]
        out[j, :V] = (np.maximum(dots, 0.0) * wI[j][None, :]).sum(axis=1)
    return out


def topk_row(scores: np.ndarray, V: int, k: int) -> np.ndarray:
    """The k largest of scores[:V]; ties go to the smaller index; ascending; -1 padded.

    Readings: when V <= k every visible entry is selected; among equal scores
    the smaller compressed index wins; the output lists indices in
    ascending order.
    """
    out = np.full(k, -1, dtype=np.int64)
    if V <= k:
        out[:V] = np.arange(V)
        return out
    s = np.asarray(scores[:V], dtype=F64)
    order = np.lexsort((np.arange(V), -s))  # primary key -s, then index
    out[:] = np.sort(order[:k])
    return out


def indexer_topk(qI, wI, KI, pos0: int, m: int, k: int) -> np.ndarray:
    I = indexer_scores(qI, wI, KI, pos0, m)
    N = KI.shape[0]
    return np.stack([topk_row(I[j], visible(pos0 + j, m, N), k) for j in range(I.shape[0])])


# ---------------------------------------------------------------------------
# Low-precision indexer ("Paper Breakdown: DeepSeek-V4", section 4,
# "Efficiency (§2.3.4)": indexer compute FP8 in V3.2 and FP4 in V4;
# infrastructure table: FP4 quantization-aware training of the indexer QK
# path). The pages name the precision only. Readings: FP8 is the OCP E4M3
# format (4 exponent bits, bias 7, 3 mantissa bits, no infinities, largest
# finite value 448); "block scales" are one fp32 scale per row of dI values
# (one compressed key, or one (query, head) of the indexer queries).
# ---------------------------------------------------------------------------

FP8_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """Value of each non-negative finite E4M3 code 0..126 (code 127 is NaN).

    Codes 0..7 are subnormal, c * 2**-9; codes 8..126 are normal, with
    exponent field e = c // 8 and mantissa field f = c % 8:
    (1 + f/8) * 2**(e - 7) = (8 + f) * 2**(e - 10).
    """
    c = np.arange(127)
    sub = c * 2.0 ** -9
    nor = (8 + c % 8) * np.exp2(c // 8 - 10.0)
    return np.where(c < 8, sub, nor).astype(F64)


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code), saturating at +-448.

    Negative values (and -0.0) carry the sign bit 0x80. Input is taken as
    float64; NaN is not expected.
    """
    y = np.asarray(y, dtype=F64)
    a = np.minimum(np.abs(y), FP8_MAX)
    vals = e4m3_values()
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 126)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of E4M3 codes (0x7F and 0xFF decode to NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    mag = c & 0x7F
    v = np.where(mag == 127, np.nan, e4m3_values()[np.minimum(mag, 126)])
    return np.where(c & 0x80, -v, v)


def quantize_rows_fp8(x) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row E4M3 codes and scales: x ~= decode(codes) * scale[..., None].

    Per row: amax = max |x|; code = e4m3(x * (448 / amax)); scale = amax / 448.
    The quotient, the product and the scale are float32 operations: they
    decide integer codes, so they are taken in the kernel's precision. A row
    of zeros gets code 0 and scale 0.
    """
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    safe = np.where(amax > 0, amax, np.float32(1))
    inv = (np.float32(FP8_MAX) / safe).astype(np.float32)
    y = (x32 * inv[..., None]).astype(np.float32)
    codes = e4m3_encode(y)
    codes = np.where((amax > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    scale = np.where(amax > 0, (amax / np.float32(FP8_MAX)).astype(np.float32), np.float32(0))
    return codes, scale.astype(np.float32)


def indexer_scores_fp8(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int) -> np.ndarray:
    """Indexer scores on E4M3 rows: the plain indexer on the dequantised values.

    q_codes [Tq, HI, dI] with q_scales [Tq, HI]; k_codes [N, dI] with
    k_scales [N]. Since ReLU commutes with a positive scale,
    I[j, s] = ks[s] * sum_h wI[j,h] * qs[j,h] * max(0, dq[j,h,:] . dk[s,:]),
    dq, dk the decoded codes; computed here as indexer_scores of
    dq * qs and dk * ks, in float64.
    """
    q = e4m3_decode(q_codes) * np.asarray(q_scales, dtype=F64)[..., None]
    kk = e4m3_decode(k_codes) * np.asarray(k_scales, dtype=F64)[..., None]
    return indexer_scores(q, wI, kk, pos0, m)


FP4_MAX = 6.0


def e2m1_values() -> np.ndarray:
    """Value of each non-negative FP4 E2M1 code 0..7 (OCP: 2 exponent bits, bias 1, 1 mantissa bit).

    Codes 0 and 1 are 0 and the subnormal 0.5; codes 2..7 have exponent field
    e = c // 2 and mantissa bit f = c % 2: (1 + f/2) * 2**(e - 1).
    """
    c = np.arange(8)
    return np.where(c < 2, c * 0.5, (2 + c % 2) * np.exp2(c // 2 - 2.0)).astype(F64)


def e2m1_encode(y) -> np.ndarray:
    """Nearest E2M1 code of each value (ties to the even code), saturating at +-6; bit 3 = sign."""
    y = np.asarray(y, dtype=F64)
    a = np.minimum(np.abs(y), FP4_MAX)
    vals = e2m1_values()
    d = np.abs(a[..., None] - vals)                       # distance to every value
    best = d.min(axis=-1, keepdims=True)
    tied = d == best
    even = tied & (np.arange(8) % 2 == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(tied, axis=-1)).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x8, code).astype(np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    v = e2m1_values()[c & 0x7]
    return np.where(c & 0x8, -v, v)


def pack_nibbles(codes) -> np.ndarray:
    """Two 4-bit codes per byte along the last axis: element 2i in the low nibble of byte i."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def quantize_rows_fp4(x) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row E2M1 codes (unpacked, one per element) and scales, as quantize_rows_fp8 with 6 for 448."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    safe = np.where(amax > 0, amax, np.float32(1))
    inv = (np.float32(FP4_MAX) / safe).astype(np.float32)
    y = (x32 * inv[..., None]).astype(np.float32)
    codes = np.where((amax > 0)[..., None], e2m1_encode(y), np.uint8(0)).astype(np.uint8)
    scale = np.where(amax > 0, (amax / np.float32(FP4_MAX)).astype(np.float32), np.float32(0))
    return codes, scale.astype(np.float32)


def indexer_scores_fp4(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int) -> np.ndarray:
    """Indexer scores on E2M1 rows (unpacked codes): the plain indexer on the dequantised values."""
    q = e2m1_decode(q_codes) * np.asarray(q_scales, dtype=F64)[..., None]
    kk = e2m1_decode(k_codes) * np.asarray(k_scales, dtype=F64)[..., None]
    return indexer_scores(q, wI, kk, pos0, m)


# ---------------------------------------------------------------------------
# FP4 indexer with block scales ("Paper Breakdown: DeepSeek-V4", "Efficiency
# (§2.3.4)": FP4 indexer QK path in V4). Reading: the block scales are those
# of the OCP Microscaling (MX) formats, the published standard for FP4 with
# shared scales: blocks of 32 consecutive values along dI share one E8M0
# scale (a power of two, 2**(code - 127)); the shared exponent is
# floor(log2(amax)) - 2 (2 = the exponent of E2M1's largest value, 6 =
# 1.5 * 2**2), and each value is stored as E2M1(x / scale) rounded to
# nearest, ties to even, saturating at +-6. An all-zero block takes scale
# code 0 and zero codes; exponents below -127 are clamped to code 0. MX-FP8
# (the FP8 setting with the same block scales) stores E4M3 values with the
# shared exponent floor(log2(amax)) - 8.
# ---------------------------------------------------------------------------

MX_BLOCK = 32
E2M1_EMAX = 2   # E2M1's largest value 6 = 1.5 * 2**2
E4M3_EMAX = 8   # E4M3's largest value 448 = 1.75 * 2**8 (MX-FP8, the same layout with E4M3 values)


def mx_scale_codes(amax, emax: int = E2M1_EMAX) -> np.ndarray:
    """E8M0 code of each block's shared scale from its largest magnitude (fp32 values)."""
    a = np.asarray(amax, dtype=F64)
    _, ex = np.frexp(a)                       # a = f * 2**ex, f in [0.5, 1): floor(log2 a) = ex - 1
    e = ex.astype(np.int64) - 1 - emax
    return np.where(a > 0, np.clip(e + 127, 0, 254), 0).astype(np.uint8)


def _quantize_rows_mx(x, emax: int, encode) -> Tuple[np.ndarray, np.ndarray]:
    x32 = np.asarray(x, dtype=np.float32)
    d = x32.shape[-1]
    assert d % MX_BLOCK == 0
    xb = x32.reshape(x32.shape[:-1] + (d // MX_BLOCK, MX_BLOCK)).astype(F64)
    amax = np.abs(xb).max(axis=-1)
    sc = mx_scale_codes(amax, emax)
    y = xb / np.exp2(sc.astype(F64) - 127)[..., None]   # exact: a power-of-two divisor
    codes = np.where((amax > 0)[..., None], encode(y), np.uint8(0)).astype(np.uint8)
    return codes.reshape(x32.shape), sc


def _dequantize_mx(codes, scales, decode) -> np.ndarray:
    c = np.asarray(codes)
    d = c.shape[-1]
    v = decode(c).reshape(c.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    v = v * np.exp2(np.asarray(scales, dtype=F64) - 127)[..., None]
    return v.reshape(c.shape)


def quantize_rows_mxfp4(x) -> Tuple[np.ndarray, np.ndarray]:
    """MX-FP4 codes (unpacked, one per element) and E8M0 scale codes ([..., dim / 32]) of fp32 rows."""
    return _quantize_rows_mx(x, E2M1_EMAX, e2m1_encode)


def dequantize_mxfp4(codes, scales) -> np.ndarray:
    return _dequantize_mx(codes, scales, e2m1_decode)


def indexer_scores_mxfp4(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int) -> np.ndarray:
    """Indexer scores on MX-FP4 rows: the plain indexer on the dequantised values."""
    return indexer_scores(dequantize_mxfp4(q_codes, q_scales), wI, dequantize_mxfp4(k_codes, k_scales), pos0, m)


def quantize_rows_mxfp8(x) -> Tuple[np.ndarray, np.ndarray]:
    """MX-FP8 codes (E4M3, one byte per element) and E8M0 scale codes ([..., dim / 32]) of fp32 rows:
    shared exponent floor(log2 amax) - 8, values E4M3(x / scale), nearest even, saturating at 448."""
    return _quantize_rows_mx(x, E4M3_EMAX, e4m3_encode)


def dequantize_mxfp8(codes, scales) -> np.ndarray:
    return _dequantize_mx(codes, scales, e4m3_decode)


def indexer_scores_mxfp8(q_codes, q_scales, wI, k_codes, k_scales, pos0: int, m: int) -> np.ndarray:
    """Indexer scores on MX-FP8 rows: the plain indexer on the dequantised values."""
    return indexer_scores(dequantize_mxfp8(q_codes, q_scales), wI, dequantize_mxfp8(k_codes, k_scales), pos0, m)


# ---------------------------------------------------------------------------
# FP8 KV storage ("Paper Breakdown: DeepSeek-V4", "Efficiency (§2.3.4)": V4
# stores the KV cache as FP8 for the non-RoPE dims and BF16 for the RoPE dims).
# Readings: the FP8 part is OCP E4M3 with one scale per entry; the scale is a
# power of two, the smallest that keeps the entry's non-RoPE values within
# +-448, so the stored values are exact multiples and dequantisation is exact.
# ---------------------------------------------------------------------------

def kv_scale_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2**e (0 where amax == 0)."""
    a = np.asarray(amax, dtype=F64)
    _, E = np.frexp(np.where(a > 0, a, 1.0))      # a = f * 2**E, f in [0.5, 1): a in [2**(E-1), 2**E)
    e = E - 9                                      # a * 2**-e in [256, 512)
    e = np.where(a * np.exp2(-e) > FP8_MAX, e + 1, e)
    return np.where(a > 0, e, 0).astype(np.int64)


def quantize_kv_fp8(x, rope_dims: int):
    """One compressed entry (or a stack of them) to its FP8 + BF16 storage.

    Returns (codes [..., d - rope_dims] uint8, rope [..., rope_dims] bf16
    values as float64, scale [...] float64 powers of two).
    """
    x = np.asarray(x, dtype=F64)
    nope = x.shape[-1] - rope_dims
    xn = x[..., :nope]
    e = kv_scale_exponent(np.max(np.abs(xn), axis=-1))
    scale = np.exp2(e.astype(F64))
    codes = e4m3_encode(xn * np.exp2(-e.astype(F64))[..., None])
    return codes, round_bf16(x[..., nope:]), scale


def dequantize_kv_fp8(codes, rope, scale) -> np.ndarray:
    """Stored FP8 + BF16 entry back to its values: decode(codes) * scale, then the RoPE dims."""
    v = e4m3_decode(codes) * np.asarray(scale, dtype=F64)[..., None]
    return np.concatenate([v, np.asarray(rope, dtype=F64)], axis=-1)


# ---------------------------------------------------------------------------
# Core MQA attention over compressed entries + sliding window + sink
# ("Paper Breakdown: DeepSeek-V4", CSA §2.3.1, HCA §2.3.2, §2.3.3)
# ---------------------------------------------------------------------------

def prepare_query(q, t: int, apply_norm: bool, norm_w, eps, rope_dims, rope_base):
    """RMSNorm per head, then RoPE at the query's absolute position t."""
    x = rmsnorm(q, norm_w, eps) if apply_norm else np.asarray(q, dtype=F64)
    return rope(x, np.full(x.shape[:-1], t), rope_dims, rope_base)


def attend_one(qt: np.ndarray, keys: np.ndarray, sink: Optional[np.ndarray], scale: float):
    """Softmax attention of prepared queries qt [H, d] over keys [n, d] (K = V = entry).

    The sink z_h joins the denominator with a zero value vector. Returns o [H, d]
    and lse [H] = log(exp(z_h) + sum_j exp(l_j)).
    """
    H = qt.shape[0]
    z = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=F64)
    l = (qt @ keys.T) * scale  # [H, n]
    M = np.maximum(z, l.max(axis=1) if l.shape[1] else -np.inf)
    p = np.exp(l - M[:, None])
    D = np.exp(z - M) + p.sum(axis=1)
    o = (p @ keys) / D[:, None]
    return o, M + np.log(D)


def attention(q, kv, win, win_pos0: int, pos0: int, m: int, w: int, idx=None, sink=None,
              scale: float = 0.0, apply_q_norm: bool = True, q_norm_w=None, eps: float = 1e-6,
              rope_dims: int = 0, rope_base: float = 10000.0, rope_on_output: bool = True,
              rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """CSA (idx given) or HCA (idx None) attention for one sequence.

    q: [Tq, H, d] raw queries (query j at t = pos0 + j); kv: [N, d] compressed
    entries as stored; win: [W, d] prepared window rows, row r at position
    win_pos0 + r; idx: [Tq, k] selected entries (-1 = none) for CSA.
    Key set of query t: the selected (CSA) or all V_t visible (HCA) entries,
    plus the window rows at positions max(0, t-w+1) .. t.

    Readings: scale 0 means 1/sqrt(d); no de-duplication between window rows
    and compressed entries; "relative position on core outputs" is read as
    rotating the output's last rope_dims dims back by -t, so that each value's
    rotary phase becomes its position relative to the query (a flag).
    `rows` restricts the computation to a subset of query rows (returned in
    that order).
    """
    q = np.asarray(q, dtype=F64)
    kv = np.asarray(kv, dtype=F64)
    win = np.asarray(win, dtype=F64)
    Tq, H, d = q.shape
    N = kv.shape[0]
    sc = scale if scale > 0 else 1.0 / math.sqrt(d)
    rows = range(Tq) if rows is None else rows
    outs, lses = [], []
    for j in rows:
        t = pos0 + j
        if idx is None:
            comp = kv[:visible(t, m, N)]
        else:
            sel = [int(s) for s in idx[j] if 0 <= s < N]
            comp = kv[sel]
        lo = max(0, t - w + 1)
        if lo < win_pos0 or t - win_pos0 >= win.shape[0]:
            raise ValueError(f"window rows at positions {win_pos0}..{win_pos0 + win.shape[0] - 1} "
                             f"do not cover query {t}'s window {lo}..{t}")
        wrows = win[lo - win_pos0:t - win_pos0 + 1]
        keys = np.concatenate([comp, wrows], axis=0)
        qt = prepare_query(q[j], t, apply_q_norm, q_norm_w, eps, rope_dims, rope_base)
        o, lse = attend_one(qt, keys, sink, sc)
        if rope_on_output:
            o = rope(o, np.full(H, -t), rope_dims, rope_base)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------
# Projections around the core attention ("Paper Breakdown: DeepSeek-V4",
# section 4, CSA §2.3.1: low-rank indexer queries from a shared latent c_t^Q;
# "MQA core attention + grouped output projection"; HCA §2.3.2: same MQA +
# grouped projection). The pages give no shapes; the readings are named here.
# ---------------------------------------------------------------------------

def lowrank_proj(cq, W) -> np.ndarray:
    """Query (or indexer-query) heads from the shared latent: out[t] = c^Q_t W.

    Reading: both the attention queries and the indexer queries are one plain
    product of the token's latent c^Q_t [r] with a weight [r, heads * dim]; the
    per-head query RMSNorm and RoPE stay in the attention (they follow it).
    """
    return np.asarray(cq, dtype=F64) @ np.asarray(W, dtype=F64)


def grouped_out_proj_mid(o, Wg) -> np.ndarray:
    """First stage of the grouped output projection, per token:
    u[t, g] = concat(o[t, h] for h in group g) @ Wg[g].

    Reading: the H heads form G contiguous groups of H/G heads; each group's
    concatenated outputs [(H/G) * d] have their own projection Wg[g] [(H/G) d, d_g].
    o: [T, H, d]; Wg: [G, (H/G) d, d_g] -> u: [T, G, d_g].
    """
    o = np.asarray(o, dtype=F64)
    Wg = np.asarray(Wg, dtype=F64)
    T, H, d = o.shape
    G = Wg.shape[0]
    og = o.reshape(T, G, (H // G) * d)
    return np.stack([og[:, g, :] @ Wg[g] for g in range(G)], axis=1)


def grouped_out_proj(o, Wg, Wo, round_mid: bool = True) -> np.ndarray:
    """Grouped output projection: y[t] = concat_g(u[t, g]) @ Wo, u from
    grouped_out_proj_mid. Wo: [G d_g, D] -> y: [T, D].

    round_mid: the intermediate u is a stored bf16 tensor on the GPU path, so it
    is rounded to bf16 here too (a rounding point the kernels share).
    """
    u = grouped_out_proj_mid(o, Wg)
    if round_mid:
        u = round_bf16(u)
    T = u.shape[0]
    return u.reshape(T, -1) @ np.asarray(Wo, dtype=F64)


# ---------------------------------------------------------------------------
# Whole-layer drivers (compress -> [indexer -> top-k] -> attention)
# ---------------------------------------------------------------------------

def prepare_window(raw, win_pos0: int, apply_norm=True, norm_w=None, eps=1e-6,
                   rope_dims=0, rope_base=10000.0) -> np.ndarray:
    """Raw per-token KV rows -> window rows: RMSNorm + RoPE at each row's own position."""
    return hca_compress(raw, None, None, 1, win_pos0, apply_norm, norm_w, eps, rope_dims, rope_base)
