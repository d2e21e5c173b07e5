/*
 * cskv.h -- C ABI of libcskv.so, the gfx950 (MI355X) implementation of the
 * DeepSeek-V4 hybrid compressed attention layer: CSA (compressed sparse
 * attention) and HCA (heavily compressed attention).
 *
 * Sources, by page title and section:
 *   [PB]  "Paper Breakdown: DeepSeek-V4", section 4 "Hybrid Attention: CSA +
 *         HCA (§2.3)": CSA (§2.3.1), HCA (§2.3.2), Additional Techniques
 *         (§2.3.3: query/KV RMSNorm, partial RoPE on the last 64 dims,
 *         sliding window, per-head sink logits).
 *   [HW]  "How DeepSeek-V4 architecture and training work together",
 *         section "Two compressed views of one history" (4-to-1 pooling,
 *         1024 selected entries per query, 128-token window).
 *   [IV]  "Inside DeepSeek V4", "Two compression regimes" (4x overlapping vs
 *         128x non-overlapping) and "Local window" (128 uncompressed entries
 *         in every CSA and HCA layer).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensors are row-major and contiguous, last dimension fastest.
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except
 *    where stated. The library never allocates, frees or synchronises, and
 *    keeps no state between calls: scratch memory comes only from the
 *    caller's `workspace`, sized by the matching *_workspace_size call.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream). Outputs are valid once that stream reaches this point.
 *  - `dtype` selects the storage type of q, kv, window rows, streams and
 *    outputs: CSKV_BF16 (fp32 accumulation, bf16 matrix cores) or CSKV_F32.
 *    Head weights `wI`, sink logits, norm gains and `lse` are always fp32;
 *    indices are int32; positions and lengths are int64.
 *  - Device pointers must be 16-byte aligned.
 *  - Positions are absolute token positions. Compressed entry i covers the
 *    block of tokens [m*i, m*i + m - 1] and sits at rotary position m*i; a
 *    query at position t may see entry i only once that block is complete:
 *    i < V_t = min(N, floor((t + 1) / m)).
 *  - Return value: CSKV_OK (0) or a negative CSKV_ERR_* code. Arguments are
 *    validated before any HIP call; a failed validation enqueues nothing.
 *    A launch failure returns CSKV_ERR_HIP. No exception crosses the ABI.
 *  - Results are deterministic: no floating-point atomics, fixed reduction
 *    order, so repeated calls give bit-identical outputs.
 */
#ifndef CSKV_H_
#define CSKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CSKV_OK = 0,
  CSKV_ERR_INVALID_ARG = -1,  /* null pointer where one is required, bad enum */
  CSKV_ERR_BAD_SHAPE = -2,    /* sizes inconsistent or out of the supported range */
  CSKV_ERR_BAD_DTYPE = -3,    /* dtype not CSKV_BF16 / CSKV_F32 */
  CSKV_ERR_MISALIGNED = -4,   /* a pointer is not 16-byte aligned */
  CSKV_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required */
  CSKV_ERR_UNSUPPORTED = -6,  /* valid request outside this build's limits (e.g. k > CSKV_MAX_TOPK) */
  CSKV_ERR_HIP = -7           /* a kernel launch failed */
};

enum { CSKV_BF16 = 0, CSKV_F32 = 1, CSKV_FP8 = 2 /* E4M3 codes, fp32 row scales */,
       CSKV_FP4 = 3 /* E2M1 codes, two per byte, fp32 row scales */,
       CSKV_MXFP4 = 4 /* E2M1 codes, two per byte, one E8M0 scale per 32 values */,
       CSKV_MXFP8 = 5 /* E4M3 codes, one E8M0 scale per 32 values */ };
enum { CSKV_MODE_CSA = 0, CSKV_MODE_HCA = 1 };

#define CSKV_MAX_TOPK 2048
#define CSKV_MAX_DIM 1024     /* d (KV/head dim) and dI upper bound */
#define CSKV_MAX_HEADS 128

/* Library version as 10000*major + 100*minor + patch. */
int cskv_version(void);
/* Static text for a status code (never NULL). */
const char* cskv_status_string(int status);

/*
 * csa_compress -- overlapped 1/m KV compression with two softmax-weighted
 * streams [PB §2.3.1 "KV Compression"; IV "Two compression regimes"].
 *
 * For each complete block i of m new tokens and each channel, one softmax
 * runs over 2m logits: the m b-stream rows of the previous block (Zb + B^b)
 * and the m a-stream rows of block i (Za + B^a). The entry is the
 * softmax-weighted sum of the matching Cb and Ca rows. Optionally followed by
 * RMSNorm over the c channels and RoPE on the last rope_dims channels at
 * position pos0 + m*i ([PB §2.3.3]). Used for the KV entries (d = 512, norm
 * and RoPE on) and for the indexer keys (dI = 128, both off) [PB §2.3.1,
 * "Indexer keys compressed same way"].
 *
 *   Ca, Cb, Za, Zb : [batch, T, c]   token streams, positions pos0 .. pos0+T-1
 *   B              : [2m, c]         rows 0..m-1 = B^b, rows m..2m-1 = B^a
 *   prev_Cb,prev_Zb: [batch, m, c]   b-stream rows at positions pos0-m .. pos0-1
 *                                    (the tail of the previous chunk), or both
 *                                    NULL: then entry 0's b-half is left out of
 *                                    its softmax (first block of a sequence)
 *   T >= 0, 1 <= m <= 128, pos0 % m == 0, c % 8 == 0, 8 <= c <= CSKV_MAX_DIM
 *   apply_norm     : 0/1; norm_w [c] fp32 or NULL (gain 1); eps > 0
 *   rope_dims      : 0 (off) or even, <= c; rope_base > 0
 *   out            : [batch, out_ld, c]; entry i of sequence b goes to row
 *                    b*out_ld + i, so new entries can be appended in place
 *                    to a cache (pass the pointer to the first new row);
 *                    out_ld = 0 means floor(T/m), else out_ld >= floor(T/m).
 *                    A trailing partial block is not emitted (the caller
 *                    carries it to the next chunk).
 */
int csa_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb, const void* B,
                 const void* prev_Cb, const void* prev_Zb, int batch, int64_t T, int c, int m,
                 int64_t pos0, int apply_norm, const float* norm_w, float eps, int rope_dims,
                 float rope_base, void* out, int64_t out_ld, int dtype, void* stream);

/*
 * hca_compress -- non-overlapped 1/m' compression of one stream [PB §2.3.2;
 * IV "Two compression regimes"]: entry i is the per-channel softmax over
 * the m' rows of block i (Z + B) weighting C, then optional RMSNorm + RoPE
 * at position pos0 + m'*i. With m' = 1 the softmax is over a single row, so
 * the call prepares raw sliding-window rows (RMSNorm + RoPE at each row's own
 * position) [PB §2.3.1 "Sliding window KV (uncompressed)"; IV "Local window"].
 *
 *   C   : [batch, T, c]; Z : [batch, T, c] or NULL (uniform weights)
 *   B   : [m', c] or NULL (zero bias)
 *   1 <= m' <= 4096, pos0 % m' == 0; other arguments as in csa_compress
 *   out : [batch, out_ld, c] as in csa_compress (out_ld = 0: floor(T/m'))
 */
int hca_compress(const void* C, const void* Z, const void* B, int batch, int64_t T, int c, int m,
                 int64_t pos0, int apply_norm, const float* norm_w, float eps, int rope_dims,
                 float rope_base, void* out, int64_t out_ld, int dtype, void* stream);

/*
 * indexer_topk -- lightning-indexer scores over compressed keys, then per
 * query top-k [PB §2.3.1 "DSA on Compressed KV (lightning indexer + top-k)";
 * HW "Two compressed views of one history" (k = 1024)].
 *
 *   I[t, s] = sum_h wI[t, h] * max(0, qI[t, h, :] . KI[s, :])  for s < V_t
 *
 * out_idx[t] lists the k entries of largest I in ascending index order;
 * among equal scores the smaller index wins; when V_t <= k all visible
 * entries are listed and the rest is -1.
 *
 *   qI  : [batch, Tq, HI, dI]  indexer queries, query j at position pos0 + j
 *   wI  : [batch, Tq, HI]      fp32 head weights
 *   KI  : [batch, N, dI]       compressed indexer keys (entries 0 .. N-1)
 *   1 <= HI <= CSKV_MAX_HEADS; bf16: dI in {32, 64, 128}; f32: dI % 16 == 0 and
 *   (HI * dI + HI) * 4 <= 48 KiB
 *   1 <= k <= CSKV_MAX_TOPK, m >= 1
 *   out_idx   : [batch, Tq, k] int32
 *   workspace : cskv_indexer_workspace_size(...) bytes of device memory (fp32
 *               score rows, and per-part candidates when few long rows are
 *               selected with several workgroups per row)
 */
size_t cskv_indexer_workspace_size(int batch, int64_t Tq, int64_t N, int HI, int k, int dtype);
int indexer_topk(const void* qI, const float* wI, const void* KI, int batch, int64_t Tq, int64_t N,
                 int HI, int dI, int64_t pos0, int m, int k, int32_t* out_idx, void* workspace,
                 size_t ws_bytes, int dtype, void* stream);

/*
 * indexer_scores / topk_select -- the two halves of indexer_topk, for callers
 * that keep the score matrix themselves (e.g. to time or reuse it).
 *
 * indexer_scores writes scores[(b*Tq + j)*ld + s] = I[t, s] (fp32) for every
 * visible entry s < V_t of query j; entries past V_t up to the end of the
 * swept key range may hold -inf and later ones are left untouched.
 *   scores : [batch, Tq, ld] fp32, ld >= N and ld % 4 == 0
 *   other arguments and limits as in indexer_topk
 * topk_select reads such a matrix and writes out_idx exactly as indexer_topk
 * does (k largest of the first V_t scores, smaller index first among equal
 * scores, ascending, -1 padded). Its workspace is optional (see
 * cskv_topk_workspace_size); ld % 4 == 0 and 16-byte aligned rows.
 *
 * Block maxima (optional; NULL = none), for decode-shaped calls. With
 * block_max != NULL (dtype CSKV_BF16 only, else CSKV_ERR_UNSUPPORTED) and
 * Tq < 64, indexer_scores also writes, for every 32-entry block
 * i < ceil(V_t / 32) of query j,
 *   block_max[(b*Tq + j)*bm_ld + i] = max over s in [32 i, min(32 i + 32, V_t))
 *                                     of key(scores[(b*Tq + j)*ld + s])
 * where key(x) is the fp32 bit pattern of x with the sign bit set when x is
 * non-negative and every bit flipped when it is negative (larger x, larger
 * key; key > 0 for every score). Later blocks, and the whole of block_max
 * when Tq >= 64, are left untouched (the many-query scorer is bound by the
 * matrix cores, and the maxima would cost it more than they save).
 *   block_max : [batch, Tq, bm_ld] uint32, bm_ld >= ceil(N / 32), bm_ld % 4 == 0,
 *               16-byte aligned (else CSKV_ERR_BAD_SHAPE / CSKV_ERR_MISALIGNED)
 * topk_select given the block maxima that indexer_scores wrote with the same
 * batch, Tq, N, pos0 and m reads only the blocks of largest maxima of long
 * rows, without a pass over the whole score rows: it does so when Tq < 64 and
 * every row of the call has at least 2k blocks and at most 8192 (k = 1024:
 * 65536 <= V_t <= 262144), and ignores them otherwise. The result is the same
 * either way; maxima that do not match the scores give an unspecified
 * selection (within the row's first V_t entries).
 */
int indexer_scores(const void* qI, const float* wI, const void* KI, int batch, int64_t Tq, int64_t N,
                   int HI, int dI, int64_t pos0, int m, float* scores, int64_t ld, uint32_t* block_max,
                   int64_t bm_ld, int dtype, void* stream);
int topk_select(const float* scores, int64_t ld, const uint32_t* block_max, int64_t bm_ld, int batch,
                int64_t Tq, int64_t N, int64_t pos0, int m, int k, int32_t* out_idx, void* workspace,
                size_t ws_bytes, void* stream);

/*
 * cskv_topk_workspace_size -- device bytes topk_select may use to select few
 * long rows (at most 64 rows of at least 4 x 8192 visible entries, e.g.
 * decode) with several workgroups per row; 0 when the call has no use for
 * it. A NULL or smaller workspace is allowed: every row is then selected by
 * one workgroup, with the same result.
 */
size_t cskv_topk_workspace_size(int batch, int64_t Tq, int64_t N, int k);

/*
 * FP8 lightning indexer [PB §2.3.4 "Efficiency": indexer compute FP8 in
 * V3.2, FP4 in V4; infrastructure table: FP4 quantization-aware training of
 * the indexer QK path]. The pages name the precision only; here the format is
 * OCP FP8 E4M3 (bias 7, no infinities, largest finite 448) with one fp32
 * scale per row.
 *
 * cskv_quantize_fp8 -- per-row E4M3 quantisation of x [rows, dim]:
 *   amax = max |x[r, :]|; codes[r, :] = E4M3(x[r, :] * (448 / amax)), nearest
 *   value, ties to the even code, saturating; scales[r] = amax / 448. The
 *   quotient and product are correctly rounded fp32. A row of zeros gets
 *   codes 0 and scale 0.
 *   x : [rows, dim] (dtype CSKV_BF16 or CSKV_F32); 4 <= dim <= 1024, dim % 4 == 0
 *   codes : [rows, dim] uint8; scales : [rows] fp32
 *   Use it on indexer keys ([batch*N, dI]) and indexer queries
 *   ([batch*Tq*HI, dI]).
 *
 * indexer_scores_fp8 / indexer_topk_fp8 -- indexer_scores / indexer_topk on
 * E4M3 rows:
 *   I[t, s] = k_scale[s] * sum_h wI[t,h] * q_scale[t,h]
 *                        * max(0, dq[t,h,:] . dk[s,:])
 *   with dq, dk the decoded codes (exact products, fp32 sums on
 *   v_mfma_f32_32x32x64_f8f6f4), which equals the bf16 formula on the
 *   dequantised rows.
 *   qI : [batch, Tq, HI, dI] uint8, q_scale : [batch, Tq, HI] fp32
 *   KI : [batch, N, dI] uint8,      k_scale : [batch, N] fp32
 *   dI in {64, 128}; other arguments, limits and outputs as in indexer_scores /
 *   indexer_topk; the workspace of indexer_topk_fp8 is
 *   cskv_indexer_workspace_size(batch, Tq, N, HI, k, CSKV_FP8) bytes.
 */
int cskv_quantize_fp8(const void* x, int64_t rows, int dim, int dtype, uint8_t* codes, float* scales,
                      void* stream);
int indexer_scores_fp8(const uint8_t* qI, const float* q_scale, const float* wI, const uint8_t* KI,
                       const float* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                       int64_t pos0, int m, float* scores, int64_t ld, void* stream);
int indexer_topk_fp8(const uint8_t* qI, const float* q_scale, const float* wI, const uint8_t* KI,
                     const float* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                     int64_t pos0, int m, int k, int32_t* out_idx, void* workspace, size_t ws_bytes,
                     void* stream);

/*
 * FP4 lightning indexer -- the V4 setting of the same table [PB §2.3.4]:
 * OCP FP4 E2M1 codes (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 * negatives; bit 3 is the sign), two per byte (element 2i in the low nibble
 * of byte i), one fp32 scale per row.
 *
 * cskv_quantize_fp4 -- as cskv_quantize_fp8 with 6 in place of 448:
 *   codes = E2M1(x * (6 / amax)) (nearest, ties to the even code,
 *   saturating); scales = amax / 6.
 *   codes : [rows, dim / 2] bytes
 * indexer_scores_fp4 / indexer_topk_fp4 -- as the FP8 calls on E2M1 rows:
 *   qI : [batch, Tq, HI, dI / 2], KI : [batch, N, dI / 2] bytes. Products of
 *   two E2M1 values are multiples of 1/4 below 36, so each dot product is
 *   exact and only the fp32 head sum rounds. The workspace of
 *   indexer_topk_fp4 is cskv_indexer_workspace_size(..., CSKV_FP4) bytes.
 */
int cskv_quantize_fp4(const void* x, int64_t rows, int dim, int dtype, uint8_t* codes, float* scales,
                      void* stream);
int indexer_scores_fp4(const uint8_t* qI, const float* q_scale, const float* wI, const uint8_t* KI,
                       const float* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                       int64_t pos0, int m, float* scores, int64_t ld, void* stream);
int indexer_topk_fp4(const uint8_t* qI, const float* q_scale, const float* wI, const uint8_t* KI,
                     const float* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                     int64_t pos0, int m, int k, int32_t* out_idx, void* workspace, size_t ws_bytes,
                     void* stream);

/*
 * MX-FP4 lightning indexer -- the FP4 indexer of [PB §2.3.4] with block
 * scales, in the layout of the OCP Microscaling (MX) formats: every 32
 * consecutive values of a row share one E8M0 scale byte (value
 * 2^(code - 127)); the values are the E2M1 codes of cskv_quantize_fp4.
 *
 * cskv_quantize_mxfp4 -- per 32-value block: amax = max |x| (x as fp32),
 *   code = clamp(floor(log2 amax) - 2 + 127, 0, 254) (0 for an all-zero
 *   block), codes = E2M1(x * 2^(127 - code)) (nearest, ties to the even
 *   code, saturating at +-6).
 *   x : [rows, dim] bf16 or fp32 (dtype), dim % 32 == 0, dim <= 1024
 *   codes : [rows, dim / 2] bytes, scales : [rows, dim / 32] bytes;
 *   caller-owned device buffers, 16-byte aligned.
 * indexer_scores_mxfp4 / indexer_topk_mxfp4 -- indexer_scores / indexer_topk on
 *   MX-FP4 rows:
 *   I[t, s] = sum_h wI[t,h] * max(0, q[t,h,:] . k[s,:])
 *   with q, k the decoded rows (code value times its block's scale), the
 *   block scales applied by v_mfma_scale_f32_32x32x64_f8f6f4. Each block's
 *   sum of E2M1 products is exact; the matrix core may truncate when it
 *   adds blocks of different scales (about one fp32 ulp of the dot product),
 *   then the head sum rounds in fp32.
 *   qI : [batch, Tq, HI, 64] bytes, q_scale : [batch, Tq, HI, 4] bytes
 *   KI : [batch, N, 64] bytes,      k_scale : [batch, N, 4] bytes
 *   dI = 128 only (CSKV_ERR_UNSUPPORTED otherwise); other arguments, limits
 *   and outputs as in indexer_scores / indexer_topk; the workspace of
 *   indexer_topk_mxfp4 is cskv_indexer_workspace_size(..., CSKV_MXFP4) bytes.
 */
int cskv_quantize_mxfp4(const void* x, int64_t rows, int dim, int dtype, uint8_t* codes, uint8_t* scales,
                        void* stream);
int indexer_scores_mxfp4(const uint8_t* qI, const uint8_t* q_scale, const float* wI, const uint8_t* KI,
                         const uint8_t* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                         int64_t pos0, int m, float* scores, int64_t ld, void* stream);
int indexer_topk_mxfp4(const uint8_t* qI, const uint8_t* q_scale, const float* wI, const uint8_t* KI,
                       const uint8_t* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                       int64_t pos0, int m, int k, int32_t* out_idx, void* workspace, size_t ws_bytes,
                       void* stream);

/*
 * MX-FP8 lightning indexer -- the FP8 setting of [PB §2.3.4] with the same
 * block scales: E4M3 values (one byte each), one E8M0 scale byte per 32.
 *
 * cskv_quantize_mxfp8 -- as cskv_quantize_mxfp4 with E4M3 values and
 *   code = clamp(floor(log2 amax) - 8 + 127, 0, 254) (E4M3's largest value
 *   is 1.75 * 2^8); codes = E4M3(x * 2^(127 - code)) (nearest, ties to the
 *   even code, saturating at +-448).
 *   codes : [rows, dim] bytes, scales : [rows, dim / 32] bytes.
 * indexer_scores_mxfp8 / indexer_topk_mxfp8 -- as the MX-FP4 calls on E4M3
 *   rows: qI : [batch, Tq, HI, 128], KI : [batch, N, 128] bytes; scales as
 *   for MX-FP4. E4M3 products are summed as in indexer_scores_fp8 (groups of
 *   8 on a grid 2^-13 below the group's largest), then scaled per block. The
 *   workspace of indexer_topk_mxfp8 is
 *   cskv_indexer_workspace_size(..., CSKV_MXFP8) bytes.
 */
int cskv_quantize_mxfp8(const void* x, int64_t rows, int dim, int dtype, uint8_t* codes, uint8_t* scales,
                        void* stream);
int indexer_scores_mxfp8(const uint8_t* qI, const uint8_t* q_scale, const float* wI, const uint8_t* KI,
                         const uint8_t* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                         int64_t pos0, int m, float* scores, int64_t ld, void* stream);
int indexer_topk_mxfp8(const uint8_t* qI, const uint8_t* q_scale, const float* wI, const uint8_t* KI,
                       const uint8_t* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                       int64_t pos0, int m, int k, int32_t* out_idx, void* workspace, size_t ws_bytes,
                       void* stream);

/*
 * compressed_attn_prefill -- MQA core attention over compressed entries,
 * sliding window and sink [PB §2.3.1 "MQA core attention", §2.3.2 "dense on
 * compressed KV", §2.3.3; IV "Local window"].
 *
 * For query j (position t = pos0 + j) and head h:
 *   q~ = RoPE_t(RMSNorm(q[j, h]))                   (norm if apply_q_norm)
 *   keys = { kv[s] : s in idx[j], s >= 0 }           (mode CSKV_MODE_CSA)
 *        | { kv[s] : s < V_t }                       (mode CSKV_MODE_HCA)
 *        + { win rows at positions max(0, t-w+1) .. t }
 *   l_e  = scale * q~ . e    (scale 0 -> 1/sqrt(d)); K = V = e (MQA)
 *   o    = sum_e exp(l_e - M) e / (exp(z_h - M) + sum_e exp(l_e - M)),
 *          z_h = sink[h] (sink NULL -> no sink), M the running maximum
 *   lse  = log(exp(z_h) + sum_e exp(l_e))
 *   if rope_on_output, o's last rope_dims dims are rotated back by -t.
 *
 *   q     : [batch, Tq, H, d]
 *   kv    : [batch, N, d]     compressed entries as stored (normed + roped)
 *   idx   : [batch, Tq, k] int32 (CSA; entries outside [0, N) are skipped),
 *           NULL for HCA
 *   win   : [batch, W, d]     prepared window rows; position p is row
 *           (p - win_pos0) mod W, so rows filled in position order from
 *           win_pos0 and a ring of W rows (row p mod W, win_pos0 = 0, as a
 *           decode loop keeps it) are both accepted. The positions
 *           max(0, pos0 - w + 1) .. pos0 + Tq - 1 must fit: W >= their count;
 *           win_pos0 >= 0.
 *   sink  : [H] fp32 or NULL;  q_norm_w : [d] fp32 or NULL (gain 1)
 *   1 <= H <= CSKV_MAX_HEADS, d % 32 == 0, 32 <= d <= 512 (bf16) or
 *   CSKV_MAX_DIM (f32), w >= 1, rope_dims even <= d
 *   out   : [batch, Tq, H, d];  lse : [batch, Tq, H] fp32 or NULL
 */
int compressed_attn_prefill(int mode, const void* q, const void* kv, const int32_t* idx,
                            const void* win, int64_t win_pos0, int64_t W, const float* sink,
                            int batch, int64_t Tq, int64_t N, int64_t pos0, int m, int k, int w,
                            int H, int d, int apply_q_norm, const float* q_norm_w, float eps,
                            int rope_dims, float rope_base, float scale, int rope_on_output,
                            void* out, float* lse, int dtype, void* stream);

/*
 * compressed_attn_decode -- the same computation for a few new query tokens
 * against a long cache, split over the key list ("split-K"): each split
 * writes a partial (max, sum, weighted sum) to the workspace and a merge
 * kernel combines the splits in a fixed order. Arguments as in
 * compressed_attn_prefill, plus:
 *   n_splits  : 0 = choose from the shape (S = min(ceil(256 / (batch * Tq)),
 *               ceil(key tiles / 2), 256), a key tile being 32 keys); else
 *               1 .. 256 splits per query
 *   workspace : cskv_decode_workspace_size(...) bytes of device memory: the
 *               fp32 partials, batch * Tq * S * H * (d + 2) * 4 bytes when
 *               S > 1 and nothing (0 bytes, NULL allowed) when S = 1. With
 *               n_splits = 0 the size covers the largest automatic S.
 * Any n_splits gives the same result up to fp32 rounding of the merge.
 * cskv_decode_workspace_size returns 0 for arguments the call would reject.
 */
size_t cskv_decode_workspace_size(int batch, int64_t Tq, int H, int d, int n_splits);
int compressed_attn_decode(int mode, const void* q, const void* kv, const int32_t* idx,
                           const void* win, int64_t win_pos0, int64_t W, const float* sink,
                           int batch, int64_t Tq, int64_t N, int64_t pos0, int m, int k, int w,
                           int H, int d, int apply_q_norm, const float* q_norm_w, float eps,
                           int rope_dims, float rope_base, float scale, int rope_on_output,
                           int n_splits, void* workspace, size_t ws_bytes, void* out, float* lse,
                           int dtype, void* stream);

/*
 * compressed_attn_decode_noalloc -- compressed_attn_decode for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. There is no workspace argument;
 * the call itself allocates nothing (no hipMalloc / hipFree). The split
 * partials live in a static device buffer of CSKV_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends.
 *   n_splits : 0 = the automatic split count of compressed_attn_decode,
 *              lowered if need be so that the partials fit the buffer (down
 *              to one split, which needs none); an explicit 1 .. 256 whose
 *              partials (batch * Tq * n_splits * H * (d + 2) * 4 bytes) exceed
 *              the buffer returns CSKV_ERR_WORKSPACE before any launch.
 *   other arguments, limits and results as in compressed_attn_decode (bf16
 *   or f32; with the same split count the output is bit-identical).
 * Every call on one GPU shares that GPU's buffer: calls that overlap on one
 * GPU (other streams, other host threads) race and must be serialised by
 * the caller. The first call on a device looks the buffer's address up
 * (hipGetSymbolAddress); a failure there returns CSKV_ERR_HIP.
 */
#define CSKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int compressed_attn_decode_noalloc(int mode, const void* q, const void* kv, const int32_t* idx,
                                   const void* win, int64_t win_pos0, int64_t W, const float* sink,
                                   int batch, int64_t Tq, int64_t N, int64_t pos0, int m, int k, int w,
                                   int H, int d, int apply_q_norm, const float* q_norm_w, float eps,
                                   int rope_dims, float rope_base, float scale, int rope_on_output,
                                   int n_splits, void* out, float* lse, int dtype, void* stream);

/*
 * FP8 KV storage [PB §2.3.4 "Efficiency": KV storage FP8 for the non-RoPE
 * dims, BF16 for the RoPE dims]. A stored entry is the E4M3 codes of its
 * first d - rope_dims values (x * 2^-e, e the smallest integer with
 * max |x| <= 448 * 2^e, nearest code, ties to even) followed by its last
 * rope_dims values in bf16: d - rope_dims + 2 * rope_dims bytes, plus one fp32
 * scale 2^e. (d - rope_dims) % 16 == 0 and rope_dims % 8 == 0; the attention
 * entry points take rope_dims in {0, 16, 32, 64}.
 *
 * cskv_quantize_kv_fp8 -- x [batch, n, d] (bf16 or f32) to out [batch,
 *   out_ld, row bytes] and scales [batch, out_ld] fp32 (out_ld = 0: n); pass
 *   pointers offset to row r0 to append to a cache. scales 4-byte aligned.
 * compressed_attn_prefill_kv8 / compressed_attn_decode_kv8 -- the attention
 *   entry points with kv such a cache ([batch, N, row bytes]) and kv_scale
 *   [batch, N]; q, win and out are bf16. The loader widens each entry to
 *   bf16 exactly (E4M3 times a power of two is a bf16 value), so the result
 *   is the bf16 attention over the dequantised entries.
 *   compressed_attn_prefill_kv8 takes an optional workspace: for HCA (every
 *   query reads every visible entry) with workspace != NULL, the entries are
 *   widened once into it (bf16 [batch, N, d], 16-byte aligned,
 *   cskv_prefill_kv8_workspace_size bytes, else CSKV_ERR_WORKSPACE) and the
 *   bf16 kernels run on them; the result is bit-identical to the route
 *   without a workspace, which widens each gathered tile in LDS. CSA ignores
 *   the workspace (NULL allowed).
 * cskv_prefill_kv8_workspace_size -- batch * N * d * 2 for HCA, 0 for CSA or
 *   arguments the call would reject.
 */
int cskv_quantize_kv_fp8(const void* x, int batch, int64_t n, int d, int rope_dims, int dtype, uint8_t* out,
                         float* scales, int64_t out_ld, void* stream);
int compressed_attn_prefill_kv8(int mode, const void* q, const uint8_t* kv, const float* kv_scale,
                                const int32_t* idx, const void* win, int64_t win_pos0, int64_t W,
                                const float* sink, int batch, int64_t Tq, int64_t N, int64_t pos0, int m,
                                int k, int w, int H, int d, int apply_q_norm, const float* q_norm_w,
                                float eps, int rope_dims, float rope_base, float scale, int rope_on_output,
                                void* workspace, size_t ws_bytes, void* out, float* lse, void* stream);
size_t cskv_prefill_kv8_workspace_size(int mode, int batch, int64_t N, int d);
int compressed_attn_decode_kv8(int mode, const void* q, const uint8_t* kv, const float* kv_scale,
                               const int32_t* idx, const void* win, int64_t win_pos0, int64_t W,
                               const float* sink, int batch, int64_t Tq, int64_t N, int64_t pos0, int m,
                               int k, int w, int H, int d, int apply_q_norm, const float* q_norm_w,
                               float eps, int rope_dims, float rope_base, float scale, int rope_on_output,
                               int n_splits, void* workspace, size_t ws_bytes, void* out, float* lse,
                               void* stream);

/* ------------------------------------------------------------------------
 * Projections around the core attention ("Paper Breakdown: DeepSeek-V4",
 * section 4, CSA §2.3.1: low-rank indexer queries from a latent c_t^Q shared
 * with the attention queries; MQA core attention + grouped output projection;
 * HCA §2.3.2: the same grouped projection). The pages give no shapes; both
 * entry points take them as arguments. bf16 only (dtype CSKV_BF16), fp32
 * accumulation, bf16 results (round to nearest even).
 *
 * cskv_lowrank_proj -- out [T, n_out] = cq [T, r] @ W [r, n_out], all
 *   row-major. One call per projection: the attention queries (n_out = H * d,
 *   read as [T, H, d]) and the indexer queries (n_out = H_I * d_I). The query
 *   RMSNorm and RoPE are applied by the attention entry points. r a multiple
 *   of 64, n_out of 8; T = 0 is a no-op.
 * cskv_grouped_out_proj -- o [T, H, d] (the attention output) in G groups of
 *   H/G contiguous heads: mid [T, G, dg] with mid[t, g] = concat(o[t, h] for
 *   h in group g) @ Wg[g], Wg [G, (H/G) * d, dg]; then y [T, D] =
 *   mid[t] (as [G * dg]) @ Wo [G * dg, D]. mid is a caller buffer of T * G *
 *   dg bf16 values (it holds the rounded intermediate on return).
 *   (H/G) * d and G * dg multiples of 64, dg and D multiples of 8.
 * Pointers 16-byte aligned. Errors: CSKV_ERR_BAD_DTYPE for a dtype other than
 * CSKV_BF16, CSKV_ERR_BAD_SHAPE for sizes outside the above, CSKV_ERR_INVALID_ARG
 * for a null pointer, CSKV_ERR_MISALIGNED; all checked before any launch.
 */
int cskv_lowrank_proj(const void* cq, const void* W, void* out, int64_t T, int64_t r, int64_t n_out, int dtype,
                      void* stream);
int cskv_grouped_out_proj(const void* o, const void* Wg, const void* Wo, void* mid, void* y, int64_t T, int H,
                          int d, int G, int64_t dg, int64_t D, int dtype, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSKV_H_ */
