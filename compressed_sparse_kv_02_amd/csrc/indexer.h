// Internal interface between the lightning-indexer scoring (indexer.hip) and
// the per-query top-k selection (topk.hip): their shared argument block and
// the host-side launchers each file provides to the other's entry points.
#pragma once

#include "device_common.h"
#include "abi_common.h"

namespace cskv {

__device__ __forceinline__ int64_t visible_entries(int64_t t, int m, int64_t N) {
  const int64_t v = (t + 1) / m;
  return v < N ? v : N;
}

struct IdxArgs {
  const void* qI;
  const float* wI;
  const void* KI;
  const float* q_scale;  // FP8/FP4: [batch][Tq][HI] scale of each (query, head) row
  const float* k_scale;  // FP8/FP4: [batch][N] scale of each key row
  float* scores;  // [batch][rows_ws][ldS]
  int32_t* out;
  int64_t Tq, N, pos0, ldS, span;  // span: keys per workgroup (prefill scoring)
  int64_t row_waves;               // decode scoring: waves sharing one query row
  int64_t row0, nrows, rows_ws;  // query rows handled by this chunk
  int HI, dI, m, k;
  // two-kernel selection of few long rows (topk_part + topk_merge)
  uint8_t* sel_ws;     // per row: keys [CAP] u32, indices [CAP] i32, part records [MAX_PARTS] int4
  int64_t part_len;    // entries per part
  int kp;              // candidates kept per part
  // Block maxima: score_key of the largest score of each block of 32 entries of a row (0 when
  // the block holds no entry of the row), row r of the chunk at bm + (b * bm_rows + r) * bm_ld.
  // bm_fused: the one-query-per-workgroup scorer writes them as it stores the scores; otherwise
  // topk_blockmax derives them from the score rows. topk_bm_select reads them.
  uint32_t* bm;
  int64_t bm_ld, bm_rows;
  int bm_fused;
};

// Rows of up to BM_MAX_BLOCKS blocks of 32 entries can be selected through block maxima.
constexpr int BM_MAX_BLOCKS = 8192;

// Rows whose visible entries run from vmin to vmax (the first and last row of a launch) take the
// block-maxima route: every row has at least 2k blocks, so the k-th largest block maximum leaves a
// few k candidates rather than the whole row, and at most BM_MAX_BLOCKS.
inline bool bm_route(int64_t vmin, int64_t vmax, int k) {
  return ceil_div(vmin, (int64_t)32) >= 2 * (int64_t)k && ceil_div(vmax, (int64_t)32) <= BM_MAX_BLOCKS;
}


// ReLU on the bit pattern: for non-NaN x, max(bits(x), 0) as int32 is bits(max(x, 0))
// (negative floats, -0.0 included, are negative as int32). One VALU op, no NaN canonicalisation.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Largest of x over each 32-lane half of the wave, in every lane: quad swaps, the half-row and
// row mirrors (DPP), then a swap between rows 0-1 and 2-3.
__device__ __forceinline__ uint32_t max_key32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));  // 7 - lane (8s)
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));  // 15 - lane (16s)
  const auto sw = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return max(sw[0], sw[1]);
}


// Scores of rows [a.row0, a.row0 + a.nrows) into a.scores; bf16 takes qb
// queries per workgroup (8 for prefill, 1 for decode).
int launch_scores(IdxArgs& a, int batch, int qb, int dtype, hipStream_t st);

// Top-k of rows [a.row0, a.row0 + a.nrows) from a.scores into a.out; sel_ws
// (optional, sel_bytes long) enables the several-workgroups-per-row route.
int launch_select(IdxArgs& a, int batch, void* sel_ws, size_t sel_bytes, hipStream_t st);

// Score chunking shared by the bf16 and FP8 entry points: score row stride,
// rows per chunk, queries per scoring workgroup.
struct IdxPlan {
  int64_t ldS, rows_ws, qb;
};
IdxPlan plan_indexer(int batch, int64_t Tq, int64_t N, int dtype);

// Low-precision scoring (dtype CSKV_FP8: E4M3 codes, CSKV_FP4: E2M1 codes) of rows
// [a.row0, a.row0 + a.nrows) into a.scores (indexer_lowp.hip).
int launch_scores_lowp(IdxArgs& a, int batch, int qb, int dtype, hipStream_t st);

// Bytes of one row's selection workspace (the several-workgroups-per-row routes).
int64_t topk_sel_stride();

// Workspace bytes for the several-workgroups-per-row selection of `rows`
// rows of up to vmax entries; 0 when that route is not taken.
size_t split_ws_bytes(int64_t rows, int64_t vmax, int k);

}  // namespace cskv
