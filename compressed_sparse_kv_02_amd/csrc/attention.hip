// MQA core attention over compressed entries + sliding window + sink, gfx950.
//
// "Paper Breakdown: DeepSeek-V4": CSA §2.3.1 (MQA core attention over the
// top-k selected compressed entries plus an uncompressed sliding window),
// HCA §2.3.2 (dense attention over every visible compressed entry plus the
// same window), §2.3.3 (query RMSNorm, partial RoPE on the last 64 dims,
// learnable per-head sink logits). "Inside DeepSeek V4", "Local window":
// 128 recent uncompressed entries in every CSA and HCA layer.
//
// bf16 kernel: a workgroup takes QG consecutive queries (HCA prefill, whose
// neighbouring queries see the same compressed entries: QG = 2, or 4 with
// 17-32 heads of 512 dims) and
// HW waves of 16 heads per query.
//  * Each wave RMSNorms and rotates its 16 query rows in registers and keeps
//    them as bf16 B operands (Q^T); RoPE cos/sin are computed once per
//    workgroup into LDS (angles formed in fp64).
//  * The key list -- selected (CSA) or visible (HCA) compressed entries, then
//    window rows -- is gathered 32 rows at a time into a double-buffered LDS
//    tile; the next tile's loads overlap this tile's math, staged through
//    registers, or, in the CSA prefill build (two workgroups per CU), copied
//    straight into LDS (global_load_lds, one 1 KiB row per wave instruction),
//    which frees the 32 staging registers (the CSA index list is staged in
//    LDS first, so row addresses never wait on a global load). K = V: one tile serves both
//    products. Keys sit in LDS rows by a fixed permutation that keeps both
//    the K-operand reads and the transpose reads free of bank conflicts.
//  * S^T = K Q^T (v_mfma_f32_16x16x32_bf16) leaves each lane the logits of
//    one head for 8 keys, exactly the B operand P^T of O^T = V^T P^T.
//  * V^T comes straight from the row-major tile through gfx950's transpose
//    LDS read (ds_read_b64_tr_b16), so no register transposes are needed and
//    each accumulator lane owns 4 contiguous output dims of a single head:
//    per-head rescale, sink, normalisation and RoPE de-rotation are in-lane.
//  * The softmax reference only moves when a logit exceeds it by 2^8, so the
//    O rescale is almost never executed; the final normalisation uses the
//    same reference, so the result is unchanged.
//  * Split-K (decode): a split writes (reference, sum, unnormalised O) and a
//    merge kernel combines splits in a fixed order, adds the sink, de-rotates.
// fp32 kernel: plain vector-ALU online softmax, one workgroup per
// (query, head); it serves the fp32 mode.
#include <atomic>
#include <mutex>

#include "device_common.h"
#include "abi_common.h"

namespace cskv {

struct AttnArgs {
  const void* q;
  const void* kv;
  const int32_t* idx;
  const void* win;
  const float* sink;
  const float* q_norm_w;
  const float* kv_scale;  // FP8 KV storage: [batch][N] power-of-two scale of each entry
  void* out;
  float* lse;
  float* part_o;   // [batch*Tq][splits][H][D]
  float* part_ml;  // [batch*Tq][splits][H][2] (running max, sum; base-2 logits)
  int64_t Tq, N, pos0, win_pos0, W;
  int m, k, w, H, D, mode, apply_q_norm, rope_dims, rope_on_output, n_splits;
  float eps, rope_base, scale_log2;
  RopeTable rope;  // theta of the first rotary pairs (host fp64)
};

__device__ __forceinline__ int64_t visible_n(int64_t t, int m, int64_t N) {
  const int64_t v = (t + 1) / m;
  return v < N ? v : N;
}

// Row of the window buffer that holds position p: (p - win_pos0) mod W. A buffer
// filled in position order from win_pos0 and a ring of W rows (position p in row
// p mod W, win_pos0 = 0) are both read this way.
__device__ __forceinline__ int64_t win_row_of(const AttnArgs& a, int64_t p) {
  int64_t r = (p - a.win_pos0) % a.W;
  return r < 0 ? r + a.W : r;
}

// Key list of query (b, j): [0, n_comp) compressed (selected or visible), then window rows.
struct KeyList {
  const int32_t* idxrow;
  int64_t n_comp, n_tot, win_row0;  // win_row0: row of position max(0, t-w+1) in `win` (0 .. W-1)
};

__device__ __forceinline__ KeyList make_keys(const AttnArgs& a, int b, int64_t j) {
  KeyList L;
  const int64_t t = a.pos0 + j;
  if (a.mode == CSKV_MODE_CSA) {
    L.idxrow = a.idx + ((int64_t)b * a.Tq + j) * a.k;
    L.n_comp = a.k;
  } else {
    L.idxrow = nullptr;
    L.n_comp = visible_n(t, a.m, a.N);
  }
  int64_t lo = t - a.w + 1;
  if (lo < 0) lo = 0;
  L.n_tot = L.n_comp + (t - lo + 1);
  L.win_row0 = win_row_of(a, lo);
  return L;
}

// Element offset of key u's row, or -1 when the key is absent / skipped.
__device__ __forceinline__ int64_t key_row(const AttnArgs& a, const KeyList& L, int b, int64_t u) {
  if (u >= L.n_tot) return -1;
  if (u < L.n_comp) {
    int64_t s = u;
    if (L.idxrow) {
      s = L.idxrow[u];
      if (s < 0 || s >= a.N) return -1;
    }
    return ((int64_t)b * a.N + s) * a.D;
  }
  int64_t r = L.win_row0 + (u - L.n_comp);  // window rows wrap at W
  if (r >= a.W) r -= a.W;
  return -2 - (((int64_t)b * a.W + r) * a.D);  // window: encoded < -1
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// gfx950 LDS transpose read: within each group of 16 lanes, lane i receives the
// (i % 4)-th 16-bit element of the 8-byte reads of lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ v4i16 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
}

// LDS row of the tile that holds logical key L (0..31): key n of the first half in
// row 2n, key 16+n in row 2n+1. Row r of 1040 bytes starts at bank 4r of gfx950's
// 128 (measured: conflicts follow this model, with 32 lanes per pass for 16- and
// 8-byte reads). A K-operand read (lane (n, g): key n, 16 bytes at byte 16g) then
// covers 4-bank groups 2n + g, all 32 distinct in a pass of g = 0, 1; the transpose
// read of 32 lanes touches keys 4g + e, g = 0, 1, i.e. 8 even rows whose 32-byte
// pieces start 8 banks apart. Both are free of bank conflicts (the counters read 0).
__device__ __forceinline__ int key_row_of(int L) {
  return 2 * (L & 15) + (L >> 4);
}
// Inverse of key_row_of.
__device__ __forceinline__ int key_of_row(int r) {
  return (r >> 1) + 16 * (r & 1);
}

// Maximum / sum over the four 16-lane groups (lanes l, l^16, l^32, l^48) in every lane.
// SWAP: through gfx950's row swaps on the vector ALU, so the partner values never leave
// the register file and no LDS round trip sits in the softmax's dependency chain; each
// swap hands every lane its own value and its partner's, combined in either order (max
// and + commute), so the result has the same bits as the cross-lane reads of !SWAP,
// which need two fewer registers (kernels at the register limit keep them).
template <bool SWAP>
__device__ __forceinline__ float group4_max(float x) {
  if constexpr (SWAP) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
  } else {
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return fmaxf(x, __shfl_xor(x, 32, 64));
  }
}
template <bool SWAP>
__device__ __forceinline__ float group4_sum(float x) {
  if constexpr (SWAP) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
  } else {
    x += __shfl_xor(x, 16, 64);
    return x + __shfl_xor(x, 32, 64);
  }
}

// Logits of a query only grow the softmax reference when they exceed it by this
// much (log2 units): the O/l rescale is then almost never needed, and P <= 2^8.
constexpr float REF_SLACK = 8.0f;

// KVR >= 0: compressed entries stored as FP8 E4M3 codes of the first D - KVR dims (one
// power-of-two scale per entry) followed by the KVR RoPE dims in bf16; the loader widens
// them to bf16 rows in LDS (exact: E4M3 times a power of two is a bf16 value), so the rest
// of the kernel is unchanged. Window rows stay bf16. KVR < 0: bf16 entries.
// OCC = 2 asks the compiler for two workgroups per CU (at most 256 registers per lane):
// CSA prefill then has two gathers in flight per CU. Its tiles are copied straight into
// LDS, so it needs no staging registers (no spills) and affords the row-swap softmax.
template <int D, int HW, int QG, int KVR, int OCC = 1>
__global__ __launch_bounds__(HW * QG * 64, OCC) void attn_mfma(AttnArgs a) {
  constexpr bool KV8 = KVR >= 0;
  constexpr int NW = HW * QG;
  constexpr int NT = NW * 64;
  constexpr int ROWE = D + 8;        // padded LDS row, bf16 elements
  constexpr int KS = D / 32;         // k-steps of S^T = K Q^T
  constexpr int NTILE = D / 16;      // 16-dim output tiles of O^T = V^T P^T
  constexpr int CPR = D / 8;         // 16-byte chunks per key row
  constexpr int TPK = NT / 32;       // loader threads per key row
  static_assert(CPR % TPK == 0, "loader mapping");
  constexpr int CPT = CPR / TPK;     // chunks per loader thread per tile
  constexpr int MAXPAIRS = D / 2;
  // One query per workgroup: its query loads are issued before anything else, so that their
  // latency overlaps the index and rotary staging and the first key tile. With two queries the
  // register budget is too tight for that, and they are loaded right before use.
  constexpr bool QEARLY = QG == 1;
  // double-buffered key tiles as two separately declared arrays: with direct-to-LDS copies
  // the compiler then sees that a copy into one buffer never feeds reads of the other
  __shared__ __attribute__((aligned(16))) uint16_t kt0[32 * ROWE], kt1[32 * ROWE];
  __shared__ __attribute__((aligned(16))) int kvq0[32], kvq1[32];  // logical key -> bit q: valid for query q
  __shared__ float rope_cs[QG][MAXPAIRS][2];
  __shared__ __attribute__((aligned(16))) float qw_s[D];  // query RMSNorm weights
  __shared__ int idx_s[CSKV_MAX_TOPK];  // CSA: the query's selected entries, staged once

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave-derived values scalar
  const int n = lane & 15, g = lane >> 4;
  const int qi = wave / HW, hw = wave % HW;
  const int64_t nqb = (a.Tq + QG - 1) / QG;
  const int64_t flat = (int64_t)gridDim.x - 1 - blockIdx.x;  // later (longer) rows first
  const int b = (int)(flat / nqb);
  const int64_t jb = (flat % nqb) * QG;
  const int64_t jl = (jb + QG < a.Tq ? jb + QG : a.Tq) - 1;  // last query of the tile
  const int64_t j = jb + qi < a.Tq ? jb + qi : jl;
  const bool qvalid = jb + qi < a.Tq;
  const int h = hw * 16 + n;
  const bool hvalid = qvalid && h < a.H;
  const int split = blockIdx.y;
  const bool csa = a.mode == CSKV_MODE_CSA;

  // Key list shared by the tile's queries: [0, n_comp) compressed, then window positions lo .. t_last.
  const int64_t t_first = a.pos0 + jb, t_last = a.pos0 + jl;
  const int32_t* idxrow = csa ? a.idx + ((int64_t)b * a.Tq + jb) * a.k : nullptr;
  const int64_t n_comp = csa ? a.k : visible_n(t_last, a.m, a.N);
  int64_t lo = t_first - a.w + 1;
  if (lo < 0) lo = 0;
  const int64_t n_tot = n_comp + (t_last - lo + 1);
  const int64_t nblk = (n_tot + 31) / 32;
  const int64_t bps = (nblk + a.n_splits - 1) / a.n_splits;
  const int64_t blk0 = (int64_t)split * bps;
  const int64_t blk1 = blk0 + bps < nblk ? blk0 + bps : nblk;

  // query rows: 16 bytes per lane per k-step, all in flight together
  const uint16_t* qp = (const uint16_t*)a.q + (((int64_t)b * a.Tq + j) * a.H + (hvalid ? h : 0)) * D;
  u32x4 qraw[KS];
  auto load_q = [&]() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = *reinterpret_cast<const u32x4*>(qp + ks * 32 + 8 * g);
  };
  if constexpr (QEARLY) load_q();

  // Stage the selected-entry list in LDS so that row addresses never wait on a global load.
  if (csa)
    for (int i = tid; i < a.k; i += NT) idx_s[i] = idxrow[i];
  // Query RMSNorm weights (1 when absent), read back as vectors in the query prologue.
  for (int i = tid; i < D; i += NT) qw_s[i] = a.q_norm_w ? a.q_norm_w[i] : 1.f;
  // Rotary cos/sin of every pair at each query's position, once per workgroup.
  const int npairs = a.rope_dims / 2;
  for (int i = tid; i < QG * npairs; i += NT) {
    const int q = i / npairs, pj = i % npairs;
    const int64_t jq = jb + q < a.Tq ? jb + q : jl;
    rope_cos_sin(a.pos0 + jq, pj, a.rope_dims, a.rope_base, &rope_cs[q][pj][0], &rope_cs[q][pj][1]);
  }
  __syncthreads();

  bf16x8 qb[KS];  // query prologue output: bf16 B operands of S^T (lane: head n, dims 32ks+8g..+7)
  float m_ref = -INFINITY, l_run = 0.f;  // per head n, identical in the four lane groups
  f32x4 o[NTILE];                        // O^T tile tt: lane holds dims 16tt+4g+i of head n
#pragma unroll
  for (int tt = 0; tt < NTILE; ++tt) o[tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- gather loader: thread -> (key row kr, chunks c0 + TPK*i)
  const int kr = tid / TPK, c0 = tid % TPK;
  const uint16_t* kvb = (const uint16_t*)a.kv + (int64_t)b * a.N * D;
  constexpr int nope8 = (D - (KV8 ? KVR : 0)) / 8;      // KV8: 16-byte LDS chunks that hold FP8 codes
  constexpr int64_t rb8 = (D - (KV8 ? KVR : 0)) + 2 * (KV8 ? KVR : 0);  // KV8: bytes per stored entry
  const uint8_t* kv8b = (const uint8_t*)a.kv + (int64_t)b * a.N * rb8;
  const int64_t wbase = (int64_t)b * a.W;
  const int64_t wr_lo = win_row_of(a, lo);  // window row of position lo; rows wrap at W
  // per-query bounds of the tile's queries, for the loader's validity bits
  int64_t vis_q[QG], t_q[QG];
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    t_q[q] = a.pos0 + (jb + q < a.Tq ? jb + q : jl);
    vis_q[q] = csa ? 0 : visible_n(t_q[q], a.m, a.N);
  }
  // register staging of one key row's share: chunks, validity bits and (KV8) the entry's scale
  // and whether it is an FP8 row (not a window row or padding)
  struct Stage {
    u32x4 v[CPT];
    int ok;
    float sc;
    bool is8;
  };
  // Loader thread: key u = blk*32 + kr of the key list goes to LDS row kr; its validity
  // bits (bit q: query q of the tile may attend to it) go to the logical slot of row kr.
  auto gload = [&](int64_t blk, Stage& st) {
    const int64_t u = blk * 32 + kr;
    const uint16_t* src = nullptr;
    const uint8_t* src8 = nullptr;
    int ok = 0;
    if (u < n_comp) {
      const int64_t s_ = csa ? (int64_t)idx_s[u] : u;
      if (s_ >= 0 && s_ < a.N) {
        if constexpr (KV8) {
          src8 = kv8b + s_ * rb8;
          st.sc = a.kv_scale[(int64_t)b * a.N + s_];
        } else {
          src = kvb + s_ * D;
        }
#pragma unroll
        for (int q = 0; q < QG; ++q) ok |= (csa || s_ < vis_q[q]) ? (1 << q) : 0;
      }
    } else if (u < n_tot) {
      const int64_t pos = lo + (u - n_comp);
      int64_t wr = wr_lo + (u - n_comp);
      if (wr >= a.W) wr -= a.W;
      src = (const uint16_t*)a.win + (wbase + wr) * D;
#pragma unroll
      for (int q = 0; q < QG; ++q) ok |= (pos >= t_q[q] - a.w + 1 && pos <= t_q[q]) ? (1 << q) : 0;
    }
    // is8 depends on addresses only: selecting on the loaded scale here would wait for that
    // load before the current tile's compute and expose the full gather latency.
    st.is8 = KV8 && src8 != nullptr;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int oc = c0 + TPK * i;  // 16-byte chunk of the bf16 row: dims 8*oc .. +8
      u32x4 v = {0u, 0u, 0u, 0u};
      if (KV8 && src8) {
        if (oc < nope8) {
          const uint2 c = *reinterpret_cast<const uint2*>(src8 + 8 * oc);  // 8 E4M3 codes
          v = u32x4{c.x, c.y, 0u, 0u};
        } else {
          v = *reinterpret_cast<const u32x4*>(src8 + 8 * nope8 + 16 * (oc - nope8));
        }
      } else if (src) {
        v = *reinterpret_cast<const u32x4*>(src + oc * 8);
      }
      st.v[i] = v;
    }
    st.ok = ok;
  };
  auto lstore = [&](uint16_t* ktb, int* kvqb, const Stage& st) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int oc = c0 + TPK * i;
      u32x4 v = st.v[i];
      if (KV8 && st.is8 && oc < nope8) {  // widen 8 codes to bf16 (times the power-of-two scale)
        const uint32_t c01 = v.x, c23 = v.y;
        v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c01, st.sc, false));
        v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c01, st.sc, true));
        v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c23, st.sc, false));
        v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c23, st.sc, true));
      }
      *reinterpret_cast<u32x4*>(&ktb[kr * ROWE + oc * 8]) = v;
    }
    if (c0 == 0) kvqb[key_of_row(kr)] = st.ok;
  };
  // bf16 entries of 512 dims: one key row is one 1 KiB wave copy straight into LDS
  // (global_load_lds_dwordx4, lane l -> bytes 16 l .. 16 l + 15 of the row), so no staging
  // registers. Wave w copies LDS rows w, w + NW, ...; an absent key copies a window row
  // (finite data; its validity bits are 0, so its weight is exactly 0).
  constexpr bool DMA = KVR < 0 && D == 512 && OCC == 2;
  constexpr bool DMA8 = KV8 && D == 512 && OCC == 2;  // see dma8 below
  auto dma = [&](int64_t blk, uint16_t* ktb, int* kvqb) {
#pragma unroll
    for (int i = 0; i < 32 / NW; ++i) {
      const int rr = wave + i * NW;
      const int L = key_of_row(rr);
      const int64_t u = blk * 32 + L;
      const uint16_t* src = (const uint16_t*)a.win + wbase * D;
      int ok = 0;
      if (u < n_comp) {
        const int64_t s_ = csa ? (int64_t)idx_s[u] : u;
        if (s_ >= 0 && s_ < a.N) {
          src = kvb + s_ * D;
#pragma unroll
          for (int q = 0; q < QG; ++q) ok |= (csa || s_ < vis_q[q]) ? (1 << q) : 0;
        }
      } else if (u < n_tot) {
        const int64_t pos = lo + (u - n_comp);
        int64_t wr = wr_lo + (u - n_comp);
        if (wr >= a.W) wr -= a.W;
        src = (const uint16_t*)a.win + (wbase + wr) * D;
#pragma unroll
        for (int q = 0; q < QG; ++q) ok |= (pos >= t_q[q] - a.w + 1 && pos <= t_q[q]) ? (1 << q) : 0;
      }
      __builtin_amdgcn_global_load_lds((const void*)(src + lane * 8),
                                       (__attribute__((address_space(3))) void*)(&ktb[rr * ROWE]), 16, 0, 0);
      if (lane == 0) kvqb[L] = ok;
    }
  };
  // every copy of the tile has landed and every wave is done with the other buffer; the
  // explicit full wait is visible to the compiler's wait tracking (one in inline asm is not)
  auto wait_barrier = [&]() {
    if constexpr (DMA || DMA8) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // KV8 entries at two workgroups per CU: each stored entry (D - KVR codes, then the KVR RoPE
  // dims in bf16) is copied straight into LDS at byte D - KVR of its row, which puts the RoPE
  // dims where the bf16 row has them; the wave that copied a row then widens its codes to bf16
  // in front of them (expand8). Window rows and absent keys are copied as whole bf16 rows. Lane
  // l widens the wave's row l / 8 (chunks of 8 codes l % 8, l % 8 + 8, ...) and loads that
  // row's scale with the copies. A wave's LDS operations run in order, so its reads of the
  // codes precede its overlapping writes (other lanes' bytes) without a barrier; wave-scope
  // fences keep the compiler from moving them across each other.
  constexpr int NCH8 = (D - (KV8 ? KVR : 0)) / 8;  // 8-code chunks per stored entry
  constexpr int CPT8 = NCH8 >= 8 ? (NCH8 + 7) / 8 : 1;
  bool exp8 = false;  // DMA8: this thread's expansion row holds codes
  float sc8 = 0.f;    // DMA8: and its scale
  auto dma8 = [&](int64_t blk, uint16_t* ktb, int* kvqb) {
    static_assert(!DMA8 || (32 / NW == 8 && D == 512), "expansion mapping: 8 lanes per row, 8 rows per wave");
#pragma unroll
    for (int i = 0; i < 32 / NW; ++i) {
      const int rr = wave + i * NW;
      const int L = key_of_row(rr);
      const int64_t u = blk * 32 + L;
      const uint16_t* src = (const uint16_t*)a.win + wbase * D;
      const uint8_t* src8 = nullptr;
      int ok = 0;
      if (u < n_comp) {
        const int64_t s_ = csa ? (int64_t)idx_s[u] : u;
        if (s_ >= 0 && s_ < a.N) {
          src8 = kv8b + s_ * rb8;
#pragma unroll
          for (int q = 0; q < QG; ++q) ok |= (csa || s_ < vis_q[q]) ? (1 << q) : 0;
        }
      } else if (u < n_tot) {
        const int64_t pos = lo + (u - n_comp);
        int64_t wr = wr_lo + (u - n_comp);
        if (wr >= a.W) wr -= a.W;
        src = (const uint16_t*)a.win + (wbase + wr) * D;
#pragma unroll
        for (int q = 0; q < QG; ++q) ok |= (pos >= t_q[q] - a.w + 1 && pos <= t_q[q]) ? (1 << q) : 0;
      }
      if (src8) {
        if (lane * 16 < rb8)
          __builtin_amdgcn_global_load_lds(
              (const void*)(src8 + 16 * lane),
              (__attribute__((address_space(3))) void*)((uint8_t*)&ktb[rr * ROWE] + (D - KVR)), 16, 0, 0);
      } else {
        __builtin_amdgcn_global_load_lds((const void*)(src + lane * 8),
                                         (__attribute__((address_space(3))) void*)(&ktb[rr * ROWE]), 16, 0, 0);
      }
      if (lane == 0) kvqb[L] = ok;
    }
    {  // the scale of this lane's expansion row
      const int64_t u = blk * 32 + key_of_row(wave + (lane >> 3) * NW);
      exp8 = false;
      if (u < n_comp) {
        const int64_t s_ = csa ? (int64_t)idx_s[u] : u;
        if (s_ >= 0 && s_ < a.N) {
          exp8 = true;
          sc8 = a.kv_scale[(int64_t)b * a.N + s_];
        }
      }
    }
  };
  auto expand8 = [&](uint16_t* ktb) {
    uint8_t* rowb = (uint8_t*)&ktb[(wave + (lane >> 3) * NW) * ROWE];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    uint2 cd[CPT8];
#pragma unroll
    for (int i = 0; i < CPT8; ++i) {
      const int c = (tid & 7) + 8 * i;
      cd[i] = (exp8 && c < NCH8) ? *reinterpret_cast<const uint2*>(rowb + (D - KVR) + 8 * c) : uint2{0u, 0u};
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int i = 0; i < CPT8; ++i) {
      const int c = (tid & 7) + 8 * i;
      if (exp8 && c < NCH8) {
        u32x4 v;
        v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cd[i].x, sc8, false));
        v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cd[i].x, sc8, true));
        v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cd[i].y, sc8, false));
        v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cd[i].y, sc8, true));
        *reinterpret_cast<u32x4*>(rowb + 16 * c) = v;
      }
    }
  };

  // one key tile: S^T, online softmax, O^T update, from buffer (ktb, kvqb)
  auto tile = [&](const uint16_t* ktb, const int* kvqb) {
    // S^T = K Q^T: s0 -> keys 4g+i, s1 -> keys 16+4g+i; column = head n
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* kp = &ktb[key_row_of(n) * ROWE + 8 * g];  // logical key n; 16+n is the next row
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kp + ks * 32);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kp + ROWE + ks * 32);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb[ks], s1, 0, 0, 0);
    }
    const int4 d0 = *reinterpret_cast<const int4*>(&kvqb[4 * g]);
    const int4 d1 = *reinterpret_cast<const int4*>(&kvqb[16 + 4 * g]);
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    // masking only where some key of the tile is invalid for this wave's query (tile edges)
    const int vall = d0.x & d0.y & d0.z & d0.w & d1.x & d1.y & d1.z & d1.w;
    if (__ballot(((vall >> qi) & 1) == 0) != 0) {
      sv[0] = ((d0.x >> qi) & 1) ? sv[0] : -INFINITY;
      sv[1] = ((d0.y >> qi) & 1) ? sv[1] : -INFINITY;
      sv[2] = ((d0.z >> qi) & 1) ? sv[2] : -INFINITY;
      sv[3] = ((d0.w >> qi) & 1) ? sv[3] : -INFINITY;
      sv[4] = ((d1.x >> qi) & 1) ? sv[4] : -INFINITY;
      sv[5] = ((d1.y >> qi) & 1) ? sv[5] : -INFINITY;
      sv[6] = ((d1.z >> qi) & 1) ? sv[6] : -INFINITY;
      sv[7] = ((d1.w >> qi) & 1) ? sv[7] : -INFINITY;
    }
    // sv holds raw dot products; base-2 logits are sv * scale_log2 (> 0, so the maximum commutes)
    float mb = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mb = group4_max<OCC == 1 || DMA || DMA8>(mb) * a.scale_log2;
    // lazy reference: move it only when a logit exceeds it by REF_SLACK
    const bool upd = mb > m_ref + REF_SLACK;
    float alpha = 1.f;
    if (upd) {
      alpha = __builtin_amdgcn_exp2f(m_ref - mb);  // 0 when the reference was -inf
      m_ref = mb;
    }
    float p[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // v_exp_f32 directly: arguments are <= REF_SLACK, and a result below the normal
      // range (a weight under 2^-126 of the largest) flushes to zero
      p[i] = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], a.scale_log2, -m_ref));
      ps += p[i];
    }
    ps = group4_sum<OCC == 1 || DMA || DMA8>(ps);
    l_run = l_run * alpha + ps;
    if (__ballot(upd) != 0) {
#pragma unroll
      for (int tt = 0; tt < NTILE; ++tt) o[tt] *= alpha;
    }
    u32x4 pp;
    pp[0] = pack_bf16x2(p[0], p[1]);
    pp[1] = pack_bf16x2(p[2], p[3]);
    pp[2] = pack_bf16x2(p[4], p[5]);
    pp[3] = pack_bf16x2(p[6], p[7]);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pp);

    // O^T += V^T P^T: A = V^T via transpose reads (lane n of group g: keys 4g+e / 16+4g+e for
    // e = n/4, dims 16tt + 4(n%4) .. +3), B = P^T already in this lane (head n, 8 keys).
    const uint16_t* vp0 = &ktb[key_row_of(4 * g + (n >> 2)) * ROWE + 4 * (n & 3)];
    const uint16_t* vp1 = vp0 + ROWE;
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) {
      const v4i16 lo4 = lds_read_tr16(vp0 + 16 * tt);
      const v4i16 hi4 = lds_read_tr16(vp1 + 16 * tt);
      const v4i16 av[2] = {lo4, hi4};
      o[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb, o[tt], 0, 0, 0);
    }
  };
  // ---- query prologue: RMSNorm, RoPE at t -> qb
  auto query_prologue = [&]() {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (!hvalid) qraw[ks] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = __uint_as_float(qraw[ks][e] << 16), x1 = __uint_as_float(qraw[ks][e] & 0xffff0000u);
        ss += x0 * x0;
        ss += x1 * x1;
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = a.apply_q_norm ? rsqrtf(ss / (float)D + a.eps) : 1.f;
    const int rstart = D - a.rope_dims;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&qw_s[ks * 32 + 8 * g]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&qw_s[ks * 32 + 8 * g + 4]);
      const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(qraw[ks][e] << 16) * (inv * wv[2 * e]);
        x[2 * e + 1] = __uint_as_float(qraw[ks][e] & 0xffff0000u) * (inv * wv[2 * e + 1]);
      }
      if (a.rope_dims > 0 && ks * 32 + 8 * g + 8 > rstart) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int dim = ks * 32 + 8 * g + e;
          if (dim >= rstart) {
            const float cs = rope_cs[qi][(dim - rstart) >> 1][0], sn = rope_cs[qi][(dim - rstart) >> 1][1];
            const float x0 = x[e], x1 = x[e + 1];
            x[e] = x0 * cs - x1 * sn;
            x[e + 1] = x0 * sn + x1 * cs;
          }
        }
      }
      u32x4 pk;
      pk[0] = pack_bf16x2(x[0], x[1]);
      pk[1] = pack_bf16x2(x[2], x[3]);
      pk[2] = pack_bf16x2(x[4], x[5]);
      pk[3] = pack_bf16x2(x[6], x[7]);
      qb[ks] = __builtin_bit_cast(bf16x8, pk);
    }
  };
  if constexpr (DMA8) {
    // tile pairs as in the bf16 route below; each wave widens its rows of the next tile once
    // its own copies have landed, before the barrier that hands the tile over
    if constexpr (!QEARLY) load_q();
    if (blk0 < blk1) dma8(blk0, kt0, kvq0);
    query_prologue();
    if (blk0 < blk1) {
      __builtin_amdgcn_s_waitcnt(0);
      expand8(kt0);
    }
    __syncthreads();
    for (int64_t blk = blk0; blk < blk1; blk += 2) {
      if (blk + 1 < blk1) dma8(blk + 1, kt1, kvq1);
      tile(kt0, kvq0);
      if (blk + 1 < blk1) {
        __builtin_amdgcn_s_waitcnt(0);
        expand8(kt1);
      }
      __syncthreads();
      if (blk + 1 < blk1) {
        if (blk + 2 < blk1) dma8(blk + 2, kt0, kvq0);
        tile(kt1, kvq1);
        if (blk + 2 < blk1) {
          __builtin_amdgcn_s_waitcnt(0);
          expand8(kt0);
        }
        __syncthreads();
      }
    }
  } else if constexpr (DMA) {
    // the first tile's copies are in flight while the queries are prepared
    if constexpr (!QEARLY) load_q();
    if (blk0 < blk1) dma(blk0, kt0, kvq0);
    query_prologue();
    wait_barrier();
    // tile pairs: buffer 0 holds the even tiles of the range, buffer 1 the odd ones
    for (int64_t blk = blk0; blk < blk1; blk += 2) {
      if (blk + 1 < blk1) dma(blk + 1, kt1, kvq1);
      tile(kt0, kvq0);
      wait_barrier();
      if (blk + 1 < blk1) {
        if (blk + 2 < blk1) dma(blk + 2, kt0, kvq0);
        tile(kt1, kvq1);
        wait_barrier();
      }
    }
  } else {
    // register-staged: the next tile's rows are loaded into registers during this tile (the
    // first one while the queries are prepared)
    Stage st;
    if constexpr (QEARLY) {
      if (blk0 < blk1) gload(blk0, st);
      query_prologue();
    } else {
      load_q();
      query_prologue();
      if (blk0 < blk1) gload(blk0, st);
    }
    if (blk0 < blk1) lstore(kt0, kvq0, st);
    __syncthreads();
    for (int64_t blk = blk0; blk < blk1; ++blk) {
      const bool odd = ((blk - blk0) & 1) != 0;
      if (blk + 1 < blk1) gload(blk + 1, st);
      tile(odd ? kt1 : kt0, odd ? kvq1 : kvq0);
      if (blk + 1 < blk1) lstore(odd ? kt0 : kt1, odd ? kvq0 : kvq1, st);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds O[head n][16tt + 4g + i]
  if (!qvalid) return;  // uniform for the wave
  const int64_t row = (int64_t)b * a.Tq + j;
  if (a.n_splits > 1) {
    if constexpr (D == 512 && NW <= 4) {
      // fp32 partials through LDS as whole rows too, in two halves of 256 dims (1 KiB each)
      uint8_t* reg = (uint8_t*)(wave < 2 ? kt0 : kt1) + (wave & 1) * 16 * (D * 2 + 16);
      float* pw = a.part_o + ((row * a.n_splits + split) * a.H + hw * 16) * (int64_t)D + 4 * lane;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (half) __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the first half's reads precede
#pragma unroll
        for (int tt = 0; tt < NTILE / 2; ++tt)
          *reinterpret_cast<f32x4*>(reg + n * (D * 2 + 16) + 64 * tt + 16 * g) = o[half * (NTILE / 2) + tt];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(reg + i * (D * 2 + 16) + 16 * lane);
          if (hw * 16 + i < a.H) *reinterpret_cast<f32x4*>(pw + (int64_t)i * D + half * (D / 2)) = v;
        }
      }
    } else {
      if (!hvalid) return;
      float* po = a.part_o + ((row * a.n_splits + split) * a.H + h) * (int64_t)D + 4 * g;
#pragma unroll
      for (int tt = 0; tt < NTILE; ++tt) *reinterpret_cast<f32x4*>(po + 16 * tt) = o[tt];
    }
    if (g == 0 && hvalid) {
      float* pm = a.part_ml + ((row * a.n_splits + split) * a.H + h) * 2;
      pm[0] = m_ref;
      pm[1] = l_run;
    }
    return;
  }
  const float z = (a.sink && hvalid) ? a.sink[h] * 1.4426950408889634f : -INFINITY;
  const float M = fmaxf(m_ref, z);
  const float em = m_ref == -INFINITY ? 0.f : exp2f(m_ref - M);
  const float lt = l_run * em + (z == -INFINITY ? 0.f : exp2f(z - M));
  const float fac = lt > 0.f ? em / lt : 0.f;
  if (a.lse && g == 0 && hvalid) a.lse[row * a.H + h] = (M + log2f(lt)) * 0.6931471805599453f;
  const int rstart = D - a.rope_dims;
  // normalised, de-rotated bf16 values of dims 16tt + 4g .. + 3 of head n
  auto out4 = [&](int tt) {
    float v[4] = {o[tt][0] * fac, o[tt][1] * fac, o[tt][2] * fac, o[tt][3] * fac};
    const int d0 = 16 * tt + 4 * g;
    if (a.rope_on_output && a.rope_dims > 0 && d0 >= rstart) {
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float cs = rope_cs[qi][(d0 + e - rstart) >> 1][0];
        const float sn = -rope_cs[qi][(d0 + e - rstart) >> 1][1];  // rotate back by -t
        const float x0 = v[e], x1 = v[e + 1];
        v[e] = x0 * cs - x1 * sn;
        v[e + 1] = x0 * sn + x1 * cs;
      }
    }
    return uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  };
  if constexpr (D == 512 && NW <= 4) {
    // Through LDS, so that each store instruction writes one whole 1 KiB head row (a lane's
    // own values cover 32-byte pieces of 16 rows): wave w stages its 16 head rows (padded to
    // 1040 bytes) in the tile buffers, which every wave has finished with (the loop ended on a
    // barrier); the regions of different waves are disjoint, so only wave-scope ordering is
    // needed.
    static_assert(2 * 16 * (D * 2 + 16) == 2 * 32 * ROWE, "four waves' rows fill the two tile buffers");
    uint8_t* reg = (uint8_t*)(wave < 2 ? kt0 : kt1) + (wave & 1) * 16 * (D * 2 + 16);
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) *reinterpret_cast<uint2*>(reg + n * (D * 2 + 16) + 32 * tt + 8 * g) = out4(tt);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    uint16_t* ob = (uint16_t*)a.out + (row * a.H + hw * 16) * (int64_t)D + 8 * lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(reg + i * (D * 2 + 16) + 16 * lane);
      if (hw * 16 + i < a.H) *reinterpret_cast<u32x4*>(ob + (int64_t)i * D) = v;
    }
  } else {
    if (!hvalid) return;
    uint16_t* op = (uint16_t*)a.out + (row * a.H + h) * (int64_t)D + 4 * g;
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) *reinterpret_cast<uint2*>(op + 16 * tt) = out4(tt);
  }
}

// Merge split partials in split order, add the sink, normalise, de-rotate. One workgroup per
// (query, head): thread s reads split s's (max, sum), the maximum and the weighted sum are
// block reductions in a fixed order, and each thread sums its two output dims over the splits
// with eight partial loads in flight.
template <typename T>
__global__ __launch_bounds__(256) void attn_merge(AttnArgs a) {
  __shared__ float wsplit[256];
  __shared__ float red[4];
  __shared__ float scal[2];
  const int64_t row = blockIdx.x;  // b*Tq + j
  const int h = blockIdx.y;
  const int D = a.D;
  const int S = a.n_splits;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t j = row % a.Tq;
  const int64_t t = a.pos0 + j;
  const float* pm = a.part_ml + (row * S * a.H) * 2;
  const float z = a.sink ? a.sink[h] * 1.4426950408889634f : -INFINITY;
  float ms = -INFINITY, ls = 0.f;
  if (tid < S) {
    ms = pm[(tid * a.H + h) * 2];
    ls = pm[(tid * a.H + h) * 2 + 1];
  }
  float M = wave_max(ms);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), z);
  const float w = (tid < S && ms != -INFINITY) ? exp2f(ms - M) : 0.f;
  wsplit[tid] = w;
  float lw = wave_sum(w * ls);
  __syncthreads();  // red[] read above by every thread before it is reused
  if (lane == 0) red[wave] = lw;
  __syncthreads();
  if (tid == 0) {
    const float lt = ((red[0] + red[1]) + (red[2] + red[3])) + (z == -INFINITY ? 0.f : exp2f(z - M));
    scal[0] = lt > 0.f ? 1.f / lt : 0.f;
    if (a.lse) a.lse[row * a.H + h] = (M + log2f(lt)) * 0.6931471805599453f;
  }
  __syncthreads();
  const float inv = scal[0];
  const int rstart = D - a.rope_dims;
  for (int d = 2 * tid; d < D; d += 2 * blockDim.x) {
    const float* po = a.part_o + (row * S * a.H + h) * (int64_t)D + d;
    const int64_t sstride = (int64_t)a.H * D;
    float x0 = 0.f, x1 = 0.f;
    int s = 0;
    for (; s + 8 <= S; s += 8) {
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float2*>(po + (s + u) * sstride);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        x0 += v[u].x * wsplit[s + u];
        x1 += v[u].y * wsplit[s + u];
      }
    }
    for (; s < S; ++s) {
      const float2 v = *reinterpret_cast<const float2*>(po + s * sstride);
      x0 += v.x * wsplit[s];
      x1 += v.y * wsplit[s];
    }
    x0 *= inv;
    x1 *= inv;
    if (a.rope_on_output && a.rope_dims > 0 && d >= rstart) {
      float cs, sn;
      rope_cos_sin_t(a.rope, -t, (d - rstart) >> 1, a.rope_dims, a.rope_base, &cs, &sn);
      const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
    }
    T* op = (T*)a.out + (row * a.H + h) * (int64_t)D + d;
    Elem<T>::store(op, 0, x0);
    Elem<T>::store(op, 1, x1);
  }
}

// fp32 mode: one workgroup per (query, head), vector ALUs, online softmax over 256-key chunks.
__global__ __launch_bounds__(256) void attn_f32(AttnArgs a) {
  extern __shared__ float sh[];
  float* qs = sh;                 // [D]
  float* ps = qs + a.D;           // [256]
  float* red = ps + 256;          // [8]
  int64_t* rows = reinterpret_cast<int64_t*>(red + 8);  // [256]
  const int D = a.D, tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int b = (int)(row / a.Tq);
  const int64_t j = row % a.Tq;
  const int h = blockIdx.y;
  const int64_t t = a.pos0 + j;
  const float* qp = (const float*)a.q + (row * a.H + h) * (int64_t)D;
  auto block_sum = [&](float v) {
    v = wave_sum(v);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    float tot = 0.f;
    for (int q = 0; q < 4; ++q) tot += red[q];
    return tot;
  };
  auto block_max = [&](float v) {
    v = wave_max(v);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    float tot = -INFINITY;
    for (int q = 0; q < 4; ++q) tot = fmaxf(tot, red[q]);
    return tot;
  };
  float ss = 0.f;
  for (int d = tid; d < D; d += 256) {
    const float x = qp[d];
    qs[d] = x;
    ss += x * x;
  }
  ss = block_sum(ss);
  const float inv = a.apply_q_norm ? rsqrtf(ss / (float)D + a.eps) : 1.f;
  for (int d = tid; d < D; d += 256) qs[d] *= inv * (a.q_norm_w ? a.q_norm_w[d] : 1.f);
  __syncthreads();
  const int rstart = D - a.rope_dims;
  for (int d = rstart + 2 * tid; a.rope_dims > 0 && d < D; d += 512) {
    float cs, sn;
    rope_cos_sin_t(a.rope, t, (d - rstart) >> 1, a.rope_dims, a.rope_base, &cs, &sn);
    const float x0 = qs[d], x1 = qs[d + 1];
    qs[d] = x0 * cs - x1 * sn;
    qs[d + 1] = x0 * sn + x1 * cs;
  }
  __syncthreads();

  const KeyList L = make_keys(a, b, j);
  const float* kvb = (const float*)a.kv;
  const float* wnb = (const float*)a.win;
  constexpr int MAXD = CSKV_MAX_DIM / 256;
  float acc[MAXD];
  for (int i = 0; i < MAXD; ++i) acc[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int64_t base = 0; base < L.n_tot; base += 256) {
    const int64_t u = base + tid;
    const int64_t off = key_row(a, L, b, u);
    rows[tid] = off;
    float lg = -INFINITY;
    if (off != -1) {
      const float* kp = off >= 0 ? kvb + off : wnb + (-2 - off);
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], kp[d], dot);
      lg = dot * a.scale_log2;
    }
    const float mb = block_max(lg);
    const float m_new = fmaxf(m_run, mb);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    const float p = (m_new == -INFINITY || lg == -INFINITY) ? 0.f : exp2f(lg - m_new);
    ps[tid] = p;
    const float psum = block_sum(p);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const int cnt = (int)((L.n_tot - base) < 256 ? (L.n_tot - base) : 256);
    for (int i = 0; i < MAXD; ++i) {
      const int d = tid + 256 * i;
      if (d >= D) break;
      float x = acc[i] * alpha;
      for (int uu = 0; uu < cnt; ++uu) {
        const int64_t o2 = rows[uu];
        if (o2 == -1) continue;
        const float* kp = o2 >= 0 ? kvb + o2 : wnb + (-2 - o2);
        x = fmaf(ps[uu], kp[d], x);
      }
      acc[i] = x;
    }
    __syncthreads();
  }
  const float z = a.sink ? a.sink[h] * 1.4426950408889634f : -INFINITY;
  const float M = fmaxf(m_run, z);
  const float em = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
  const float lt = l_run * em + (z == -INFINITY ? 0.f : exp2f(z - M));
  const float fac = lt > 0.f ? em / lt : 0.f;
  if (a.lse && tid == 0) a.lse[row * a.H + h] = (M + log2f(lt)) * 0.6931471805599453f;
  for (int i = 0; i < MAXD; ++i) {
    const int d = tid + 256 * i;
    if (d < D) qs[d] = acc[i] * fac;  // reuse qs as the output row
  }
  __syncthreads();
  for (int d = rstart + 2 * tid; a.rope_on_output && a.rope_dims > 0 && d < D; d += 512) {
    float cs, sn;
    rope_cos_sin_t(a.rope, -t, (d - rstart) >> 1, a.rope_dims, a.rope_base, &cs, &sn);
    const float x0 = qs[d], x1 = qs[d + 1];
    qs[d] = x0 * cs - x1 * sn;
    qs[d + 1] = x0 * sn + x1 * cs;
  }
  __syncthreads();
  float* op = (float*)a.out + (row * a.H + h) * (int64_t)D;
  for (int d = tid; d < D; d += 256) op[d] = qs[d];
}

// ---------------------------------------------------------------------------- host
template <int D, int HW, int QG, int KVR>
static void launch_kvr(const AttnArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (KVR <= D) {
    // 256-thread workgroups over bf16 entries, not split (CSA prefill with 49-64 heads; HCA
    // prefill with 17-32 heads and two queries per workgroup, taken for calls of 2-3 queries):
    // two per CU, so the compiler keeps each lane within 256 registers; built for one per CU they
    // took twice that and ran alone on the CU
    if constexpr (D == 512 && HW * QG == 4) {
      if (a.n_splits == 1) {
        hipLaunchKernelGGL((attn_mfma<D, HW, QG, KVR, 2>), grid, dim3(HW * QG * 64), 0, st, a);
        return;
      }
    }
    hipLaunchKernelGGL((attn_mfma<D, HW, QG, KVR>), grid, dim3(HW * QG * 64), 0, st, a);
  }
}

// FP8 entries are compiled for RoPE widths 0, 16, 32 and 64 (validated before launch).
template <int D, int HW, int QG>
static void launch_attn(const AttnArgs& a, dim3 grid, hipStream_t st) {
  if (!a.kv_scale) return launch_kvr<D, HW, QG, -1>(a, grid, st);
  switch (a.rope_dims) {
    case 0: return launch_kvr<D, HW, QG, 0>(a, grid, st);
    case 16: return launch_kvr<D, HW, QG, 16>(a, grid, st);
    case 32: return launch_kvr<D, HW, QG, 32>(a, grid, st);
    default: return launch_kvr<D, HW, QG, 64>(a, grid, st);
  }
}

// Workgroup shape: HW waves of 16 heads per query; QG queries share one key stream
// (HCA, where neighbouring queries see the same compressed entries and overlapping windows).
template <int D, int HW>
static bool dispatch_qg(int qg, const AttnArgs& a, int batch, hipStream_t st) {
  const unsigned splits = (unsigned)a.n_splits;
  switch (qg) {
    case 1:
      if constexpr ((D / 8) % (HW * 2) == 0) {
        launch_attn<D, HW, 1>(a, dim3((unsigned)(batch * a.Tq), splits), st);
        return true;
      }
      return false;
    case 2:
      if constexpr (HW * 2 <= 8 && (D / 8) % (HW * 2 * 2) == 0) {
        launch_attn<D, HW, 2>(a, dim3((unsigned)(batch * ((a.Tq + 1) / 2)), splits), st);
        return true;
      }
      return false;
    case 4:
      if constexpr (D == 512 && HW == 2) {
        launch_attn<D, HW, 4>(a, dim3((unsigned)(batch * ((a.Tq + 3) / 4)), splits), st);
        return true;
      }
      return false;
    default: return false;
  }
}

template <int D>
static bool dispatch_hw(int hw, int qg, const AttnArgs& a, int batch, hipStream_t st) {
  switch (hw) {
    case 1: return dispatch_qg<D, 1>(qg, a, batch, st);
    case 2: return dispatch_qg<D, 2>(qg, a, batch, st);
    case 4: return dispatch_qg<D, 4>(qg, a, batch, st);
    case 8: return dispatch_qg<D, 8>(qg, a, batch, st);
    default: return false;
  }
}

#ifndef CSKV_HCA_QG
#define CSKV_HCA_QG 2
#endif
#ifndef CSKV_HCA_QG32
#define CSKV_HCA_QG32 4
#endif

static bool dispatch_attn(const AttnArgs& a, int batch, hipStream_t st) {
  const int hw = a.H <= 16 ? 1 : a.H <= 32 ? 2 : a.H <= 64 ? 4 : 8;
  // HCA prefill: CSKV_HCA_QG queries per workgroup share the gathered key tiles
  int qg = (a.mode == CSKV_MODE_HCA && a.n_splits == 1 && a.Tq >= 2 && hw <= 4 && a.D >= 128) ? CSKV_HCA_QG : 1;
  // 17-32 heads of 512 dims: four queries (eight waves) per workgroup share the key tiles
  // (16K HCA attention 0.65 -> 0.59 ms against two)
  if (qg > 1 && hw == 2 && a.D == 512 && a.Tq >= 4) qg = CSKV_HCA_QG32;
  switch (a.D) {
    case 64: return dispatch_hw<64>(hw, qg, a, batch, st);
    case 128: return dispatch_hw<128>(hw, qg, a, batch, st);
    case 256: return dispatch_hw<256>(hw, qg, a, batch, st);
    case 512: return dispatch_hw<512>(hw, qg, a, batch, st);
    default: return false;
  }
}

static int validate_attn(int mode, const void* q, const void* kv, const int32_t* idx, const void* win,
                         int64_t win_pos0, int64_t W, const float* sink, int batch, int64_t Tq,
                         int64_t N, int64_t pos0, int m, int k, int w, int H, int d,
                         int apply_q_norm, const float* q_norm_w, float eps, int rope_dims,
                         float rope_base, float scale, void* out, float* lse, int dtype) {
  if (dtype != CSKV_BF16 && dtype != CSKV_F32) return CSKV_ERR_BAD_DTYPE;
  if (mode != CSKV_MODE_CSA && mode != CSKV_MODE_HCA) return CSKV_ERR_INVALID_ARG;
  if (batch < 0 || Tq < 0 || N < 0 || pos0 < 0 || m < 1 || w < 1 || W < 0) return CSKV_ERR_BAD_SHAPE;
  if (H < 1 || H > CSKV_MAX_HEADS) return CSKV_ERR_BAD_SHAPE;
  if (dtype == CSKV_BF16 && d != 64 && d != 128 && d != 256 && d != 512) return CSKV_ERR_UNSUPPORTED;
  if (d < 32 || d % 32 != 0 || d > CSKV_MAX_DIM) return CSKV_ERR_BAD_SHAPE;
  if (rope_dims < 0 || rope_dims > d || (rope_dims & 1)) return CSKV_ERR_BAD_SHAPE;
  if (rope_dims > 0 && !(rope_base > 0.f)) return CSKV_ERR_INVALID_ARG;
  if (apply_q_norm && !(eps > 0.f)) return CSKV_ERR_INVALID_ARG;
  if (!(scale >= 0.f)) return CSKV_ERR_INVALID_ARG;
  if (mode == CSKV_MODE_CSA && (k < 1 || k > CSKV_MAX_TOPK)) return k < 1 ? CSKV_ERR_BAD_SHAPE : CSKV_ERR_UNSUPPORTED;
  if (batch == 0 || Tq == 0) return CSKV_OK;
  int64_t lo = pos0 - w + 1;
  if (lo < 0) lo = 0;
  // positions lo .. pos0 + Tq - 1 must fit in the W rows of `win`
  if (win_pos0 < 0 || W < pos0 + Tq - lo) return CSKV_ERR_BAD_SHAPE;
  if (!q || !win || !out || (N > 0 && !kv) || (mode == CSKV_MODE_CSA && !idx)) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(q, kv, idx, win, sink, q_norm_w, out, lse)) return CSKV_ERR_MISALIGNED;
  return CSKV_OK;
}

// FP8 KV storage: bf16 path only; whole 16-byte chunks of codes and of RoPE dims.
static int validate_kv8(const float* kv_scale, int64_t N, int d, int rope_dims, int dtype) {
  if (dtype != CSKV_BF16) return CSKV_ERR_BAD_DTYPE;
  if ((d - rope_dims) % 16 != 0 || rope_dims % 8 != 0) return CSKV_ERR_BAD_SHAPE;
  if (rope_dims != 0 && rope_dims != 16 && rope_dims != 32 && rope_dims != 64) return CSKV_ERR_UNSUPPORTED;
  if (N > 0 && !aligned16(kv_scale)) return CSKV_ERR_MISALIGNED;
  return CSKV_OK;
}

static AttnArgs make_args(int mode, const void* q, const void* kv, const int32_t* idx, const void* win,
                          int64_t win_pos0, int64_t W, const float* sink, int64_t Tq, int64_t N,
                          int64_t pos0, int m, int k, int w, int H, int d, int apply_q_norm,
                          const float* q_norm_w, float eps, int rope_dims, float rope_base,
                          float scale, int rope_on_output, void* out, float* lse) {
  AttnArgs a{};
  a.q = q; a.kv = kv; a.idx = idx; a.win = win; a.sink = sink; a.q_norm_w = q_norm_w;
  a.out = out; a.lse = lse;
  a.Tq = Tq; a.N = N; a.pos0 = pos0; a.win_pos0 = win_pos0; a.W = W;
  a.m = m; a.k = k; a.w = w; a.H = H; a.D = d; a.mode = mode; a.apply_q_norm = apply_q_norm;
  a.rope_dims = rope_dims; a.rope_on_output = rope_on_output; a.n_splits = 1;
  a.eps = eps; a.rope_base = rope_base;
  fill_rope_table(a.rope, rope_base, rope_dims);
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  a.scale_log2 = sc * 1.4426950408889634f;
  return a;
}

static int launch_f32(const AttnArgs& a, int batch, hipStream_t st) {
  const size_t shm = (size_t)(a.D + 256 + 8) * 4 + 256 * 8;
  hipLaunchKernelGGL(attn_f32, dim3((unsigned)(batch * a.Tq), (unsigned)a.H), dim3(256), shm, st, a);
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

static int64_t max_keys(int mode, int64_t Tq, int64_t N, int64_t pos0, int m, int k, int w) {
  const int64_t tl = pos0 + Tq - 1;
  int64_t nc = mode == CSKV_MODE_CSA ? k : ((tl + 1) / m < N ? (tl + 1) / m : N);
  return nc + (w < tl + 1 ? w : tl + 1);
}

}  // namespace cskv

using namespace cskv;

static int attn_prefill_impl(int mode, const void* q, const void* kv, const float* kv_scale, const int32_t* idx,
                             const void* win, int64_t win_pos0, int64_t W, const float* sink, int batch,
                             int64_t Tq, int64_t N, int64_t pos0, int m, int k, int w, int H, int d,
                             int apply_q_norm, const float* q_norm_w, float eps, int rope_dims, float rope_base,
                             float scale, int rope_on_output, void* out, float* lse, int dtype, void* stream) {
  int st = validate_attn(mode, q, kv, idx, win, win_pos0, W, sink, batch, Tq, N, pos0, m, k, w, H, d,
                         apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, out, lse, dtype);
  if (!st && kv_scale) st = validate_kv8(kv_scale, N, d, rope_dims, dtype);
  if (st || batch == 0 || Tq == 0) return st;
  AttnArgs a = make_args(mode, q, kv, idx, win, win_pos0, W, sink, Tq, N, pos0, m, k, w, H, d,
                         apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output,
                         out, lse);
  a.kv_scale = kv_scale;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == CSKV_F32) return launch_f32(a, batch, s);
  if (!dispatch_attn(a, batch, s)) return CSKV_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

extern "C" int compressed_attn_prefill(int mode, const void* q, const void* kv, const int32_t* idx,
                                       const void* win, int64_t win_pos0, int64_t W,
                                       const float* sink, int batch, int64_t Tq, int64_t N,
                                       int64_t pos0, int m, int k, int w, int H, int d,
                                       int apply_q_norm, const float* q_norm_w, float eps,
                                       int rope_dims, float rope_base, float scale,
                                       int rope_on_output, void* out, float* lse, int dtype,
                                       void* stream) {
  return attn_prefill_impl(mode, q, kv, nullptr, idx, win, win_pos0, W, sink, batch, Tq, N, pos0, m, k, w, H, d,
                           apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output, out, lse,
                           dtype, stream);
}

// FP8 + BF16 stored entries -> bf16 rows: each 8-code chunk widened exactly (E4M3 times the entry's
// power-of-two scale, the same conversion the attention loader applies), the RoPE dims copied. One
// wave per entry, 16-byte pieces.
__global__ __launch_bounds__(256) void dequant_kv8_kernel(const uint8_t* kv, const float* kv_scale, int64_t rows,
                                                          int d, int rope, uint16_t* out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int nope = d - rope;
  const uint8_t* src = kv + r * (int64_t)(nope + 2 * rope);
  uint16_t* dst = out + r * (int64_t)d;
  const float sc = kv_scale[r];
  const int nch8 = nope / 8, nch = nch8 + rope / 8;
  for (int c = lane; c < nch; c += 64) {
    u32x4 v;
    if (c < nch8) {
      const uint2 cc = *reinterpret_cast<const uint2*>(src + 8 * c);
      v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cc.x, sc, false));
      v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cc.x, sc, true));
      v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cc.y, sc, false));
      v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cc.y, sc, true));
    } else {
      v = *reinterpret_cast<const u32x4*>(src + nope + 16 * (c - nch8));
    }
    *reinterpret_cast<u32x4*>(dst + 8 * c) = v;
  }
}

// HCA prefill over an FP8 cache: every query of the call reads every visible entry, so the
// entries are widened once into the workspace and the bf16 kernels run on them.
extern "C" size_t cskv_prefill_kv8_workspace_size(int mode, int batch, int64_t N, int d) {
  if (mode != CSKV_MODE_HCA || batch <= 0 || N <= 0 || d <= 0) return 0;
  return (size_t)batch * (size_t)N * (size_t)d * 2;
}

extern "C" int compressed_attn_prefill_kv8(int mode, const void* q, const uint8_t* kv, const float* kv_scale,
                                           const int32_t* idx, const void* win, int64_t win_pos0, int64_t W,
                                           const float* sink, int batch, int64_t Tq, int64_t N, int64_t pos0,
                                           int m, int k, int w, int H, int d, int apply_q_norm,
                                           const float* q_norm_w, float eps, int rope_dims, float rope_base,
                                           float scale, int rope_on_output, void* workspace, size_t ws_bytes,
                                           void* out, float* lse, void* stream) {
  if (N > 0 && !kv_scale) return CSKV_ERR_INVALID_ARG;
  if (mode == CSKV_MODE_HCA && workspace && N > 0 && batch > 0 && Tq > 0) {
    int st = validate_attn(mode, q, kv, idx, win, win_pos0, W, sink, batch, Tq, N, pos0, m, k, w, H, d,
                           apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, out, lse, CSKV_BF16);
    if (!st) st = validate_kv8(kv_scale, N, d, rope_dims, CSKV_BF16);
    if (st) return st;
    if (!aligned16(workspace)) return CSKV_ERR_MISALIGNED;
    if (ws_bytes < cskv_prefill_kv8_workspace_size(mode, batch, N, d)) return CSKV_ERR_WORKSPACE;
    const int64_t rows = (int64_t)batch * N;
    hipLaunchKernelGGL(dequant_kv8_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, (hipStream_t)stream,
                       kv, kv_scale, rows, d, rope_dims, (uint16_t*)workspace);
    if (hipGetLastError() != hipSuccess) return CSKV_ERR_HIP;
    return attn_prefill_impl(mode, q, workspace, nullptr, idx, win, win_pos0, W, sink, batch, Tq, N, pos0, m, k,
                             w, H, d, apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output,
                             out, lse, CSKV_BF16, stream);
  }
  return attn_prefill_impl(mode, q, kv, N > 0 ? kv_scale : nullptr, idx, win, win_pos0, W, sink, batch, Tq, N,
                           pos0, m, k, w, H, d, apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale,
                           rope_on_output, out, lse, CSKV_BF16, stream);
}

// Automatic split count: about one workgroup per CU over the call (256 / queries), at least 2 key
// tiles per split, at most 256. Every split costs a query prologue and an fp32 partial of H x d
// written and merged, so more splits than CUs only add traffic. Without the key count this is
// bounded by the first term alone.
static int64_t auto_splits_bound(int batch, int64_t Tq) {
  int64_t s = (256 + batch * Tq - 1) / (batch * Tq);
  return s > 256 ? 256 : (s < 1 ? 1 : s);
}

static int decode_splits(int batch, int64_t Tq, int64_t max_k, int n_splits) {
  if (n_splits > 0) return n_splits;
  const int64_t nblk = (max_k + 31) / 32;
  int64_t s = auto_splits_bound(batch, Tq);
  const int64_t cap = (nblk + 1) / 2;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}

static size_t decode_partial_bytes(int batch, int64_t Tq, int S, int H, int d) {
  return S > 1 ? (size_t)batch * Tq * S * H * ((size_t)d + 2) * 4 : 0;
}

extern "C" size_t cskv_decode_workspace_size(int batch, int64_t Tq, int H, int d, int n_splits) {
  if (batch <= 0 || Tq <= 0 || H <= 0 || d <= 0 || n_splits < 0 || n_splits > 256) return 0;
  const int S = n_splits > 0 ? n_splits : (int)auto_splits_bound(batch, Tq);
  return decode_partial_bytes(batch, Tq, S, H, d);
}

// Split-K launch: S splits write fp32 partials into `part` (S > 1: decode_partial_bytes of
// it), then attn_merge combines them; S = 1 runs the single-pass kernel and needs no partials.
static int launch_decode(AttnArgs& a, int batch, int S, void* part, hipStream_t s) {
  if (S == 1) {
    if (!dispatch_attn(a, batch, s)) return CSKV_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
  }
  a.n_splits = S;
  a.part_o = (float*)part;
  a.part_ml = a.part_o + (size_t)batch * a.Tq * S * a.H * a.D;
  if (!dispatch_attn(a, batch, s)) return CSKV_ERR_UNSUPPORTED;
  if (hipGetLastError() != hipSuccess) return CSKV_ERR_HIP;
  hipLaunchKernelGGL((attn_merge<bf16>), dim3((unsigned)(batch * a.Tq), (unsigned)a.H), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

static int attn_decode_impl(int mode, const void* q, const void* kv, const float* kv_scale, const int32_t* idx,
                            const void* win, int64_t win_pos0, int64_t W, const float* sink, int batch,
                            int64_t Tq, int64_t N, int64_t pos0, int m, int k, int w, int H, int d,
                            int apply_q_norm, const float* q_norm_w, float eps, int rope_dims, float rope_base,
                            float scale, int rope_on_output, int n_splits, void* workspace, size_t ws_bytes,
                            void* out, float* lse, int dtype, void* stream) {
  int st = validate_attn(mode, q, kv, idx, win, win_pos0, W, sink, batch, Tq, N, pos0, m, k, w, H, d,
                         apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, out, lse, dtype);
  if (!st && kv_scale) st = validate_kv8(kv_scale, N, d, rope_dims, dtype);
  if (st) return st;
  if (n_splits < 0 || n_splits > 256) return CSKV_ERR_BAD_SHAPE;
  if (batch == 0 || Tq == 0) return CSKV_OK;
  AttnArgs a = make_args(mode, q, kv, idx, win, win_pos0, W, sink, Tq, N, pos0, m, k, w, H, d,
                         apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output,
                         out, lse);
  a.kv_scale = kv_scale;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == CSKV_F32) return launch_f32(a, batch, s);
  const int S = decode_splits(batch, Tq, max_keys(mode, Tq, N, pos0, m, k, w), n_splits);
  if (S > 1) {
    const size_t need = decode_partial_bytes(batch, Tq, S, H, d);
    if (!workspace || ws_bytes < need) return CSKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return CSKV_ERR_MISALIGNED;
  }
  return launch_decode(a, batch, S, workspace, s);
}

extern "C" int compressed_attn_decode(int mode, const void* q, const void* kv, const int32_t* idx,
                                      const void* win, int64_t win_pos0, int64_t W,
                                      const float* sink, int batch, int64_t Tq, int64_t N,
                                      int64_t pos0, int m, int k, int w, int H, int d,
                                      int apply_q_norm, const float* q_norm_w, float eps,
                                      int rope_dims, float rope_base, float scale,
                                      int rope_on_output, int n_splits, void* workspace,
                                      size_t ws_bytes, void* out, float* lse, int dtype,
                                      void* stream) {
  return attn_decode_impl(mode, q, kv, nullptr, idx, win, win_pos0, W, sink, batch, Tq, N, pos0, m, k, w, H, d,
                          apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output, n_splits,
                          workspace, ws_bytes, out, lse, dtype, stream);
}

extern "C" int compressed_attn_decode_kv8(int mode, const void* q, const uint8_t* kv, const float* kv_scale,
                                          const int32_t* idx, const void* win, int64_t win_pos0, int64_t W,
                                          const float* sink, int batch, int64_t Tq, int64_t N, int64_t pos0,
                                          int m, int k, int w, int H, int d, int apply_q_norm,
                                          const float* q_norm_w, float eps, int rope_dims, float rope_base,
                                          float scale, int rope_on_output, int n_splits, void* workspace,
                                          size_t ws_bytes, void* out, float* lse, void* stream) {
  if (N > 0 && !kv_scale) return CSKV_ERR_INVALID_ARG;
  return attn_decode_impl(mode, q, kv, N > 0 ? kv_scale : nullptr, idx, win, win_pos0, W, sink, batch, Tq, N,
                          pos0, m, k, w, H, d, apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale,
                          rope_on_output, n_splits, workspace, ws_bytes, out, lse, CSKV_BF16, stream);
}

// ---------------------------------------------------------------------------- allocation-free decode
// compressed_attn_decode for callers that cannot allocate device memory: the split partials
// live in `scratch`, a file-scope device array of CSKV_NOALLOC_SCRATCH_BYTES. Each GPU the
// library runs on holds its own copy until the process ends; its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only that address is
// handed to kernels -- in host code the array's name is a host-side stand-in, not a device
// address. Every call on a GPU shares that GPU's array, so calls that overlap on one GPU
// (different streams, or host threads) race on it. The partials need no clearing: every split
// writes its whole partial, an empty split included.
static __device__ __align__(256) unsigned char scratch[CSKV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
std::atomic<void*> scratch_addr[kMaxDevices];

// Device address of this device's `scratch`, for the device that `stream` runs on.
int scratch_address(hipStream_t stream, void** addr) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return CSKV_ERR_HIP;
  int dev = cur;
  if (stream) {
    hipDevice_t sd;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return CSKV_ERR_HIP;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return CSKV_ERR_UNSUPPORTED;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (dev != cur && hipSetDevice(dev) != hipSuccess) return CSKV_ERR_HIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (dev != cur && hipSetDevice(cur) != hipSuccess) return CSKV_ERR_HIP;
      if (e != hipSuccess || !p) return CSKV_ERR_HIP;
      scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return CSKV_OK;
}
}  // namespace

extern "C" int compressed_attn_decode_noalloc(int mode, const void* q, const void* kv, const int32_t* idx,
                                              const void* win, int64_t win_pos0, int64_t W, const float* sink,
                                              int batch, int64_t Tq, int64_t N, int64_t pos0, int m, int k, int w,
                                              int H, int d, int apply_q_norm, const float* q_norm_w, float eps,
                                              int rope_dims, float rope_base, float scale, int rope_on_output,
                                              int n_splits, void* out, float* lse, int dtype, void* stream) {
  int st = validate_attn(mode, q, kv, idx, win, win_pos0, W, sink, batch, Tq, N, pos0, m, k, w, H, d,
                         apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, out, lse, dtype);
  if (st) return st;
  if (n_splits < 0 || n_splits > 256) return CSKV_ERR_BAD_SHAPE;
  if (batch == 0 || Tq == 0) return CSKV_OK;
  int S = 1;
  if (dtype == CSKV_BF16) {
    S = decode_splits(batch, Tq, max_keys(mode, Tq, N, pos0, m, k, w), n_splits);
    const size_t per_split = decode_partial_bytes(batch, Tq, 2, H, d) / 2;
    if (S > 1 && decode_partial_bytes(batch, Tq, S, H, d) > CSKV_NOALLOC_SCRATCH_BYTES) {
      if (n_splits > 0) return CSKV_ERR_WORKSPACE;  // an explicit split count beyond the scratch
      const size_t fit = CSKV_NOALLOC_SCRATCH_BYTES / per_split;
      S = fit >= 2 ? (int)fit : 1;
    }
  }
  AttnArgs a = make_args(mode, q, kv, idx, win, win_pos0, W, sink, Tq, N, pos0, m, k, w, H, d,
                         apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output,
                         out, lse);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == CSKV_F32) return launch_f32(a, batch, s);
  void* part = nullptr;
  if (S > 1) {
    st = scratch_address(s, &part);
    if (st) return st;
  }
  return launch_decode(a, batch, S, part, s);
}
