// MQA core attention over compressed entries + sliding window + sink, gfx950.
//
// "Paper Breakdown: DeepSeek-V4": CSA §2.3.1 (MQA core attention over the
// top-k selected compressed entries plus an uncompressed sliding window),
// HCA §2.3.2 (dense attention over every visible compressed entry plus the
// same window), §2.3.3 (query RMSNorm, partial RoPE on the last 64 dims,
// learnable per-head sink logits). "Inside DeepSeek V4", "Local window":
// 128 recent uncompressed entries in every CSA and HCA layer.
//
// bf16 kernel (one workgroup = one query, all heads; wave w = heads
// 16w..16w+15):
//  * The query rows are RMSNormed and rotated at the query's position in
//    registers, rounded to bf16 and kept as MFMA B operands (Q^T).
//  * The query's key list -- selected or visible compressed entries, then
//    window rows -- is gathered 32 rows at a time into a double-buffered LDS
//    tile (K = V: one tile serves both products).
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 puts keys on rows, so after the
//    online-softmax update each lane already holds its P values in the
//    layout of the A operand of O = P V (lane = head, 8 keys); no shuffle.
//  * For O = P V each lane reads 8 keys x 8 contiguous dims from LDS with
//    16-byte loads and transposes them in registers into 8 B operands, so
//    every O accumulator lane owns 8 contiguous output dims (16-byte stores,
//    RoPE pairs in-lane).
//  * Split-K (decode): a split writes (max, sum, unnormalised O) and a merge
//    kernel combines splits in a fixed order, adds the sink and de-rotates.
// fp32 kernel: plain vector-ALU online softmax, one workgroup per
// (query, head); it serves the fp32 mode.
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
  void* out;
  float* lse;
  float* part_o;   // [batch*Tq][splits][H][D]
  float* part_ml;  // [batch*Tq][splits][H][2] (running max, sum; base-2 logits)
  int64_t Tq, N, pos0, win_pos0, W;
  int m, k, w, H, D, mode, apply_q_norm, rope_dims, rope_on_output, n_splits;
  float eps, rope_base, scale_log2;
};

__device__ __forceinline__ int64_t visible_n(int64_t t, int m, int64_t N) {
  const int64_t v = (t + 1) / m;
  return v < N ? v : N;
}

// Key list of query (b, j): [0, n_comp) compressed (selected or visible), then window rows.
struct KeyList {
  const int32_t* idxrow;
  int64_t n_comp, n_tot, win_row0;  // win_row0: row of position max(0, t-w+1) in `win`
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
  L.win_row0 = lo - a.win_pos0;
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
  return -2 - (((int64_t)b * a.W + L.win_row0 + (u - L.n_comp)) * a.D);  // window: encoded < -1
}

// Key slot mapping shared by the P (A) and V (B) operands of O = P V:
// slot jj of lane group g holds key (jj < 4 ? 4g + jj : 16 + 4g + jj - 4),
// which is where S^T = K Q^T leaves the logits.
__device__ __forceinline__ int pv_key(int g, int jj) { return jj < 4 ? 4 * g + jj : 12 + 4 * g + jj; }

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_mfma(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int ROWE = D + 8;        // padded LDS row, bf16 elements
  constexpr int KS = D / 32;         // k-steps of S^T = K Q^T
  constexpr int DG = D < 128 ? D : 128;
  constexpr int E = DG / 16;         // contiguous output dims per lane per group (8 or 4)
  constexpr int NG = D / DG;
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int CHUNKS = 32 * CPR;
  constexpr int CPT = (CHUNKS + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][32 * ROWE];
  __shared__ uint32_t kvalid[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t flat = (int64_t)gridDim.x - 1 - blockIdx.x;  // later (longer) rows first
  const int b = (int)(flat / a.Tq);
  const int64_t j = flat % a.Tq;
  const int split = blockIdx.y;
  const int64_t t = a.pos0 + j;
  const int h = wave * 16 + n;
  const bool hvalid = h < a.H;
  const KeyList L = make_keys(a, b, j);
  const int64_t nblk = (L.n_tot + 31) / 32;
  const int64_t bps = (nblk + a.n_splits - 1) / a.n_splits;
  const int64_t blk0 = (int64_t)split * bps;
  const int64_t blk1 = blk0 + bps < nblk ? blk0 + bps : nblk;

  // ---- query prologue: RMSNorm, RoPE at t, bf16 B operands (lane: head n, dims 32ks + 8g + 0..7)
  bf16x8 qb[KS];
  {
    const uint16_t* qp = (const uint16_t*)a.q + (((int64_t)b * a.Tq + j) * a.H + (hvalid ? h : 0)) * D;
    float x[KS][8];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      load_vec<bf16, 8>(reinterpret_cast<const bf16*>(qp + ks * 32 + 8 * g), x[ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!hvalid) x[ks][e] = 0.f;
        ss += x[ks][e] * x[ks][e];
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = a.apply_q_norm ? rsqrtf(ss / (float)D + a.eps) : 1.f;
    const int rstart = D - a.rope_dims;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dim = ks * 32 + 8 * g + e;
        x[ks][e] *= inv * (a.q_norm_w ? a.q_norm_w[dim] : 1.f);
      }
      if (a.rope_dims > 0 && ks * 32 + 8 * g + 8 > rstart) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int dim = ks * 32 + 8 * g + e;
          if (dim >= rstart) {
            float cs, sn;
            rope_cos_sin(t, (dim - rstart) >> 1, a.rope_dims, a.rope_base, &cs, &sn);
            const float x0 = x[ks][e], x1 = x[ks][e + 1];
            x[ks][e] = x0 * cs - x1 * sn;
            x[ks][e + 1] = x0 * sn + x1 * cs;
          }
        }
      }
      u32x4 pk;
      pk[0] = pack_bf16x2(x[ks][0], x[ks][1]);
      pk[1] = pack_bf16x2(x[ks][2], x[ks][3]);
      pk[2] = pack_bf16x2(x[ks][4], x[ks][5]);
      pk[3] = pack_bf16x2(x[ks][6], x[ks][7]);
      qb[ks] = __builtin_bit_cast(bf16x8, pk);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;  // per head n (same in all four lane groups)
  f32x4 o[NG][E];
#pragma unroll
  for (int gr = 0; gr < NG; ++gr)
#pragma unroll
    for (int e = 0; e < E; ++e) o[gr][e] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- gather loader: 32 key rows per tile
  const uint16_t* kvb = (const uint16_t*)a.kv;
  const uint16_t* wnb = (const uint16_t*)a.win;
  u32x4 pre[CPT];
  bool pre_ok = false;  // thread tid < 32: validity of key tid of the prefetched tile
  auto gload = [&](int64_t blk) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ch < CHUNKS) {
        const int64_t off = key_row(a, L, b, blk * 32 + ch / CPR);
        if (off >= 0)
          v = *reinterpret_cast<const u32x4*>(kvb + off + (ch % CPR) * 8);
        else if (off < -1)
          v = *reinterpret_cast<const u32x4*>(wnb + (-2 - off) + (ch % CPR) * 8);
      }
      pre[c] = v;
    }
    if (tid < 32) pre_ok = key_row(a, L, b, blk * 32 + tid) != -1;
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < CHUNKS) *reinterpret_cast<u32x4*>(&kt[buf][(ch / CPR) * ROWE + (ch % CPR) * 8]) = pre[c];
    }
    if (wave == 0) {
      const uint64_t bal = __ballot(tid < 32 && pre_ok);
      if (tid == 0) kvalid[buf] = (uint32_t)bal;
    }
  };

  if (blk0 < blk1) {
    gload(blk0);
    lstore(0);
  }
  __syncthreads();
  for (int64_t blk = blk0; blk < blk1; ++blk) {
    const int buf = (int)((blk - blk0) & 1);
    if (blk + 1 < blk1) gload(blk + 1);

    // S^T = K Q^T: s0 -> keys 4g+i, s1 -> keys 16+4g+i; column = head n
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* kp = &kt[buf][n * ROWE + 8 * g];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kp + ks * 32);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kp + 16 * ROWE + ks * 32);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb[ks], s1, 0, 0, 0);
    }
    const uint32_t vm = kvalid[buf];
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = ((vm >> (4 * g + i)) & 1u) ? s0[i] * a.scale_log2 : -INFINITY;
      sv[4 + i] = ((vm >> (16 + 4 * g + i)) & 1u) ? s1[i] * a.scale_log2 : -INFINITY;
    }
    float mb = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mb = fmaxf(mb, sv[i]);
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float m_new = fmaxf(m_run, mb);
    float alpha = 1.f, p[8];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = exp2f(sv[i] - m_new);
    }
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ps += p[i];
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;

    // rescale O rows (heads 4g+i) by their alpha
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
    for (int gr = 0; gr < NG; ++gr)
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[gr][e][i] *= al[i];

    u32x4 pp;
    pp[0] = pack_bf16x2(p[0], p[1]);
    pp[1] = pack_bf16x2(p[2], p[3]);
    pp[2] = pack_bf16x2(p[4], p[5]);
    pp[3] = pack_bf16x2(p[6], p[7]);
    const bf16x8 pa = __builtin_bit_cast(bf16x8, pp);

    // O += P V, 8 keys x E dims per lane, transposed in registers into E B operands
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) {
      uint32_t vr[8][E / 2];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const uint16_t* vp = &kt[buf][pv_key(g, jj) * ROWE + gr * DG + E * n];
        if constexpr (E == 8) {
          const u32x4 r = *reinterpret_cast<const u32x4*>(vp);
          vr[jj][0] = r[0]; vr[jj][1] = r[1]; vr[jj][2] = r[2]; vr[jj][3] = r[3];
        } else {
          const uint2 r = *reinterpret_cast<const uint2*>(vp);
          vr[jj][0] = r.x; vr[jj][1] = r.y;
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        u32x4 bv;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const uint32_t lo = vr[2 * q2][e >> 1], hi = vr[2 * q2 + 1][e >> 1];
          bv[q2] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        o[gr][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, bv), o[gr][e], 0, 0, 0);
      }
    }
    if (blk + 1 < blk1) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue. Lane holds O[head 4g+i][gr*DG + E*n + e].
  const int64_t row = (int64_t)b * a.Tq + j;
  if (a.n_splits > 1) {
    float* po = a.part_o + ((row * a.n_splits + split) * a.H) * (int64_t)D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = wave * 16 + 4 * g + i;
      if (hh >= a.H) continue;
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) {
        float v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = o[gr][e][i];
        store_vec<float, 4>(po + (int64_t)hh * D + gr * DG + E * n, v);
        if constexpr (E == 8) store_vec<float, 4>(po + (int64_t)hh * D + gr * DG + E * n + 4, v + 4);
      }
    }
    if (g == 0 && hvalid) {
      float* pm = a.part_ml + ((row * a.n_splits + split) * a.H + h) * 2;
      pm[0] = m_run;
      pm[1] = l_run;
    }
    return;
  }

  // single split: fold the sink, normalise, de-rotate, store
  const float z = (a.sink && hvalid) ? a.sink[h] * 1.4426950408889634f : -INFINITY;
  const float M = fmaxf(m_run, z);
  const float em = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
  const float lt = l_run * em + (z == -INFINITY ? 0.f : exp2f(z - M));
  const float fac = lt > 0.f ? em / lt : 0.f;
  if (a.lse && g == 0 && hvalid) a.lse[row * a.H + h] = (M + log2f(lt)) * 0.6931471805599453f;
  float fi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fi[i] = __shfl(fac, 4 * g + i, 64);
  const int rstart = D - a.rope_dims;
#pragma unroll
  for (int gr = 0; gr < NG; ++gr) {
    const int d0 = gr * DG + E * n;
    float cs[E / 2], sn[E / 2];
    const bool rot = a.rope_on_output && a.rope_dims > 0 && d0 + E > rstart;
    if (rot) {
#pragma unroll
      for (int e = 0; e < E; e += 2) {
        cs[e / 2] = 1.f;
        sn[e / 2] = 0.f;
        if (d0 + e >= rstart) rope_cos_sin(-t, (d0 + e - rstart) >> 1, a.rope_dims, a.rope_base, &cs[e / 2], &sn[e / 2]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = wave * 16 + 4 * g + i;
      float v[E];
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = o[gr][e][i] * fi[i];
      if (rot) {
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          const float x0 = v[e], x1 = v[e + 1];
          v[e] = x0 * cs[e / 2] - x1 * sn[e / 2];
          v[e + 1] = x0 * sn[e / 2] + x1 * cs[e / 2];
        }
      }
      if (hh < a.H) store_vec<bf16, E>((bf16*)a.out + (row * a.H + hh) * D + d0, v);
    }
  }
}

// Merge split partials in split order, add the sink, normalise, de-rotate.
template <typename T>
__global__ __launch_bounds__(256) void attn_merge(AttnArgs a) {
  __shared__ float wsplit[256];
  __shared__ float scal[2];
  const int64_t row = blockIdx.x;  // b*Tq + j
  const int h = blockIdx.y;
  const int D = a.D;
  const int S = a.n_splits;
  const int64_t j = row % a.Tq;
  const int64_t t = a.pos0 + j;
  const float* pm = a.part_ml + (row * S * a.H) * 2;
  if (threadIdx.x == 0) {
    const float z = a.sink ? a.sink[h] * 1.4426950408889634f : -INFINITY;
    float M = z;
    for (int s = 0; s < S; ++s) M = fmaxf(M, pm[(s * a.H + h) * 2]);
    float lt = (z == -INFINITY) ? 0.f : exp2f(z - M);
    for (int s = 0; s < S; ++s) {
      const float ms = pm[(s * a.H + h) * 2];
      const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
      wsplit[s] = w;
      lt += w * pm[(s * a.H + h) * 2 + 1];
    }
    scal[0] = lt > 0.f ? 1.f / lt : 0.f;
    if (a.lse) a.lse[row * a.H + h] = (M + log2f(lt)) * 0.6931471805599453f;
  }
  __syncthreads();
  const float inv = scal[0];
  const int rstart = D - a.rope_dims;
  for (int d = 2 * threadIdx.x; d < D; d += 2 * blockDim.x) {
    float x0 = 0.f, x1 = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* po = a.part_o + ((row * S + s) * a.H + h) * (int64_t)D + d;
      x0 += po[0] * wsplit[s];
      x1 += po[1] * wsplit[s];
    }
    x0 *= inv;
    x1 *= inv;
    if (a.rope_on_output && a.rope_dims > 0 && d >= rstart) {
      float cs, sn;
      rope_cos_sin(-t, (d - rstart) >> 1, a.rope_dims, a.rope_base, &cs, &sn);
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
    rope_cos_sin(t, (d - rstart) >> 1, a.rope_dims, a.rope_base, &cs, &sn);
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
    rope_cos_sin(-t, (d - rstart) >> 1, a.rope_dims, a.rope_base, &cs, &sn);
    const float x0 = qs[d], x1 = qs[d + 1];
    qs[d] = x0 * cs - x1 * sn;
    qs[d + 1] = x0 * sn + x1 * cs;
  }
  __syncthreads();
  float* op = (float*)a.out + (row * a.H + h) * (int64_t)D;
  for (int d = tid; d < D; d += 256) op[d] = qs[d];
}

// ---------------------------------------------------------------------------- host
template <int D, int NW>
static void launch_attn(const AttnArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_mfma<D, NW>), grid, dim3(NW * 64), 0, st, a);
}

template <int D>
static bool dispatch_nw(int nw, const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (nw) {
    case 1: launch_attn<D, 1>(a, grid, st); return true;
    case 2: launch_attn<D, 2>(a, grid, st); return true;
    case 4: launch_attn<D, 4>(a, grid, st); return true;
    case 8: launch_attn<D, 8>(a, grid, st); return true;
    default: return false;
  }
}

static bool dispatch_attn(const AttnArgs& a, dim3 grid, hipStream_t st) {
  const int nw = a.H <= 16 ? 1 : a.H <= 32 ? 2 : a.H <= 64 ? 4 : 8;
  switch (a.D) {
    case 64: return dispatch_nw<64>(nw, a, grid, st);
    case 128: return dispatch_nw<128>(nw, a, grid, st);
    case 256: return dispatch_nw<256>(nw, a, grid, st);
    case 512: return dispatch_nw<512>(nw, a, grid, st);
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
  if (win_pos0 < 0 || win_pos0 > lo || win_pos0 + W < pos0 + Tq) return CSKV_ERR_BAD_SHAPE;
  if (!q || !win || !out || (N > 0 && !kv) || (mode == CSKV_MODE_CSA && !idx)) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(q, kv, idx, win, sink, q_norm_w, out, lse)) return CSKV_ERR_MISALIGNED;
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

extern "C" int compressed_attn_prefill(int mode, const void* q, const void* kv, const int32_t* idx,
                                       const void* win, int64_t win_pos0, int64_t W,
                                       const float* sink, int batch, int64_t Tq, int64_t N,
                                       int64_t pos0, int m, int k, int w, int H, int d,
                                       int apply_q_norm, const float* q_norm_w, float eps,
                                       int rope_dims, float rope_base, float scale,
                                       int rope_on_output, void* out, float* lse, int dtype,
                                       void* stream) {
  int st = validate_attn(mode, q, kv, idx, win, win_pos0, W, sink, batch, Tq, N, pos0, m, k, w, H, d,
                         apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, out, lse, dtype);
  if (st || batch == 0 || Tq == 0) return st;
  AttnArgs a = make_args(mode, q, kv, idx, win, win_pos0, W, sink, Tq, N, pos0, m, k, w, H, d,
                         apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output,
                         out, lse);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == CSKV_F32) return launch_f32(a, batch, s);
  if (!dispatch_attn(a, dim3((unsigned)(batch * Tq), 1), s)) return CSKV_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

static int decode_splits(int batch, int64_t Tq, int64_t max_k, int n_splits) {
  if (n_splits > 0) return n_splits;
  const int64_t nblk = (max_k + 31) / 32;
  int64_t s = (1024 + batch * Tq - 1) / (batch * Tq);
  const int64_t cap = (nblk + 3) / 4;
  if (s > cap) s = cap;
  if (s > 256) s = 256;
  if (s < 1) s = 1;
  return (int)s;
}

extern "C" size_t cskv_decode_workspace_size(int batch, int64_t Tq, int H, int d, int n_splits) {
  if (batch <= 0 || Tq <= 0) return 0;
  const int s = n_splits > 0 ? n_splits : 256;
  return (size_t)batch * Tq * s * H * ((size_t)d + 2) * 4 + 256;
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
  int st = validate_attn(mode, q, kv, idx, win, win_pos0, W, sink, batch, Tq, N, pos0, m, k, w, H, d,
                         apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, out, lse, dtype);
  if (st) return st;
  if (n_splits < 0 || n_splits > 256) return CSKV_ERR_BAD_SHAPE;
  if (batch == 0 || Tq == 0) return CSKV_OK;
  AttnArgs a = make_args(mode, q, kv, idx, win, win_pos0, W, sink, Tq, N, pos0, m, k, w, H, d,
                         apply_q_norm, q_norm_w, eps, rope_dims, rope_base, scale, rope_on_output,
                         out, lse);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == CSKV_F32) return launch_f32(a, batch, s);
  const int S = decode_splits(batch, Tq, max_keys(mode, Tq, N, pos0, m, k, w), n_splits);
  if (S == 1) {
    if (!dispatch_attn(a, dim3((unsigned)(batch * Tq), 1), s)) return CSKV_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
  }
  const size_t need = (size_t)batch * Tq * S * H * ((size_t)d + 2) * 4;
  if (!workspace || ws_bytes < need) return CSKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CSKV_ERR_MISALIGNED;
  a.n_splits = S;
  a.part_o = (float*)workspace;
  a.part_ml = a.part_o + (size_t)batch * Tq * S * H * d;
  if (!dispatch_attn(a, dim3((unsigned)(batch * Tq), (unsigned)S), s)) return CSKV_ERR_UNSUPPORTED;
  if (hipGetLastError() != hipSuccess) return CSKV_ERR_HIP;
  hipLaunchKernelGGL((attn_merge<bf16>), dim3((unsigned)(batch * Tq), (unsigned)H), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}
