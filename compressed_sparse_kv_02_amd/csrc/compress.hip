// KV compression kernels for gfx950.
//
// CSA compressor ("Paper Breakdown: DeepSeek-V4", §2.3.1 KV Compression):
// entry i pools 2m rows -- the m b-stream rows of block i-1 and the m
// a-stream rows of block i -- under one per-channel softmax of Z + B.
// HCA compressor (§2.3.2): entry i pools the m' rows of block i of one stream.
// Both are followed by optional RMSNorm over the channels and RoPE on the
// last rope_dims channels (§2.3.3) at the entry's position. m' = 1 prepares
// raw sliding-window rows: the softmax over one row is the row itself.
//
// The softmax is per channel, over the entry's rows, so a lane that owns a
// few channels needs nothing from other lanes until the RMSNorm. Three
// kernels, all HBM-streaming (every input byte read once):
//  * rows (one row per entry): a group of lanes per row, each lane 8 (bf16)
//    or 4 (fp32) channels per 16-byte load, several rows' loads in flight per
//    group; RMSNorm's sum of squares is a butterfly over the group's lanes.
//  * pool (2..32 rows per entry, e.g. CSA with m = 4): a group of lanes per
//    entry keeps an online softmax (max, sum, weighted sum) per channel in
//    registers over the entry's rows, loaded four rows at a time.
//  * block (more than 32 rows, e.g. HCA with m' = 128): a workgroup per
//    entry, its waves take interleaved rows, and one wave merges their
//    partial softmaxes from LDS in wave order.
// No kernel uses an atomic; every reduction has a fixed order, so results
// are deterministic. Rotary angles: each lane takes theta_j = base^(-2j/rope_dims)
// from the host's fp64 table (kernel argument), and the angle pos * theta_j
// is reduced modulo 2 pi in fp64 before an fp32 sincos.
#include <algorithm>

#include "device_common.h"
#include "abi_common.h"

namespace cskv {

struct CompressArgs {
  const void* Ca;  // HCA: C
  const void* Cb;
  const void* Za;  // HCA: Z (may be null -> uniform)
  const void* Zb;
  const void* B;   // CSA: [2m, c]; HCA: [m, c] or null
  const void* prev_Cb;
  const void* prev_Zb;
  void* out;
  const float* norm_w;
  int64_t T, pos0, out_ld;
  int c, m, n_out;
  int csa;  // 1: two streams, overlapped; 0: one stream
  int apply_norm, rope_dims;
  float eps, rope_base;
  int lpe;    // lanes per entry (power of two <= 64)
  int batch;  // sequences (the row and pool kernels stride over batch * n_out entries)
  RopeTable rope;  // theta of the first rotary pairs (host fp64)
};

__device__ __forceinline__ void rope_apply(double theta, int64_t pos, float& x0, float& x1) {
  const double inv_two_pi = 0.15915494309189533576888376337251;
  const double two_pi = 6.283185307179586476925286766559;
  double ang = (double)pos * theta;
  ang = __builtin_fma(-two_pi, rint(ang * inv_two_pi), ang);  // |ang| <= pi (+ rounding)
  float sn, cs;
  sincosf((float)ang, &sn, &cs);
  const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
  x0 = y0;
  x1 = y1;
}

// Per-lane rotary table: theta of each pair (channels ch, ch + 1) in this lane's channel groups,
// 0 where the pair is not rotated (ch < c - rope_dims; a group may straddle that boundary).
template <int VEC, int CPL>
__device__ __forceinline__ void rope_table(const CompressArgs& a, int gi, int LPE, double (&th)[CPL][VEC / 2]) {
  const int rstart = a.c - a.rope_dims;
#pragma unroll
  for (int cg = 0; cg < CPL; ++cg) {
    const int ch0 = (gi + LPE * cg) * VEC;
#pragma unroll
    for (int p = 0; p < VEC / 2; ++p) {
      const int ch = ch0 + 2 * p;
      th[cg][p] = (a.rope_dims > 0 && ch >= rstart && ch < a.c)
                      ? rope_theta_of(a.rope, (ch - rstart) >> 1, a.rope_dims, a.rope_base) : 0.0;
    }
  }
}

// RoPE at `pos` on the last rope_dims channels of y (a lane group's channel groups), then store.
template <typename T, int VEC, int CPL>
__device__ __forceinline__ void finish_rotate_store(const CompressArgs& a, float (&y)[CPL][VEC], int gi, int LPE,
                                                    const double (&th)[CPL][VEC / 2], int64_t pos, T* op) {
  const int groups = a.c / VEC;
  const int rstart = a.c - a.rope_dims;
#pragma unroll
  for (int cg = 0; cg < CPL; ++cg) {
    const int ch0 = (gi + LPE * cg) * VEC;
    if (gi + LPE * cg >= groups) continue;
    if (a.rope_dims > 0 && ch0 + VEC > rstart) {
#pragma unroll
      for (int p = 0; p < VEC / 2; ++p)
        if (ch0 + 2 * p >= rstart) rope_apply(th[cg][p], pos, y[cg][2 * p], y[cg][2 * p + 1]);
    }
    store_vec<T, VEC>(op + ch0, y[cg]);
  }
}

// Entry epilogue for a lane group of LPE lanes holding y[cg][v] = channel (gi + LPE cg) VEC + v:
// RMSNorm over the c channels, RoPE at `pos` on the last rope_dims channels, store to `op`.
template <typename T, int VEC, int CPL>
__device__ __forceinline__ void finish_entry(const CompressArgs& a, float (&y)[CPL][VEC], int gi, int LPE,
                                             const double (&th)[CPL][VEC / 2], int64_t pos, T* op) {
  const int groups = a.c / VEC;
  if (a.apply_norm) {
    float ss = 0.f;
#pragma unroll
    for (int cg = 0; cg < CPL; ++cg)
      if (gi + LPE * cg < groups)
#pragma unroll
        for (int v = 0; v < VEC; ++v) ss += y[cg][v] * y[cg][v];
    for (int o = LPE >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float inv = rsqrtf(ss / (float)a.c + a.eps);
#pragma unroll
    for (int cg = 0; cg < CPL; ++cg) {
      const int ch0 = (gi + LPE * cg) * VEC;
#pragma unroll
      for (int v = 0; v < VEC; ++v) y[cg][v] *= inv * (a.norm_w && ch0 < a.c ? a.norm_w[ch0 + v] : 1.f);
    }
  }
  finish_rotate_store<T, VEC, CPL>(a, y, gi, LPE, th, pos, op);
}

// Rows of entry e of sequence b: CSA [b-half (m rows, when present), a-half (m rows)];
// HCA the m rows of block e. Returns the pointers of logical row r.
template <typename T>
__device__ __forceinline__ void entry_row(const CompressArgs& a, int b, int64_t e, int r, const T*& cp,
                                          const T*& zp, const T*& bp) {
  const int m = a.m;
  const int64_t seq = (int64_t)b * a.T * a.c;
  if (a.csa) {
    const int p = r % m;
    if (r < m) {  // b-half: block e-1 (or the previous chunk's tail)
      if (e > 0) {
        const int64_t row = (e - 1) * m + p;
        cp = (const T*)a.Cb + seq + row * a.c;
        zp = (const T*)a.Zb + seq + row * a.c;
      } else {
        cp = (const T*)a.prev_Cb + ((int64_t)b * m + p) * a.c;
        zp = (const T*)a.prev_Zb + ((int64_t)b * m + p) * a.c;
      }
      bp = (const T*)a.B + (int64_t)p * a.c;
    } else {
      const int64_t row = e * m + p;
      cp = (const T*)a.Ca + seq + row * a.c;
      zp = (const T*)a.Za + seq + row * a.c;
      bp = (const T*)a.B + (int64_t)(m + p) * a.c;
    }
  } else {
    const int64_t row = e * m + r;
    cp = (const T*)a.Ca + seq + row * a.c;
    zp = a.Za ? (const T*)a.Za + seq + row * a.c : nullptr;
    bp = a.B ? (const T*)a.B + (int64_t)r * a.c : nullptr;
  }
}

__device__ __forceinline__ void entry_rows(const CompressArgs& a, int64_t e, int& first, int& nrows) {
  const bool has_b = a.csa && (e > 0 || a.prev_Cb != nullptr);
  nrows = a.csa ? (has_b ? 2 * a.m : a.m) : a.m;
  first = a.csa ? (has_b ? 0 : a.m) : 0;
}

template <int VEC>
__device__ __forceinline__ void softmax_step(float (&mx)[VEC], float (&sm)[VEC], float (&acc)[VEC],
                                             const float (&zv)[VEC], const float (&cv)[VEC]) {
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const float nm = fmaxf(mx[v], zv[v]);
    const float sc = __expf(mx[v] - nm);  // exp(-inf) = 0 on the first row
    const float e = __expf(zv[v] - nm);
    sm[v] = sm[v] * sc + e;
    acc[v] = acc[v] * sc + e * cv[v];
    mx[v] = nm;
  }
}

// One row per entry (m = 1): the softmax over a single row is that row. A lane group takes
// EPL rows per pass, all loads issued before any use.
template <typename T, int VEC, int CPL, int EPL>
__global__ __launch_bounds__(256) void compress_rows_kernel(CompressArgs a) {
  const int lane = threadIdx.x & 63;
  const int LPE = a.lpe, gi = lane & (LPE - 1), gpw = 64 / LPE;
  const int groups = a.c / VEC;
  const int64_t task0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * gpw + lane / LPE;
  const int64_t ntask = (int64_t)gridDim.x * 4 * gpw;
  const int64_t n_tot = (int64_t)a.n_out * a.batch;
  double th[CPL][VEC / 2];
  rope_table<VEC, CPL>(a, gi, LPE, th);
  for (int64_t t = task0 * EPL; t < n_tot; t += ntask * EPL) {
    float y[EPL][CPL][VEC];
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const int64_t el = t + q < n_tot ? t + q : n_tot - 1;
      const int b = (int)(el / a.n_out);
      const int64_t e = el % a.n_out;
      const T* cp = (const T*)a.Ca + ((int64_t)b * a.T + e) * a.c;
#pragma unroll
      for (int cg = 0; cg < CPL; ++cg) {
        const int g = gi + LPE * cg;
        if (g < groups) load_vec<T, VEC>(cp + g * VEC, y[q][cg]);
        else
#pragma unroll
          for (int v = 0; v < VEC; ++v) y[q][cg][v] = 0.f;
      }
    }
    // RMSNorm of the EPL rows together: their butterfly reductions are independent, so the
    // shuffles of different rows overlap instead of running one row after another
    if (a.apply_norm) {
      float ss[EPL];
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        ss[q] = 0.f;
#pragma unroll
        for (int cg = 0; cg < CPL; ++cg)
#pragma unroll
          for (int v = 0; v < VEC; ++v) ss[q] += y[q][cg][v] * y[q][cg][v];
      }
      for (int o = LPE >> 1; o > 0; o >>= 1)
#pragma unroll
        for (int q = 0; q < EPL; ++q) ss[q] += __shfl_xor(ss[q], o, 64);
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        const float inv = rsqrtf(ss[q] / (float)a.c + a.eps);
#pragma unroll
        for (int cg = 0; cg < CPL; ++cg) {
          const int ch0 = (gi + LPE * cg) * VEC;
#pragma unroll
          for (int v = 0; v < VEC; ++v) y[q][cg][v] *= inv * (a.norm_w && ch0 < a.c ? a.norm_w[ch0 + v] : 1.f);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      if (t + q >= n_tot) break;
      const int b = (int)((t + q) / a.n_out);
      const int64_t e = (t + q) % a.n_out;
      finish_rotate_store<T, VEC, CPL>(a, y[q], gi, LPE, th, a.pos0 + e,
                                       (T*)a.out + ((int64_t)b * a.out_ld + e) * a.c);
    }
  }
}

// 16-byte vector of VEC elements, kept packed until used (4 registers for 8 bf16 or 4 fp32 values).
template <typename T, int VEC>
__device__ __forceinline__ u32x4 load16(const T* p) {
  static_assert(sizeof(T) * VEC == 16, "one 16-byte load per channel group");
  return *reinterpret_cast<const u32x4*>(p);
}

template <typename T, int VEC>
__device__ __forceinline__ void unpack16(const u32x4& r, float (&out)[VEC]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(r[i] << 16);
      out[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(r[i]);
  }
}

// 2 .. 8 rows per entry (CSA with m <= 4): a lane group per entry; every row's C, Z and bias vector
// is loaded (24 loads per lane for 8 rows, packed) before the online softmax runs over them.
template <typename T, int VEC, int CPL>
__global__ __launch_bounds__(256) void compress_pool8_kernel(CompressArgs a) {
  const int lane = threadIdx.x & 63;
  const int LPE = a.lpe, gi = lane & (LPE - 1), gpw = 64 / LPE;
  const int groups = a.c / VEC;
  const int64_t task0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * gpw + lane / LPE;
  const int64_t ntask = (int64_t)gridDim.x * 4 * gpw;
  const int64_t n_tot = (int64_t)a.n_out * a.batch;
  double th[CPL][VEC / 2];
  rope_table<VEC, CPL>(a, gi, LPE, th);
  for (int64_t el = task0; el < n_tot; el += ntask) {
    const int b = (int)(el / a.n_out);
    const int64_t e = el % a.n_out;
    int first, nrows;
    entry_rows(a, e, first, nrows);
    u32x4 craw[8][CPL], zraw[8][CPL], braw[8][CPL];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = first + (i < nrows ? i : nrows - 1);
      const T *cp, *zp, *bp;
      entry_row<T>(a, b, e, r, cp, zp, bp);
#pragma unroll
      for (int cg = 0; cg < CPL; ++cg) {
        const int g = gi + LPE * cg < groups ? gi + LPE * cg : groups - 1;
        craw[i][cg] = load16<T, VEC>(cp + g * VEC);
        zraw[i][cg] = zp ? load16<T, VEC>(zp + g * VEC) : u32x4{0u, 0u, 0u, 0u};
        braw[i][cg] = bp ? load16<T, VEC>(bp + g * VEC) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    float mx[CPL][VEC], sm[CPL][VEC], acc[CPL][VEC];
#pragma unroll
    for (int cg = 0; cg < CPL; ++cg)
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        mx[cg][v] = -INFINITY;
        sm[cg][v] = 0.f;
        acc[cg][v] = 0.f;
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i >= nrows) break;
#pragma unroll
      for (int cg = 0; cg < CPL; ++cg) {
        float cv[VEC], zv[VEC], bv[VEC];
        unpack16<T, VEC>(craw[i][cg], cv);
        unpack16<T, VEC>(zraw[i][cg], zv);
        unpack16<T, VEC>(braw[i][cg], bv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) zv[v] += bv[v];
        softmax_step<VEC>(mx[cg], sm[cg], acc[cg], zv, cv);
      }
    }
    float y[CPL][VEC];
#pragma unroll
    for (int cg = 0; cg < CPL; ++cg)
#pragma unroll
      for (int v = 0; v < VEC; ++v) y[cg][v] = acc[cg][v] / sm[cg][v];
    finish_entry<T, VEC, CPL>(a, y, gi, LPE, th, a.pos0 + e * a.m, (T*)a.out + ((int64_t)b * a.out_ld + e) * a.c);
  }
}

// 9 .. 32 rows per entry: a lane group per entry, online softmax in registers, rows four at a time.
template <typename T, int VEC, int CPL>
__global__ __launch_bounds__(256) void compress_pool_kernel(CompressArgs a) {
  constexpr int RB = 4;
  const int lane = threadIdx.x & 63;
  const int LPE = a.lpe, gi = lane & (LPE - 1), gpw = 64 / LPE;
  const int groups = a.c / VEC;
  const int64_t task0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * gpw + lane / LPE;
  const int64_t ntask = (int64_t)gridDim.x * 4 * gpw;
  const int64_t n_tot = (int64_t)a.n_out * a.batch;
  double th[CPL][VEC / 2];
  rope_table<VEC, CPL>(a, gi, LPE, th);
  for (int64_t el = task0; el < n_tot; el += ntask) {
    const int b = (int)(el / a.n_out);
    const int64_t e = el % a.n_out;
    int first, nrows;
    entry_rows(a, e, first, nrows);
    float mx[CPL][VEC], sm[CPL][VEC], acc[CPL][VEC];
#pragma unroll
    for (int cg = 0; cg < CPL; ++cg)
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        mx[cg][v] = -INFINITY;
        sm[cg][v] = 0.f;
        acc[cg][v] = 0.f;
      }
    for (int r0 = 0; r0 < nrows; r0 += RB) {
      float cv[RB][CPL][VEC], zv[RB][CPL][VEC];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int r = first + (r0 + i < nrows ? r0 + i : nrows - 1);
        const T *cp, *zp, *bp;
        entry_row<T>(a, b, e, r, cp, zp, bp);
#pragma unroll
        for (int cg = 0; cg < CPL; ++cg) {
          const int g = gi + LPE * cg < groups ? gi + LPE * cg : groups - 1;
          load_vec<T, VEC>(cp + g * VEC, cv[i][cg]);
          if (zp) {
            load_vec<T, VEC>(zp + g * VEC, zv[i][cg]);
          } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) zv[i][cg][v] = 0.f;
          }
          if (bp) {
            float bv[VEC];
            load_vec<T, VEC>(bp + g * VEC, bv);
#pragma unroll
            for (int v = 0; v < VEC; ++v) zv[i][cg][v] += bv[v];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (r0 + i >= nrows) break;
#pragma unroll
        for (int cg = 0; cg < CPL; ++cg) softmax_step<VEC>(mx[cg], sm[cg], acc[cg], zv[i][cg], cv[i][cg]);
      }
    }
    float y[CPL][VEC];
#pragma unroll
    for (int cg = 0; cg < CPL; ++cg)
#pragma unroll
      for (int v = 0; v < VEC; ++v) y[cg][v] = acc[cg][v] / sm[cg][v];
    finish_entry<T, VEC, CPL>(a, y, gi, LPE, th, a.pos0 + e * a.m, (T*)a.out + ((int64_t)b * a.out_ld + e) * a.c);
  }
}

// More than 32 rows per entry: a workgroup of NW waves per entry; wave w takes rows w, w + NW,
// ...; wave 0 merges the partial softmaxes in wave order and finishes the entry.
template <typename T, int VEC, int CPL, int NW>
__global__ __launch_bounds__(NW * 64) void compress_block_kernel(CompressArgs a) {
  constexpr int W = CPL * VEC;  // floats per lane
  __shared__ __attribute__((aligned(16))) float part[3][NW][64 * W];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int groups = a.c / VEC;
  const int64_t e = blockIdx.x;
  const int b = blockIdx.y;
  int first, nrows;
  entry_rows(a, e, first, nrows);
  float mx[CPL][VEC], sm[CPL][VEC], acc[CPL][VEC];
#pragma unroll
  for (int cg = 0; cg < CPL; ++cg)
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      mx[cg][v] = -INFINITY;
      sm[cg][v] = 0.f;
      acc[cg][v] = 0.f;
    }
  // RB rows per wave per round, every load of the round issued before the first softmax step
  // (raw 16-byte pieces, widened at use): a 128-row entry at 8 waves is one round trip
  static_assert(VEC * sizeof(T) == 16, "16-byte pieces");
  constexpr int RB = (NW >= 16 ? 8 : 16) / CPL;  // 48 or 24 loads per lane in flight
  for (int r0 = wave; r0 < nrows; r0 += NW * RB) {
    uint4 craw[RB][CPL], zraw[RB][CPL], braw[RB][CPL];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int rr = r0 + i * NW;
      const int r = first + (rr < nrows ? rr : r0);
      const T *cp, *zp, *bp;
      entry_row<T>(a, b, e, r, cp, zp, bp);
#pragma unroll
      for (int cg = 0; cg < CPL; ++cg) {
        const int g = lane + 64 * cg < groups ? lane + 64 * cg : groups - 1;
        craw[i][cg] = *reinterpret_cast<const uint4*>(cp + g * VEC);
        zraw[i][cg] = zp ? *reinterpret_cast<const uint4*>(zp + g * VEC) : uint4{0u, 0u, 0u, 0u};
        braw[i][cg] = bp ? *reinterpret_cast<const uint4*>(bp + g * VEC) : uint4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (r0 + i * NW >= nrows) break;
#pragma unroll
      for (int cg = 0; cg < CPL; ++cg) {
        float cv[VEC], zv[VEC], bv[VEC];
        unpack16<T, VEC>(craw[i][cg], cv);
        unpack16<T, VEC>(zraw[i][cg], zv);
        unpack16<T, VEC>(braw[i][cg], bv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) zv[v] += bv[v];  // an absent Z or B reads as +0
        softmax_step<VEC>(mx[cg], sm[cg], acc[cg], zv, cv);
      }
    }
  }
#pragma unroll
  for (int cg = 0; cg < CPL; ++cg)
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      part[0][wave][lane * W + cg * VEC + v] = mx[cg][v];
      part[1][wave][lane * W + cg * VEC + v] = sm[cg][v];
      part[2][wave][lane * W + cg * VEC + v] = acc[cg][v];
    }
  __syncthreads();
  if (wave != 0) return;
  double th[CPL][VEC / 2];
  rope_table<VEC, CPL>(a, lane, 64, th);
  float y[CPL][VEC];
#pragma unroll
  for (int cg = 0; cg < CPL; ++cg)
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const int o = lane * W + cg * VEC + v;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, part[0][w][o]);
      float S = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = part[0][w][o];
        if (mw == -INFINITY) continue;  // the wave saw no rows
        const float sc = __expf(mw - M);
        S += part[1][w][o] * sc;
        A += part[2][w][o] * sc;
      }
      y[cg][v] = A / S;
    }
  finish_entry<T, VEC, CPL>(a, y, lane, 64, th, a.pos0 + e * a.m, (T*)a.out + ((int64_t)b * a.out_ld + e) * a.c);
}

// FP8 KV storage of compressed entries ("Paper Breakdown: DeepSeek-V4", §2.3.4
// "Efficiency": FP8 for the non-RoPE dims, BF16 for the RoPE dims). One wave per
// entry: the first d - rope dims become E4M3 codes of x * 2^-e, e the smallest
// integer with max |x| <= 448 * 2^e (exact scaling), the RoPE dims are kept as
// bf16, and 2^e is the entry's scale.
template <typename T>
__global__ __launch_bounds__(256) void quantize_kv_fp8_kernel(const T* x, int64_t n, int d, int rope,
                                                             uint8_t* out, float* scales, int64_t out_ld) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (r >= n) return;
  const T* xr = x + ((int64_t)b * n + r) * d;
  const int nope = d - rope, nch = d / 8;
  float v[2][8];
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = lane + 64 * q;
    if (c < nch) {
      load_vec<T, 8>(xr + 8 * c, v[q]);
      if (8 * c < nope)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[q][i]));
    }
  }
  amax = wave_max(amax);
  int e = 0;
  if (amax > 0.f) {
    int E;
    frexpf(amax, &E);  // amax in [2^(E-1), 2^E)
    e = E - 9;         // amax * 2^-e in [256, 512)
    if (ldexpf(amax, -e) > 448.f) e += 1;
  }
  uint8_t* orow = out + ((int64_t)b * out_ld + r) * (nope + 2 * rope);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = lane + 64 * q;
    if (c >= nch) continue;
    if (8 * c < nope) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0 |= e4m3_code(ldexpf(v[q][i], -e)) << (8 * i);
        w1 |= e4m3_code(ldexpf(v[q][4 + i], -e)) << (8 * i);
      }
      *reinterpret_cast<uint2*>(orow + 8 * c) = make_uint2(w0, w1);
    } else {
      uint4 o;
      o.x = pack_bf16x2(v[q][0], v[q][1]);
      o.y = pack_bf16x2(v[q][2], v[q][3]);
      o.z = pack_bf16x2(v[q][4], v[q][5]);
      o.w = pack_bf16x2(v[q][6], v[q][7]);
      *reinterpret_cast<uint4*>(orow + nope + 2 * (8 * c - nope)) = o;
    }
  }
  if (lane == 0) scales[(int64_t)b * out_ld + r] = ldexpf(1.f, e);
}

template <typename T, int VEC, int CPL>
static void launch_compress_t(CompressArgs& a, int batch, hipStream_t st) {
  const int groups = a.c / VEC;
  int lpe = 1;
  while (lpe < groups && lpe < 64) lpe <<= 1;
  a.lpe = lpe;
  const int rows = a.csa ? 2 * a.m : a.m;
  const int64_t n_tot = (int64_t)a.n_out * batch;
  const int gpw = 64 / lpe;
  if (rows > 32) {
    constexpr int NW = 64 / (CPL * VEC) >= 4 ? 64 / (CPL * VEC) : 4;
    hipLaunchKernelGGL((compress_block_kernel<T, VEC, CPL, NW>), dim3((unsigned)a.n_out, (unsigned)batch),
                       dim3(NW * 64), 0, st, a);
    return;
  }
  // the row and pool kernels take entries (b, e) as one index over batch * n_out, grid-strided
  a.batch = batch;
  // window rows: four per lane group in flight for long calls; one each when the call is short
  // (decode), so that the rows' dependent epilogues run in parallel groups
  const int epl = rows == 1 && n_tot > 4096 ? 4 : 1;
  const int64_t waves = ceil_div(ceil_div(n_tot, epl), gpw);
  const int64_t wgs = std::min<int64_t>(ceil_div(waves, 4), 65535);
  if (rows == 1 && epl == 4)
    hipLaunchKernelGGL((compress_rows_kernel<T, VEC, CPL, 4>), dim3((unsigned)wgs), dim3(256), 0, st, a);
  else if (rows == 1)
    hipLaunchKernelGGL((compress_rows_kernel<T, VEC, CPL, 1>), dim3((unsigned)wgs), dim3(256), 0, st, a);
  else if (rows <= 8)
    hipLaunchKernelGGL((compress_pool8_kernel<T, VEC, CPL>), dim3((unsigned)wgs), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((compress_pool_kernel<T, VEC, CPL>), dim3((unsigned)wgs), dim3(256), 0, st, a);
}

static int launch_compress(CompressArgs& a, int batch, int dtype, hipStream_t st) {
  if (a.n_out == 0 || batch == 0) return CSKV_OK;
  if (dtype == CSKV_BF16) {
    if (a.c <= 512) launch_compress_t<bf16, 8, 1>(a, batch, st);
    else launch_compress_t<bf16, 8, 2>(a, batch, st);
  } else {
    if (a.c <= 256) launch_compress_t<float, 4, 1>(a, batch, st);
    else if (a.c <= 512) launch_compress_t<float, 4, 2>(a, batch, st);
    else launch_compress_t<float, 4, 4>(a, batch, st);
  }
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

static int check_common(int batch, int64_t T, int c, int m, int64_t pos0, int apply_norm, float eps,
                        int rope_dims, float rope_base, int dtype) {
  if (dtype != CSKV_BF16 && dtype != CSKV_F32) return CSKV_ERR_BAD_DTYPE;
  if (batch < 0 || T < 0 || m < 1 || pos0 < 0) return CSKV_ERR_BAD_SHAPE;
  if (c < 8 || c > CSKV_MAX_DIM || (c % 8) != 0) return CSKV_ERR_BAD_SHAPE;
  if (pos0 % m != 0) return CSKV_ERR_BAD_SHAPE;
  if (rope_dims < 0 || rope_dims > c || (rope_dims & 1)) return CSKV_ERR_BAD_SHAPE;
  if (rope_dims > 0 && !(rope_base > 0.f)) return CSKV_ERR_INVALID_ARG;
  if (apply_norm && !(eps > 0.f)) return CSKV_ERR_INVALID_ARG;
  if ((int64_t)batch * T > ((int64_t)1 << 40)) return CSKV_ERR_BAD_SHAPE;
  return CSKV_OK;
}

}  // namespace cskv

using namespace cskv;

extern "C" int csa_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb,
                            const void* B, const void* prev_Cb, const void* prev_Zb, int batch,
                            int64_t T, int c, int m, int64_t pos0, int apply_norm,
                            const float* norm_w, float eps, int rope_dims, float rope_base,
                            void* out, int64_t out_ld, int dtype, void* stream) {
  int st = check_common(batch, T, c, m, pos0, apply_norm, eps, rope_dims, rope_base, dtype);
  if (st) return st;
  if (m > 128) return CSKV_ERR_UNSUPPORTED;
  const int64_t n_out = T / m;
  if (out_ld == 0) out_ld = n_out;
  if (out_ld < n_out) return CSKV_ERR_BAD_SHAPE;
  if (n_out > 0x7fffffff) return CSKV_ERR_BAD_SHAPE;
  if (batch > 0 && n_out > 0) {
    if (!Ca || !Cb || !Za || !Zb || !B || !out) return CSKV_ERR_INVALID_ARG;
    if ((prev_Cb == nullptr) != (prev_Zb == nullptr)) return CSKV_ERR_INVALID_ARG;
    if (!aligned16(Ca, Cb, Za, Zb, B, prev_Cb, prev_Zb, out, norm_w)) return CSKV_ERR_MISALIGNED;
  }
  CompressArgs a{};
  a.Ca = Ca; a.Cb = Cb; a.Za = Za; a.Zb = Zb; a.B = B;
  a.prev_Cb = prev_Cb; a.prev_Zb = prev_Zb; a.out = out; a.norm_w = norm_w;
  a.T = T; a.pos0 = pos0; a.out_ld = out_ld; a.c = c; a.m = m; a.n_out = (int)n_out; a.csa = 1;
  a.apply_norm = apply_norm; a.rope_dims = rope_dims; a.eps = eps; a.rope_base = rope_base;
  fill_rope_table(a.rope, rope_base, rope_dims);
  return launch_compress(a, batch, dtype, (hipStream_t)stream);
}

extern "C" int hca_compress(const void* C, const void* Z, const void* B, int batch, int64_t T,
                            int c, int m, int64_t pos0, int apply_norm, const float* norm_w,
                            float eps, int rope_dims, float rope_base, void* out, int64_t out_ld,
                            int dtype, void* stream) {
  int st = check_common(batch, T, c, m, pos0, apply_norm, eps, rope_dims, rope_base, dtype);
  if (st) return st;
  if (m > 4096) return CSKV_ERR_UNSUPPORTED;
  const int64_t n_out = T / m;
  if (out_ld == 0) out_ld = n_out;
  if (out_ld < n_out) return CSKV_ERR_BAD_SHAPE;
  if (n_out > 0x7fffffff) return CSKV_ERR_BAD_SHAPE;
  if (batch > 0 && n_out > 0) {
    if (!C || !out) return CSKV_ERR_INVALID_ARG;
    if (!aligned16(C, Z, B, out, norm_w)) return CSKV_ERR_MISALIGNED;
  }
  CompressArgs a{};
  a.Ca = C; a.Za = Z; a.B = B; a.out = out; a.norm_w = norm_w;
  a.T = T; a.pos0 = pos0; a.out_ld = out_ld; a.c = c; a.m = m; a.n_out = (int)n_out; a.csa = 0;
  a.apply_norm = apply_norm; a.rope_dims = rope_dims; a.eps = eps; a.rope_base = rope_base;
  fill_rope_table(a.rope, rope_base, rope_dims);
  return launch_compress(a, batch, dtype, (hipStream_t)stream);
}

extern "C" int cskv_quantize_kv_fp8(const void* x, int batch, int64_t n, int d, int rope_dims, int dtype,
                                    uint8_t* out, float* scales, int64_t out_ld, void* stream) {
  if (dtype != CSKV_BF16 && dtype != CSKV_F32) return CSKV_ERR_BAD_DTYPE;
  if (batch < 0 || n < 0 || d < 16 || d > CSKV_MAX_DIM || rope_dims < 0 || rope_dims > d) return CSKV_ERR_BAD_SHAPE;
  if ((d - rope_dims) % 16 != 0 || rope_dims % 8 != 0) return CSKV_ERR_BAD_SHAPE;
  if (out_ld == 0) out_ld = n;
  if (out_ld < n || ceil_div(n, (int64_t)4) > 0x7fffffff) return CSKV_ERR_BAD_SHAPE;
  if (batch == 0 || n == 0) return CSKV_OK;
  if (!x || !out || !scales) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(x, out)) return CSKV_ERR_MISALIGNED;
  if (((uintptr_t)scales) % 4 != 0) return CSKV_ERR_MISALIGNED;
  dim3 grid((unsigned)ceil_div(n, (int64_t)4), (unsigned)batch);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == CSKV_BF16)
    hipLaunchKernelGGL(quantize_kv_fp8_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)x, n, d, rope_dims, out,
                       scales, out_ld);
  else
    hipLaunchKernelGGL(quantize_kv_fp8_kernel<float>, grid, dim3(256), 0, st, (const float*)x, n, d, rope_dims, out,
                       scales, out_ld);
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}
