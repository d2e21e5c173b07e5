// KV compression kernels for gfx950.
//
// CSA compressor ("Paper Breakdown: DeepSeek-V4", §2.3.1 KV Compression):
// entry i pools 2m rows -- the m b-stream rows of block i-1 and the m
// a-stream rows of block i -- under one per-channel softmax of Z + B.
// HCA compressor (§2.3.2): entry i pools the m' rows of block i of one stream.
// Both are followed by optional RMSNorm over the channels and RoPE on the
// last rope_dims channels (§2.3.3) at the entry's position.
//
// One workgroup (256 threads) builds one entry of one sequence. Threads are
// laid out as [row group][channel group]: a channel group is VEC contiguous
// channels (one 16-byte load per row), row groups split the block's rows.
// Each thread keeps an online softmax (max, sum, weighted sum) per channel;
// the row groups are merged through LDS in a fixed order, so the result is
// deterministic. The kernel is HBM-streaming: every input byte is read once.
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
  int clp;  // channel groups per row group (power of two)
};

template <typename T, int VEC>
__global__ __launch_bounds__(256) void compress_kernel(CompressArgs a) {
  constexpr int NT = 256;
  __shared__ float part[3][NT * VEC];
  __shared__ float red[NT / 64];

  const int entry = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int CL = a.c / VEC;
  const int g = tid % a.clp;
  const int rg = tid / a.clp;
  const int RG = NT / a.clp;
  const bool active = g < CL;
  const int ch0 = g * VEC;
  const int64_t seq = (int64_t)b * a.T * a.c;

  float mx[VEC], sm[VEC], acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    mx[v] = -INFINITY;
    sm[v] = 0.f;
    acc[v] = 0.f;
  }

  // Rows of this entry's softmax: CSA: [b-half (m rows, if present), a-half (m rows)];
  // HCA: the m rows of block `entry`.
  const int m = a.m;
  bool has_b = false;
  if (a.csa) has_b = entry > 0 || a.prev_Cb != nullptr;
  const int nrows = a.csa ? (has_b ? 2 * m : m) : m;
  const int first = a.csa ? (has_b ? 0 : m) : 0;  // logical row index of the first row

  if (active) {
    for (int r = first + rg; r < first + nrows; r += RG) {
      const T* cp;
      const T* zp;
      const T* bp = nullptr;
      if (a.csa) {
        const int p = r % m;
        if (r < m) {  // b-half: block entry-1 (or previous chunk's tail)
          if (entry > 0) {
            const int64_t row = (int64_t)(entry - 1) * m + p;
            cp = (const T*)a.Cb + seq + row * a.c;
            zp = (const T*)a.Zb + seq + row * a.c;
          } else {
            cp = (const T*)a.prev_Cb + ((int64_t)b * m + p) * a.c;
            zp = (const T*)a.prev_Zb + ((int64_t)b * m + p) * a.c;
          }
          bp = (const T*)a.B + (int64_t)p * a.c;
        } else {
          const int64_t row = (int64_t)entry * m + p;
          cp = (const T*)a.Ca + seq + row * a.c;
          zp = (const T*)a.Za + seq + row * a.c;
          bp = (const T*)a.B + (int64_t)(m + p) * a.c;
        }
      } else {
        const int64_t row = (int64_t)entry * m + r;
        cp = (const T*)a.Ca + seq + row * a.c;
        zp = a.Za ? (const T*)a.Za + seq + row * a.c : nullptr;
        bp = a.B ? (const T*)a.B + (int64_t)r * a.c : nullptr;
      }
      float cv[VEC], zv[VEC], bv[VEC];
      load_vec<T, VEC>(cp + ch0, cv);
      if (zp) {
        load_vec<T, VEC>(zp + ch0, zv);
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) zv[v] = 0.f;
      }
      if (bp) {
        load_vec<T, VEC>(bp + ch0, bv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) zv[v] += bv[v];
      }
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
  }

  // Merge row groups in a fixed order (row group 0 first). Partials are stored channel-major
  // (element v of thread t at v * NT + t), so each store and read touches consecutive words.
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    part[0][v * NT + tid] = mx[v];
    part[1][v * NT + tid] = sm[v];
    part[2][v * NT + tid] = acc[v];
  }
  __syncthreads();

  float y[VEC];
  float ss = 0.f;
  if (rg == 0 && active) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      float M = -INFINITY;
      for (int q = 0; q < RG; ++q) M = fmaxf(M, part[0][v * NT + q * a.clp + g]);
      float S = 0.f, A = 0.f;
      for (int q = 0; q < RG; ++q) {
        const int o = v * NT + q * a.clp + g;
        const float mq = part[0][o];
        if (mq == -INFINITY) continue;  // row group saw no rows
        const float sc = __expf(mq - M);
        S += part[1][o] * sc;
        A += part[2][o] * sc;
      }
      y[v] = A / S;
      ss += y[v] * y[v];
    }
  }

  if (a.apply_norm) {
    // Block reduction of the sum of squares (fixed order over waves).
    float w = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = w;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < NT / 64; ++q) tot += red[q];
    const float inv = rsqrtf(tot / (float)a.c + a.eps);
    if (rg == 0 && active) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float gmul = a.norm_w ? a.norm_w[ch0 + v] : 1.f;
        y[v] = y[v] * inv * gmul;
      }
    }
  }

  if (rg == 0 && active) {
    const int rstart = a.c - a.rope_dims;
    if (a.rope_dims > 0 && ch0 + VEC > rstart) {
      const int64_t pos = a.pos0 + (int64_t)entry * m;
#pragma unroll
      for (int v = 0; v < VEC; v += 2) {
        const int ch = ch0 + v;
        if (ch >= rstart) {
          float cs, sn;
          rope_cos_sin(pos, (ch - rstart) >> 1, a.rope_dims, a.rope_base, &cs, &sn);
          const float x0 = y[v], x1 = y[v + 1];
          y[v] = x0 * cs - x1 * sn;
          y[v + 1] = x0 * sn + x1 * cs;
        }
      }
    }
    T* op = (T*)a.out + ((int64_t)b * a.out_ld + entry) * a.c + ch0;
    store_vec<T, VEC>(op, y);
  }
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

static int launch_compress(CompressArgs& a, int batch, int dtype, hipStream_t st) {
  if (a.n_out == 0 || batch == 0) return CSKV_OK;
  const int VEC = dtype == CSKV_BF16 ? 8 : 4;
  const int CL = a.c / VEC;
  int clp = 1;
  while (clp < CL) clp <<= 1;
  a.clp = clp;
  dim3 grid(a.n_out, batch), block(256);
  if (dtype == CSKV_BF16)
    hipLaunchKernelGGL((compress_kernel<bf16, 8>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((compress_kernel<float, 4>), grid, block, 0, st, a);
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
