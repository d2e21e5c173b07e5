// Device-side helpers shared by the gfx950 kernels: storage types, MFMA
// operand vectors, wave reductions and the rotary angle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cskv {

// bfloat16 is carried as raw 16-bit storage; arithmetic is always fp32.
struct bf16 {
  uint16_t v;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 r = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <>
struct Elem<bf16> {
  static __device__ __forceinline__ float load(const bf16* p, int64_t i) { return bf2f(p[i].v); }
  static __device__ __forceinline__ void store(bf16* p, int64_t i, float x) { p[i].v = f2bf(x); }
};

// The VEC elements of one 16-byte piece (8 bf16 or 4 fp32 values) as fp32.
template <typename T, int VEC>
__device__ __forceinline__ void unpack16(const uint4 r, float* out) {
  static_assert(VEC * sizeof(T) == 16, "16-byte piece");
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(T) == 2) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    } else {
      out[i] = __uint_as_float(w[i]);
    }
  }
}

// Load VEC consecutive elements (VEC * sizeof(T) bytes, aligned) as fp32.
template <typename T, int VEC>
__device__ __forceinline__ void load_vec(const T* p, float* out) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (VEC == 8) {
      uint4 r = *reinterpret_cast<const uint4*>(p);
      uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else if constexpr (VEC == 4) {
      uint2 r = *reinterpret_cast<const uint2*>(p);
      out[0] = __uint_as_float(r.x << 16);
      out[1] = __uint_as_float(r.x & 0xffff0000u);
      out[2] = __uint_as_float(r.y << 16);
      out[3] = __uint_as_float(r.y & 0xffff0000u);
    } else if constexpr (VEC == 2) {
      uint32_t r = *reinterpret_cast<const uint32_t*>(p);
      out[0] = __uint_as_float(r << 16);
      out[1] = __uint_as_float(r & 0xffff0000u);
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) out[i] = bf2f(reinterpret_cast<const uint16_t*>(p)[i]);
    }
  } else {
    if constexpr (VEC == 4) {
      float4 r = *reinterpret_cast<const float4*>(p);
      out[0] = r.x; out[1] = r.y; out[2] = r.z; out[3] = r.w;
    } else if constexpr (VEC == 2) {
      float2 r = *reinterpret_cast<const float2*>(p);
      out[0] = r.x; out[1] = r.y;
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) out[i] = reinterpret_cast<const float*>(p)[i];
    }
  }
}

template <typename T, int VEC>
__device__ __forceinline__ void store_vec(T* p, const float* in) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (VEC == 8) {
      uint4 r;
      r.x = pack_bf16x2(in[0], in[1]);
      r.y = pack_bf16x2(in[2], in[3]);
      r.z = pack_bf16x2(in[4], in[5]);
      r.w = pack_bf16x2(in[6], in[7]);
      *reinterpret_cast<uint4*>(p) = r;
    } else if constexpr (VEC == 4) {
      uint2 r;
      r.x = pack_bf16x2(in[0], in[1]);
      r.y = pack_bf16x2(in[2], in[3]);
      *reinterpret_cast<uint2*>(p) = r;
    } else if constexpr (VEC == 2) {
      *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(in[0], in[1]);
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) reinterpret_cast<uint16_t*>(p)[i] = f2bf(in[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i) reinterpret_cast<float*>(p)[i] = in[i];
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Rotary pair angles theta_j = base^(-2j / rope_dims) of the first ROPE_TABLE pairs, formed on
// the host in fp64 and passed in the kernel arguments, so that kernels evaluate no fp64 power
// (a long dependent chain) for RoPE widths up to 2 * ROPE_TABLE; wider ones fall back to it.
constexpr int ROPE_TABLE = 64;
struct RopeTable {
  double th[ROPE_TABLE];
};

__host__ inline void fill_rope_table(RopeTable& t, float base, int rope_dims) {
  for (int j = 0; j < ROPE_TABLE; ++j)
    t.th[j] = (rope_dims > 0 && j < rope_dims / 2) ? __builtin_pow((double)base, -2.0 * j / (double)rope_dims) : 0.0;
}

__device__ __forceinline__ double rope_theta_of(const RopeTable& t, int j, int rope_dims, float base) {
  return j < ROPE_TABLE ? t.th[j] : pow((double)base, -2.0 * j / (double)rope_dims);
}

// Rotary angle for pair j of a rope_dims-wide block at position pos: pos * base^(-2j/rope_dims),
// formed and reduced in fp64 on the device (kernels at their register limit use this form: the
// table lookup below changed their register allocation).
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int j, int rope_dims, float base, float* c, float* s) {
  const double theta = pow((double)base, -2.0 * j / (double)rope_dims);
  double a = (double)pos * theta;
  const double two_pi = 6.283185307179586476925286766559;
  a = a - two_pi * rint(a / two_pi);  // |a| <= pi, exact to ~1e-16 relative of pos * theta
  sincosf((float)a, s, c);
}

// cos / sin of pos * theta_j, the angle reduced modulo 2 pi in fp64 (positions to 2^20 and beyond
// keep full fp32 accuracy).
__device__ __forceinline__ void rope_cos_sin_t(const RopeTable& t, int64_t pos, int j, int rope_dims, float base,
                                               float* c, float* s) {
  const double inv_two_pi = 0.15915494309189533576888376337251;
  const double two_pi = 6.283185307179586476925286766559;
  double a = (double)pos * rope_theta_of(t, j, rope_dims, base);
  a = __builtin_fma(-two_pi, rint(a * inv_two_pi), a);
  sincosf((float)a, s, c);
}

// E4M3 code of y: nearest value, ties to the even code, saturating at +-448;
// the sign bit is set for negative y (and -0.0).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  uint32_t c;
  if (a < 0.015625f) {
    c = (uint32_t)rintf(a * 512.f);  // subnormal steps of 2^-9 (8 is the smallest normal)
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);  // round the fp32 mantissa to 3 bits, ties to even
    c = (u >> 20) - (120u << 3);       // exponent bias 127 -> 7
  }
  return sign | c;
}

// Order-preserving map of an fp32 score to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace cskv
