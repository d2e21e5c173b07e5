// Lightning-indexer scoring on low-precision rows for gfx950: FP8 (OCP
// E4M3) and FP4 (OCP E2M1, two codes per byte).
//
// "Paper Breakdown: DeepSeek-V4", section 4, "Efficiency (§2.3.4)": the
// indexer computes in FP8 in V3.2 and in FP4 in V4 (infrastructure table:
// FP4 quantization-aware training of the indexer QK path). The pages name
// the precision only; here each row (one compressed key, or one (query,
// head) of the indexer queries) carries one fp32 scale. Since ReLU commutes
// with a positive scale,
//   I[t, s] = ks[s] * sum_h (w[t,h] * qs[t,h]) * ReLU(dq[t,h,:] . dk[s,:]),
// dq, dk the decoded codes, summed by v_mfma_f32_32x32x64_f8f6f4 (64
// products per output per instruction; format field 0 = E4M3, 4 = E2M1).
// E2M1 products are multiples of 1/4 below 36 and their sums stay exact;
// E4M3 sums are rounded inside the matrix core (groups of 8 products on a
// grid 2^-13 below the group's largest).
//
// The quantisers write the codes: per row, amax = max |x|, codes =
// FMT(x * (MAX / amax)) (nearest, ties to the even code, saturating) and
// scale = amax / MAX, MAX = 448 (E4M3) or 6 (E2M1); the quotient and product
// are correctly rounded fp32.
//
// MX-FP4 / MX-FP8 (the same E2M1 / E4M3 codes with block scales, as in the
// OCP Microscaling formats): every 32 consecutive values of a row share one
// E8M0 scale 2^(code - 127), the shared exponent being floor(log2 amax) - 2
// (E2M1's largest value is 1.5 * 2^2) or - 8 (E4M3: 1.75 * 2^8) over the
// block; codes = FMT(x / scale). The scaled MFMA applies them in hardware
// (dI = 128, 4 scale bytes per row): for E2M1 each lane's 16 operand bytes
// are one block (lane half h at k-step ks holds block 2h + ks), for E4M3 a
// block is bytes 16q .. 16q+15 of lanes l and l + 32 (block 2 ks + q), see
// op_off; each lane passes its row's scale bytes shifted so that the
// instruction's byte select picks the block. Only the head weight multiplies
// the ReLU; no key scale.
//
// The scoring kernels follow the bf16 ones: 8 queries per workgroup sharing
// 256-key LDS tiles copied straight from global memory for prefill; for
// decode, interleaved 32-key blocks per wave with coalesced loads turned into
// the MFMA layout through per-wave LDS rows. A key row is DI bytes (dI for
// E4M3, dI/2 for E2M1); each lane holds one contiguous half of it (the K
// dimension permuted identically in A and B: lane half h, k-step ks holds
// bytes h*DI/2 + OB*ks .. + OB, OB = 32 bytes for E4M3, 16 for E2M1).
#include "indexer.h"

namespace cskv {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int FMT_E4M3 = 0;  // format fields of v_mfma_f32_32x32x64_f8f6f4
constexpr int FMT_E2M1 = 4;

template <int FMT>
struct LowP {
  static constexpr int BITS = FMT == FMT_E2M1 ? 4 : 8;
  static constexpr int OB = 32 * BITS / 8;  // operand bytes per lane per k-step (32 values)
};

// One wave per row (4 rows per workgroup); dim % 4 == 0, dim <= 1024.
template <typename T>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T* x, int64_t rows, int dim, uint8_t* codes,
                                                          float* scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const T* xr = x + r * dim;
  const int nc = dim / 4;  // 4-element chunks: lane takes chunks lane, lane + 64, ...
  float v[16];
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = lane + 64 * q;
    if (c < nc) {
      load_vec<T, 4>(xr + 4 * c, &v[4 * q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(v[4 * q + e]));
    }
  }
  amax = wave_max(amax);
  const float inv = amax > 0.f ? __fdiv_rn(448.f, amax) : 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = lane + 64 * q;
    if (c < nc) {
      uint32_t w = 0;
      if (amax > 0.f)
#pragma unroll
        for (int e = 0; e < 4; ++e) w |= e4m3_code(v[4 * q + e] * inv) << (8 * e);
      *reinterpret_cast<uint32_t*>(codes + r * dim + 4 * c) = w;
    }
  }
  if (lane == 0) scales[r] = amax > 0.f ? __fdiv_rn(amax, 448.f) : 0.f;
}

// E2M1 code of y (values 0, 0.5, 1, 1.5, 2, 3, 4, 6): nearest, ties to the even
// code, saturating at +-6; bit 3 is the sign (set for negative y and -0.0).
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 28) & 0x8u;
  const float a = fabsf(y);
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.f);
  return sign | c;
}

// One wave per row (4 rows per workgroup); dim % 4 == 0, dim <= 1024. Element 2i of a
// row goes to the low nibble of byte i, element 2i + 1 to the high nibble.
template <typename T>
__global__ __launch_bounds__(256) void quantize_fp4_kernel(const T* x, int64_t rows, int dim, uint8_t* codes,
                                                          float* scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const T* xr = x + r * dim;
  const int nc = dim / 4;
  float v[16];
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = lane + 64 * q;
    if (c < nc) {
      load_vec<T, 4>(xr + 4 * c, &v[4 * q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(v[4 * q + e]));
    }
  }
  amax = wave_max(amax);
  const float inv = amax > 0.f ? __fdiv_rn(6.f, amax) : 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = lane + 64 * q;
    if (c < nc) {
      uint32_t w = 0;
      if (amax > 0.f)
#pragma unroll
        for (int e = 0; e < 4; ++e) w |= e2m1_code(v[4 * q + e] * inv) << (4 * e);
      *reinterpret_cast<uint16_t*>(codes + r * (dim / 2) + 2 * c) = (uint16_t)w;
    }
  }
  if (lane == 0) scales[r] = amax > 0.f ? __fdiv_rn(amax, 6.f) : 0.f;
}

// MX rows (E2M1 or E4M3 values): one wave per row, dim % 32 == 0, dim <= 1024. Lane groups of 8
// (4 values each) cover one 32-value block; codes as in quantize_fp4_kernel / quantize_fp8_kernel,
// one E8M0 byte per block; shared exponent floor(log2 amax) - EMAX, EMAX = 2 (E2M1) or 8 (E4M3).
template <typename T, int FMT>
__global__ __launch_bounds__(256) void quantize_mx_kernel(const T* x, int64_t rows, int dim, uint8_t* codes,
                                                         uint8_t* scales) {
  constexpr int EMAX = FMT == FMT_E2M1 ? 2 : 8;
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const T* xr = x + r * dim;
  const int nc = dim / 4;  // 4-value chunks: lane takes chunks lane, lane + 64, ...; 8 chunks per block
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = lane + 64 * q;
    if (64 * q >= nc) break;  // uniform: whole 64-chunk passes only (nc is a multiple of 8)
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (c < nc) load_vec<T, 4>(xr + 4 * c, v);
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    int code = 0;
    if (amax > 0.f) {
      int ex;
      (void)frexpf(amax, &ex);  // amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
      code = min(max(ex - 1 - EMAX + 127, 0), 254);
    }
    const float inv = ldexpf(1.f, 127 - code);  // 1 / scale, exact
    if (c < nc) {
      uint32_t w = 0;
      if constexpr (FMT == FMT_E2M1) {
        if (amax > 0.f)
#pragma unroll
          for (int e = 0; e < 4; ++e) w |= e2m1_code(v[e] * inv) << (4 * e);
        *reinterpret_cast<uint16_t*>(codes + r * (dim / 2) + 2 * c) = (uint16_t)w;
      } else {
        if (amax > 0.f)
#pragma unroll
          for (int e = 0; e < 4; ++e) w |= e4m3_code(v[e] * inv) << (8 * e);
        *reinterpret_cast<uint32_t*>(codes + r * dim + 4 * c) = w;
      }
      if ((c & 7) == 0) scales[r * (dim / 32) + c / 8] = (uint8_t)code;
    }
  }
}

// MFMA operand: 32 values = 32 bytes (E4M3) or 16 bytes (E2M1, upper registers unused).
template <int FMT>
__device__ __forceinline__ i32x8 load_op(const uint8_t* p) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
  if constexpr (FMT == FMT_E2M1) {
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
  } else {
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
}

template <int FMT>
__device__ __forceinline__ f32x16 mfma_lowp(const i32x8& a, const i32x8& b, const f32x16& c) {
  // same format for both operands; zero scales select the unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, 0, 0, 0);
}

// Byte offset within a row of the q-th 16-byte chunk of the operand that lane half h holds at
// k-step ks. Plain rows: one contiguous half row per lane half (h DI/2 + OB ks + 16 q). MX-FP8: the
// matrix core forms each 32-value scale block of a k-step from bytes 16q .. 16q+15 of lane l and of
// lane l + 32 (in-bounds probe on gfx950), so those hold values 64 ks + 32 q + 16 h .. +15 of the
// row: block q of k-step ks is the row's block 2 ks + q. (E2M1 blocks are one lane's 16 bytes.)
template <int FMT, int KS8, bool MX>
__device__ __forceinline__ int op_off(int h, int ks, int q) {
  constexpr int DI = 64 * KS8 * LowP<FMT>::BITS / 8;
  if constexpr (MX && FMT == FMT_E4M3) return 64 * ks + 32 * q + 16 * h;
  else return h * (DI / 2) + LowP<FMT>::OB * ks + 16 * q;
}

template <int FMT, int KS8, bool MX>
__device__ __forceinline__ i32x8 load_op_at(const uint8_t* row, int h, int ks) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(row + op_off<FMT, KS8, MX>(h, ks, 0));
  if constexpr (FMT == FMT_E2M1) {
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
  } else {
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row + op_off<FMT, KS8, MX>(h, ks, 1));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
}

// MX scale bytes of a row (4 bytes, dI = 128) as one lane's scale operand: E2M1 lane half h holds
// blocks 2h + ks (shift 16 h, byte select ks); E4M3 lane half h supplies block 2 ks + h (shift 8 h,
// byte select 2 ks).
template <int FMT>
__device__ __forceinline__ uint32_t mx_scale_word(uint32_t bytes, int h) {
  return bytes >> ((FMT == FMT_E2M1 ? 16 : 8) * h);
}

// Block-scaled product (MX) at k-step KS; sa, sb from mx_scale_word.
template <int FMT, int KS>
__device__ __forceinline__ f32x16 mfma_mx(const i32x8& a, const i32x8& b, const f32x16& c, uint32_t sa, uint32_t sb) {
  constexpr int SEL = FMT == FMT_E2M1 ? KS : 2 * KS;
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, SEL, (int)sa, SEL, (int)sb);
}

// Query operands (A) and head weights of query j; lane holds head lane%32 of each tile. Row
// scales (MX = false) are folded into the weights (w * qs); MX block scales go to qsx: the
// head row's 4 scale bytes shifted to this lane half's two blocks.
template <int FMT, int HT, int KS8, bool MX>
__device__ __forceinline__ void load_query_lowp(const IdxArgs& a, int b, int64_t j, bool qvalid, int lane,
                                                i32x8 (&qa)[HT][KS8], float (&wv)[HT][16], uint32_t (&qsx)[HT]) {
  constexpr int DI = 64 * KS8 * LowP<FMT>::BITS / 8;  // bytes per row
  constexpr int OB = LowP<FMT>::OB;
  const uint8_t* qp = (const uint8_t*)a.qI + ((int64_t)b * a.Tq + j) * a.HI * DI;
  const float* wp = a.wI + ((int64_t)b * a.Tq + j) * a.HI;
  const float* sp = a.q_scale + ((int64_t)b * a.Tq + j) * a.HI;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = ht * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks)
      qa[ht][ks] = (qvalid && h < a.HI) ? load_op_at<FMT, KS8, MX>(qp + (int64_t)h * DI, lane >> 5, ks) : i32x8{};
    qsx[ht] = MX && qvalid && h < a.HI ? mx_scale_word<FMT>(__float_as_uint(sp[h]), lane >> 5) : 0x7f7f7f7fu;
    // accumulator rows held by this lane: 8*(i/4) + 4*(lane/32) + i%4
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = ht * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      wv[ht][i] = (qvalid && hh < a.HI) ? (MX ? wp[hh] : wp[hh] * sp[hh]) : 0.f;
    }
  }
}

// Prefill rows: 8 queries per workgroup (one per wave) sharing 256-key LDS tiles, copied
// straight from global memory into LDS (global_load_lds, no staging registers) as in the bf16
// kernel: unpadded rows, chunk c of row r at position c ^ ((r >> SH) % CPR), so the 32 rows of a
// 32-lane B read (one 16-byte chunk each) hit 32 distinct 4-bank groups. The key scales travel
// the same way (4 bytes per lane). Each 32-key sub-block reads the next one's B operands first,
// then issues its MFMAs beside the previous sub-block's ReLU / weighted head-sum.
template <int FMT, int HT, int KS8, bool MX>
__global__ __launch_bounds__(512) void indexer_score_lowp_mfma(IdxArgs a) {
  constexpr int QB = 8;                // queries per workgroup (one per wave)
  constexpr int SUB = 8;               // 32-key sub-blocks per tile (even)
  constexpr int TILE = SUB * 32;
  constexpr int DI = 64 * KS8 * LowP<FMT>::BITS / 8;  // bytes per key row
  constexpr int OB = LowP<FMT>::OB;    // operand bytes per lane per k-step
  constexpr int CPO = OB / 16;         // 16-byte chunks per operand
  constexpr int CPR = DI / 16;         // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;        // key rows per direct-to-LDS copy (64 lanes x 16 bytes)
  constexpr int IPW = 32 / RPI;        // copies per wave per tile (each wave copies 32 rows)
  constexpr int SH = CPR == 16 ? 1 : CPR == 8 ? 2 : CPR == 4 ? 3 : 4;  // log2(32 / CPR)
  static_assert(TILE == 32 * QB && CPR >= 2 && CPR <= 16 && IPW >= 1, "tile shape");
  static_assert(!MX || KS8 == 2, "MX: dI = 128 (4 scale bytes per row)");
  // two arrays per buffer kind (not [2][...]): the compiler then sees that a copy into one
  // never feeds reads of the other. Scales: wave w copies keys 32 w + (lane % 32) to 64 w + lane.
  __shared__ __attribute__((aligned(16))) uint8_t kt0[TILE * DI], kt1[TILE * DI];
  __shared__ float ks0[2 * TILE], ks1[2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int qs = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.z;
  const int64_t qblk = (int64_t)gridDim.y - 1 - blockIdx.y;  // longest rows first
  const int64_t jr = qblk * QB + qs;
  const bool qvalid = jr < a.nrows;
  const int64_t j = a.row0 + (qvalid ? jr : 0);
  int64_t jl = qblk * QB + QB - 1;
  if (jl > a.nrows - 1) jl = a.nrows - 1;
  const int64_t vmax = visible_entries(a.pos0 + a.row0 + jl, a.m, a.N);
  const int64_t kbeg = (int64_t)blockIdx.x * a.span;
  int64_t kend = kbeg + a.span;
  if (kend > vmax) kend = vmax;
  if (kbeg >= kend) return;  // uniform for the workgroup
  const int64_t vj = qvalid ? visible_entries(a.pos0 + j, a.m, a.N) : 0;
  const int nkeys = (int)(kend - kbeg);
  // visible keys of this query within this workgroup's span
  const int vrel = (int)((vj < kbeg ? kbeg : (vj > kend ? kend : vj)) - kbeg);

  i32x8 qa[HT][KS8];
  float wv[HT][16];
  uint32_t qsx[HT];
  load_query_lowp<FMT, HT, KS8, MX>(a, b, j, qvalid, lane, qa, wv, qsx);

  const uint8_t* kbase = (const uint8_t*)a.KI + ((int64_t)b * a.N + kbeg) * DI;
  const float* kscale = a.k_scale + (int64_t)b * a.N + kbeg;  // MX: 4 scale bytes per key
  float* rowp = a.scores + ((int64_t)b * a.rows_ws + (qvalid ? jr : 0)) * a.ldS + kbeg;
  const int ntiles = (nkeys + TILE - 1) / TILE;

  // direct-to-LDS copy of tile t0: wave w copies rows 32 w .. 32 w + 31 (lane l of a copy lands
  // 16 l bytes past its base: row l / CPR, position l % CPR) and their scales. Rows past the span
  // fetch row 0 (their scores are dropped).
  auto dma = [&](int t0, uint8_t* buf, float* sbuf) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int rr = 32 * qs + i * RPI + lane / CPR;
      const int c = (lane % CPR) ^ ((rr >> SH) % CPR);
      const int s = t0 + rr < nkeys ? t0 + rr : 0;
      __builtin_amdgcn_global_load_lds((const void*)(kbase + (int64_t)s * DI + c * 16),
                                       (__attribute__((address_space(3))) void*)(buf + (32 * qs + i * RPI) * DI), 16,
                                       0, 0);
    }
    const int ss = t0 + 32 * qs + (lane & 31);
    __builtin_amdgcn_global_load_lds((const void*)(kscale + (ss < nkeys ? ss : 0)),
                                     (__attribute__((address_space(3))) void*)(sbuf + 64 * qs), 4, 0, 0);
  };
  // B operand of k-step ks for the lane's key row (lane half h holds bytes h DI/2 + OB ks .. + OB):
  // its CPO chunks at their swizzled positions; bofs holds their byte offsets within a sub-block
  int bofs[KS8][CPO];
#pragma unroll
  for (int ks = 0; ks < KS8; ++ks)
#pragma unroll
    for (int q = 0; q < CPO; ++q)
      bofs[ks][q] = (lane & 31) * DI + (((op_off<FMT, KS8, MX>(lane >> 5, ks, q) / 16) ^ (((lane & 31) >> SH) % CPR)) * 16);
  auto rdB = [&](const uint8_t* kp, i32x8 (&dst)[KS8]) {
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(kp + bofs[ks][0]);
      if constexpr (CPO == 2) {
        const u32x4 hi = *reinterpret_cast<const u32x4*>(kp + bofs[ks][CPO - 1]);
        dst[ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      } else {
        dst[ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
      }
    }
  };
  auto mma = [&](const i32x8 (&bv)[KS8], f32x16 (&acc)[HT], uint32_t kx) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      if constexpr (MX) {
        acc[ht] = mfma_mx<FMT, 0>(qa[ht][0], bv[0], f32x16{}, qsx[ht], kx);
        acc[ht] = mfma_mx<FMT, 1>(qa[ht][1], bv[1], acc[ht], qsx[ht], kx);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS8; ++ks) acc[ht] = mfma_lowp<FMT>(qa[ht][ks], bv[ks], ks == 0 ? f32x16{} : acc[ht]);
      }
    }
  };
  // ReLU, folded head weights, head sum, the other lane half (the other 16 heads of each 32-head
  // tile), the key scale; lanes 0-31 store key lane%32 through a buffer descriptor that covers this
  // sub-block's keys of this row, so the hardware drops stores past the span (and of a padding
  // query) without branches
  auto finish = [&](const f32x16 (&acc)[HT], int s0, float sc) {
    float part = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 0; i < 16; ++i) part = __builtin_fmaf(relu_bits(acc[ht][i]), wv[ht][i], part);
    {  // lanes 0-31 receive lanes 32-63
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
      part += __uint_as_float(sw[1]);
    }
    const int left = nkeys - s0;
    const int nrec = (qvalid && left > 0) ? 4 * (left < 32 ? left : 32) : 0;  // 0: all dropped
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(rowp + s0, (short)0, nrec, 0x00020000);
    const float v = s0 + (lane & 31) < vrel ? (MX ? part : part * sc) : -INFINITY;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, lane < 32 ? 4 * lane : 256, 0, 0);
  };
  auto wait_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0);  // every counter at zero: the compiler's wait tracking sees it
    __syncthreads();
  };
  f32x16 acc[2][HT];
  i32x8 bv[2][KS8];
  float sc[2];     // scales of the keys of the current and previous sub-block
  uint32_t kx[2];  // MX: scale bytes of the current and next sub-block's keys, shifted to the lane half
  auto rdX = [&](const float* sb_, int sb) { return mx_scale_word<FMT>(__float_as_uint(sb_[64 * sb + lane]), lane >> 5); };
  auto tile = [&](int it, const uint8_t* kb, const float* sb_) {
    const int t0 = it * TILE;
    rdB(kb, bv[0]);
    if constexpr (MX) kx[0] = rdX(sb_, 0);
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      const bool prev = sb > 0 || it > 0;
      if (sb + 1 < SUB) {
        rdB(kb + (sb + 1) * 32 * DI, bv[(sb + 1) & 1]);
        if constexpr (MX) kx[(sb + 1) & 1] = rdX(sb_, sb + 1);
      }
      if constexpr (!MX) sc[sb & 1] = sb_[64 * sb + lane];  // lanes 32-63 read the same scales as lanes 0-31
      __builtin_amdgcn_sched_barrier(0);
      mma(bv[sb & 1], acc[sb & 1], kx[sb & 1]);
      if (prev) finish(acc[(sb + 1) & 1], t0 + sb * 32 - 32, sc[(sb + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  dma(0, kt0, ks0);
  wait_barrier();
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    dma((it + 1) * TILE, kt1, ks1);
    tile(it, kt0, ks0);
    wait_barrier();
    dma((it + 2 < ntiles ? it + 2 : it) * TILE, kt0, ks0);  // unconditional (a join would cost a full wait)
    tile(it + 1, kt1, ks1);
    wait_barrier();
  }
  if (it < ntiles) tile(it, kt0, ks0);
  finish(acc[(SUB - 1) & 1], ntiles * TILE - 32, sc[(SUB - 1) & 1]);  // last sub-block of the last tile
}

// Decode-shaped rows: row_waves waves per query row, wave r taking the 32-key
// blocks r, r + row_waves, ...; each block loaded with coalesced 16-byte loads
// one block ahead and turned into the MFMA layout through the wave's own LDS rows.
template <int FMT, int HT, int KS8, bool MX>
__global__ __launch_bounds__(256) void indexer_score_lowp_stream(IdxArgs a) {
  constexpr int DI = 64 * KS8 * LowP<FMT>::BITS / 8;  // bytes per key row
  constexpr int OB = LowP<FMT>::OB;
  constexpr int RS = DI + 16;       // padded LDS row
  constexpr int NB = 2;             // key blocks in registers: the current one + 1 in flight
  constexpr int LPB = 32 * DI / 1024;  // 1 KiB loads per 32-key block
  __shared__ __attribute__((aligned(16))) uint8_t kst[4][32 * RS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, kl = lane & 31;
  const int b = blockIdx.z;
  const int64_t jr = blockIdx.y;
  const int64_t j = a.row0 + jr;
  const int64_t vj = visible_entries(a.pos0 + j, a.m, a.N);
  const int64_t wr = (int64_t)blockIdx.x * 4 + wave;  // this wave's rank in the row
  const int64_t row_blk = (vj + 31) / 32;
  if (wr >= row_blk) return;  // per wave: the kernel has no workgroup barrier
  const int nblk = (int)((row_blk - wr + a.row_waves - 1) / a.row_waves);

  i32x8 qa[HT][KS8];
  float wv[HT][16];
  uint32_t qsx[HT];
  load_query_lowp<FMT, HT, KS8, MX>(a, b, j, true, lane, qa, wv, qsx);

  uint8_t* my = kst[wave];
  const uint8_t* kb0 = (const uint8_t*)a.KI + (int64_t)b * a.N * DI;
  const float* ksp = a.k_scale + (int64_t)b * a.N;
  float* srow = a.scores + ((int64_t)b * a.rows_ws + jr) * a.ldS;
  auto key_of = [&](int blk) { return (wr + (int64_t)blk * a.row_waves) * 32 + kl; };
  u32x4 kb[NB][LPB];
  float kss[NB];
  auto load = [&](int blk, u32x4 (&dst)[LPB], float& sc) {
    if (blk >= nblk) return;
    const int64_t key0 = (wr + (int64_t)blk * a.row_waves) * 32;
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      const int off = i * 1024 + lane * 16;
      int64_t r = key0 + off / DI;
      if (r > vj - 1) r = vj - 1;  // past the visible keys: a valid row, its score is not stored
      dst[i] = *reinterpret_cast<const u32x4*>(kb0 + r * DI + (off % DI));
    }
    int64_t s = key0 + kl;
    if (s > vj - 1) s = vj - 1;
    sc = ksp[s];
  };
  auto step = [&](int blk, const u32x4 (&src)[LPB], float sc) {
    if (blk >= nblk) return;
    // wave-scope fences: the previous block's LDS reads precede these writes, which
    // precede the reads below (other lanes' rows)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      const int off = i * 1024 + lane * 16;
      *reinterpret_cast<u32x4*>(my + (off / DI) * RS + (off % DI)) = src[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    f32x16 acc[HT];
    if constexpr (MX) {
      const uint32_t kx = mx_scale_word<FMT>(__float_as_uint(sc), half);  // the key's 4 scale bytes
      const i32x8 b0 = load_op_at<FMT, KS8, MX>(my + kl * RS, half, 0);
      const i32x8 b1 = load_op_at<FMT, KS8, MX>(my + kl * RS, half, 1);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        acc[ht] = mfma_mx<FMT, 0>(qa[ht][0], b0, f32x16{}, qsx[ht], kx);
        acc[ht] = mfma_mx<FMT, 1>(qa[ht][1], b1, acc[ht], qsx[ht], kx);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) {
        const i32x8 bv = load_op<FMT>(my + kl * RS + (DI / 2) * half + OB * ks);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma_lowp<FMT>(qa[ht][ks], bv, ks == 0 ? f32x16{} : acc[ht]);
      }
    }
    float part = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 0; i < 16; ++i) part = __builtin_fmaf(relu_bits(acc[ht][i]), wv[ht][i], part);
    part += __shfl_xor(part, 32, 64);
    const int64_t s = key_of(blk);
    const float sval = MX ? part : part * sc;
    if (lane < 32 && s < vj) srow[s] = sval;
    if (a.bm_fused) {  // the block's maximum key, for the selection (as the bf16 decode scorer)
      const uint32_t mk = max_key32(s < vj ? score_key(sval) : 0u);
      if (lane == 0) a.bm[((int64_t)b * a.bm_rows + jr) * a.bm_ld + (s >> 5)] = mk;
    }
  };

#pragma unroll
  for (int p = 0; p < NB; ++p) load(p, kb[p], kss[p]);
  for (int it = 0; it < nblk; it += NB) {
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      step(it + p, kb[p], kss[p]);
      load(it + p + NB, kb[p], kss[p]);
    }
  }
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
static constexpr int64_t LOWP_STREAM_WAVES = 4096;  // decode scoring: waves over the whole call

template <int FMT, int HT, int KS8, bool STREAM, bool MX>
static void launch_lowp(const IdxArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (STREAM)
    hipLaunchKernelGGL((indexer_score_lowp_stream<FMT, HT, KS8, MX>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((indexer_score_lowp_mfma<FMT, HT, KS8, MX>), grid, dim3(512), 0, st, a);
}

template <int FMT, bool STREAM, bool MX = false>
static bool dispatch_lowp(int ht, int ks8, const IdxArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (!MX) {
    if (ks8 == 1) {
      switch (ht) {
        case 1: launch_lowp<FMT, 1, 1, STREAM, false>(a, grid, st); return true;
        case 2: launch_lowp<FMT, 2, 1, STREAM, false>(a, grid, st); return true;
        case 4: launch_lowp<FMT, 4, 1, STREAM, false>(a, grid, st); return true;
      }
    }
  }
  if (ks8 == 2) {
    switch (ht) {
      case 1: launch_lowp<FMT, 1, 2, STREAM, MX>(a, grid, st); return true;
      case 2: launch_lowp<FMT, 2, 2, STREAM, MX>(a, grid, st); return true;
      case 4: launch_lowp<FMT, 4, 2, STREAM, MX>(a, grid, st); return true;
    }
  }
  return false;
}

int launch_scores_lowp(IdxArgs& a, int batch, int qb, int dtype, hipStream_t st) {
  const int64_t last = a.pos0 + a.row0 + a.nrows - 1;
  int64_t vmax = (last + 1) / a.m;
  if (vmax > a.N) vmax = a.N;
  if (vmax <= 0) return CSKV_OK;
  const int ht = a.HI <= 32 ? 1 : (a.HI <= 64 ? 2 : 4);
  const int ks8 = a.dI / 64;
  dim3 grid;
  if (qb == 8) {
    const int64_t qblocks = ceil_div(a.nrows, (int64_t)8);
    int64_t splits = ceil_div(1024, qblocks * batch);
    if (splits < 1) splits = 1;
    a.span = round_up(ceil_div(vmax, splits), (int64_t)128);
    splits = ceil_div(vmax, a.span);
    grid = dim3((unsigned)splits, (unsigned)qblocks, (unsigned)batch);
  } else {
    const int64_t rows = a.nrows * batch;
    int64_t per_row = ceil_div(LOWP_STREAM_WAVES, rows);
    const int64_t cap = ceil_div(vmax, (int64_t)128);
    if (per_row > cap) per_row = cap;
    a.row_waves = round_up(per_row, (int64_t)4);
    grid = dim3((unsigned)(a.row_waves / 4), (unsigned)a.nrows, (unsigned)batch);
  }
  bool ok;
  if (dtype == CSKV_MXFP4)
    ok = qb == 8 ? dispatch_lowp<FMT_E2M1, false, true>(ht, ks8, a, grid, st)
                 : dispatch_lowp<FMT_E2M1, true, true>(ht, ks8, a, grid, st);
  else if (dtype == CSKV_MXFP8)
    ok = qb == 8 ? dispatch_lowp<FMT_E4M3, false, true>(ht, ks8, a, grid, st)
                 : dispatch_lowp<FMT_E4M3, true, true>(ht, ks8, a, grid, st);
  else if (dtype == CSKV_FP4)
    ok = qb == 8 ? dispatch_lowp<FMT_E2M1, false>(ht, ks8, a, grid, st) : dispatch_lowp<FMT_E2M1, true>(ht, ks8, a, grid, st);
  else
    ok = qb == 8 ? dispatch_lowp<FMT_E4M3, false>(ht, ks8, a, grid, st) : dispatch_lowp<FMT_E4M3, true>(ht, ks8, a, grid, st);
  if (!ok) return CSKV_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

static int check_lowp_shape(int batch, int64_t Tq, int64_t N, int HI, int dI, int64_t pos0, int m, int dtype) {
  if (batch < 0 || Tq < 0 || N < 0 || pos0 < 0 || m < 1) return CSKV_ERR_BAD_SHAPE;
  if (HI < 1 || HI > CSKV_MAX_HEADS) return CSKV_ERR_BAD_SHAPE;
  if (N > ((int64_t)1 << 31) - 64) return CSKV_ERR_BAD_SHAPE;
  if (dI != 64 && dI != 128) return CSKV_ERR_UNSUPPORTED;
  if ((dtype == CSKV_MXFP4 || dtype == CSKV_MXFP8) && dI != 128) return CSKV_ERR_UNSUPPORTED;  // 4 scale bytes per row
  return CSKV_OK;
}

static int quantize_rows(int fmt, const void* x, int64_t rows, int dim, int dtype, uint8_t* codes, float* scales,
                         void* stream) {
  if (dtype != CSKV_BF16 && dtype != CSKV_F32) return CSKV_ERR_BAD_DTYPE;
  if (rows < 0 || dim < 4 || dim % 4 != 0 || dim > 1024) return CSKV_ERR_BAD_SHAPE;
  if (ceil_div(rows, (int64_t)4) > 0x7fffffff) return CSKV_ERR_BAD_SHAPE;
  if (rows == 0) return CSKV_OK;
  if (!x || !codes || !scales) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(x, codes, scales)) return CSKV_ERR_MISALIGNED;
  dim3 grid((unsigned)ceil_div(rows, (int64_t)4));
  hipStream_t st = (hipStream_t)stream;
  if (fmt == FMT_E2M1) {
    if (dtype == CSKV_BF16)
      hipLaunchKernelGGL(quantize_fp4_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)x, rows, dim, codes, scales);
    else
      hipLaunchKernelGGL(quantize_fp4_kernel<float>, grid, dim3(256), 0, st, (const float*)x, rows, dim, codes,
                         scales);
  } else {
    if (dtype == CSKV_BF16)
      hipLaunchKernelGGL(quantize_fp8_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)x, rows, dim, codes, scales);
    else
      hipLaunchKernelGGL(quantize_fp8_kernel<float>, grid, dim3(256), 0, st, (const float*)x, rows, dim, codes,
                         scales);
  }
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

static int quantize_rows_mx(int fmt, const void* x, int64_t rows, int dim, int dtype, uint8_t* codes,
                            uint8_t* scales, void* stream) {
  if (dtype != CSKV_BF16 && dtype != CSKV_F32) return CSKV_ERR_BAD_DTYPE;
  if (rows < 0 || dim < 32 || dim % 32 != 0 || dim > 1024) return CSKV_ERR_BAD_SHAPE;
  if (ceil_div(rows, (int64_t)4) > 0x7fffffff) return CSKV_ERR_BAD_SHAPE;
  if (rows == 0) return CSKV_OK;
  if (!x || !codes || !scales) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(x, codes, scales)) return CSKV_ERR_MISALIGNED;
  dim3 grid((unsigned)ceil_div(rows, (int64_t)4));
  hipStream_t st = (hipStream_t)stream;
  if (fmt == FMT_E2M1) {
    if (dtype == CSKV_BF16)
      hipLaunchKernelGGL((quantize_mx_kernel<bf16, FMT_E2M1>), grid, dim3(256), 0, st, (const bf16*)x, rows, dim, codes,
                         scales);
    else
      hipLaunchKernelGGL((quantize_mx_kernel<float, FMT_E2M1>), grid, dim3(256), 0, st, (const float*)x, rows, dim,
                         codes, scales);
  } else {
    if (dtype == CSKV_BF16)
      hipLaunchKernelGGL((quantize_mx_kernel<bf16, FMT_E4M3>), grid, dim3(256), 0, st, (const bf16*)x, rows, dim, codes,
                         scales);
    else
      hipLaunchKernelGGL((quantize_mx_kernel<float, FMT_E4M3>), grid, dim3(256), 0, st, (const float*)x, rows, dim,
                         codes, scales);
  }
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

static int scores_lowp(int dtype, const uint8_t* qI, const float* q_scale, const float* wI, const uint8_t* KI,
                       const float* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI, int64_t pos0, int m,
                       float* scores, int64_t ld, void* stream) {
  int st = check_lowp_shape(batch, Tq, N, HI, dI, pos0, m, dtype);
  if (st) return st;
  if (ld < N || ld % 4 != 0) return CSKV_ERR_BAD_SHAPE;
  if (batch == 0 || Tq == 0) return CSKV_OK;
  if (!qI || !q_scale || !wI || !scores || (N > 0 && (!KI || !k_scale))) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(qI, q_scale, wI, KI, k_scale, scores)) return CSKV_ERR_MISALIGNED;
  IdxArgs a{};
  a.qI = qI; a.q_scale = q_scale; a.wI = wI; a.KI = KI; a.k_scale = k_scale; a.scores = scores;
  a.Tq = Tq; a.N = N; a.pos0 = pos0; a.ldS = ld; a.rows_ws = Tq; a.row0 = 0; a.nrows = Tq;
  a.HI = HI; a.dI = dI; a.m = m;
  const IdxPlan p = plan_indexer(batch, Tq, N, dtype);
  return launch_scores_lowp(a, batch, (int)p.qb, dtype, (hipStream_t)stream);
}

static int topk_lowp(int dtype, const uint8_t* qI, const float* q_scale, const float* wI, const uint8_t* KI,
                     const float* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI, int64_t pos0, int m,
                     int k, int32_t* out_idx, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_lowp_shape(batch, Tq, N, HI, dI, pos0, m, dtype);
  if (st) return st;
  if (k < 1) return CSKV_ERR_BAD_SHAPE;
  if (k > CSKV_MAX_TOPK) return CSKV_ERR_UNSUPPORTED;
  if (batch == 0 || Tq == 0) return CSKV_OK;
  if (!qI || !q_scale || !wI || !out_idx || (N > 0 && (!KI || !k_scale))) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(qI, q_scale, wI, KI, k_scale, out_idx, workspace)) return CSKV_ERR_MISALIGNED;
  const IdxPlan p = plan_indexer(batch, Tq, N, dtype);
  const size_t score_bytes = (size_t)(batch * p.rows_ws * p.ldS * 4);
  const size_t need_ws = score_bytes + split_ws_bytes((int64_t)batch * p.rows_ws, N, k);
  if (!workspace || ws_bytes < need_ws) return CSKV_ERR_WORKSPACE;
  // the selection area follows the score rows (score_bytes is a multiple of 256: ldS % 64 == 0)
  uint8_t* sel_ws = need_ws > score_bytes ? (uint8_t*)workspace + score_bytes : nullptr;
  const size_t sel_bytes = sel_ws ? ws_bytes - score_bytes : 0;

  hipStream_t hs = (hipStream_t)stream;
  IdxArgs a{};
  a.qI = qI; a.q_scale = q_scale; a.wI = wI; a.KI = KI; a.k_scale = k_scale;
  a.scores = (float*)workspace; a.out = out_idx;
  a.Tq = Tq; a.N = N; a.pos0 = pos0; a.ldS = p.ldS; a.rows_ws = p.rows_ws;
  a.HI = HI; a.dI = dI; a.m = m; a.k = k;
  for (int64_t r0 = 0; r0 < Tq; r0 += p.rows_ws) {
    a.row0 = r0;
    a.nrows = (Tq - r0) < p.rows_ws ? (Tq - r0) : p.rows_ws;
    const int64_t last = pos0 + r0 + a.nrows - 1;
    int64_t vmax = (last + 1) / m;
    if (vmax > N) vmax = N;
    int64_t vmin = (pos0 + r0 + 1) / m;
    if (vmin > N) vmin = N;
    // few long rows scored one query per workgroup (decode): the scorer writes the block maxima
    // into the rows' selection workspace, and the selection reads them
    a.bm_fused = p.qb == 1 && sel_ws && bm_route(vmin, vmax, k);
    if (a.bm_fused) {
      a.bm = reinterpret_cast<uint32_t*>(sel_ws);
      a.bm_ld = topk_sel_stride() / 4;
      a.bm_rows = a.nrows;
    }
    if (vmax > k) {  // rows with V_t <= k need no scores
      st = launch_scores_lowp(a, batch, (int)p.qb, dtype, hs);
      if (st) return st;
    }
    st = launch_select(a, batch, sel_ws, sel_bytes, hs);
    if (st) return st;
  }
  return CSKV_OK;
}

}  // namespace cskv

using namespace cskv;

extern "C" int cskv_quantize_fp8(const void* x, int64_t rows, int dim, int dtype, uint8_t* codes, float* scales,
                                 void* stream) {
  return quantize_rows(FMT_E4M3, x, rows, dim, dtype, codes, scales, stream);
}

extern "C" int cskv_quantize_fp4(const void* x, int64_t rows, int dim, int dtype, uint8_t* codes, float* scales,
                                 void* stream) {
  return quantize_rows(FMT_E2M1, x, rows, dim, dtype, codes, scales, stream);
}

extern "C" int indexer_scores_fp8(const uint8_t* qI, const float* q_scale, const float* wI, const uint8_t* KI,
                                  const float* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                                  int64_t pos0, int m, float* scores, int64_t ld, void* stream) {
  return scores_lowp(CSKV_FP8, qI, q_scale, wI, KI, k_scale, batch, Tq, N, HI, dI, pos0, m, scores, ld, stream);
}

extern "C" int indexer_scores_fp4(const uint8_t* qI, const float* q_scale, const float* wI, const uint8_t* KI,
                                  const float* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                                  int64_t pos0, int m, float* scores, int64_t ld, void* stream) {
  return scores_lowp(CSKV_FP4, qI, q_scale, wI, KI, k_scale, batch, Tq, N, HI, dI, pos0, m, scores, ld, stream);
}

extern "C" int indexer_topk_fp8(const uint8_t* qI, const float* q_scale, const float* wI, const uint8_t* KI,
                                const float* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                                int64_t pos0, int m, int k, int32_t* out_idx, void* workspace, size_t ws_bytes,
                                void* stream) {
  return topk_lowp(CSKV_FP8, qI, q_scale, wI, KI, k_scale, batch, Tq, N, HI, dI, pos0, m, k, out_idx, workspace,
                   ws_bytes, stream);
}

extern "C" int indexer_topk_fp4(const uint8_t* qI, const float* q_scale, const float* wI, const uint8_t* KI,
                                const float* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                                int64_t pos0, int m, int k, int32_t* out_idx, void* workspace, size_t ws_bytes,
                                void* stream) {
  return topk_lowp(CSKV_FP4, qI, q_scale, wI, KI, k_scale, batch, Tq, N, HI, dI, pos0, m, k, out_idx, workspace,
                   ws_bytes, stream);
}

// MX-FP4: the scale arrays hold 4 E8M0 bytes per row (dI = 128); the kernels read them as one
// 32-bit word per row through the fp32 scale slots of the argument block.
extern "C" int cskv_quantize_mxfp4(const void* x, int64_t rows, int dim, int dtype, uint8_t* codes, uint8_t* scales,
                                   void* stream) {
  return quantize_rows_mx(FMT_E2M1, x, rows, dim, dtype, codes, scales, stream);
}

extern "C" int cskv_quantize_mxfp8(const void* x, int64_t rows, int dim, int dtype, uint8_t* codes, uint8_t* scales,
                                   void* stream) {
  return quantize_rows_mx(FMT_E4M3, x, rows, dim, dtype, codes, scales, stream);
}

extern "C" int indexer_scores_mxfp8(const uint8_t* qI, const uint8_t* q_scale, const float* wI, const uint8_t* KI,
                                    const uint8_t* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                                    int64_t pos0, int m, float* scores, int64_t ld, void* stream) {
  return scores_lowp(CSKV_MXFP8, qI, (const float*)q_scale, wI, KI, (const float*)k_scale, batch, Tq, N, HI, dI,
                     pos0, m, scores, ld, stream);
}

extern "C" int indexer_topk_mxfp8(const uint8_t* qI, const uint8_t* q_scale, const float* wI, const uint8_t* KI,
                                  const uint8_t* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                                  int64_t pos0, int m, int k, int32_t* out_idx, void* workspace, size_t ws_bytes,
                                  void* stream) {
  return topk_lowp(CSKV_MXFP8, qI, (const float*)q_scale, wI, KI, (const float*)k_scale, batch, Tq, N, HI, dI, pos0,
                   m, k, out_idx, workspace, ws_bytes, stream);
}

extern "C" int indexer_scores_mxfp4(const uint8_t* qI, const uint8_t* q_scale, const float* wI, const uint8_t* KI,
                                    const uint8_t* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                                    int64_t pos0, int m, float* scores, int64_t ld, void* stream) {
  return scores_lowp(CSKV_MXFP4, qI, (const float*)q_scale, wI, KI, (const float*)k_scale, batch, Tq, N, HI, dI,
                     pos0, m, scores, ld, stream);
}

extern "C" int indexer_topk_mxfp4(const uint8_t* qI, const uint8_t* q_scale, const float* wI, const uint8_t* KI,
                                  const uint8_t* k_scale, int batch, int64_t Tq, int64_t N, int HI, int dI,
                                  int64_t pos0, int m, int k, int32_t* out_idx, void* workspace, size_t ws_bytes,
                                  void* stream) {
  return topk_lowp(CSKV_MXFP4, qI, (const float*)q_scale, wI, KI, (const float*)k_scale, batch, Tq, N, HI, dI, pos0,
                   m, k, out_idx, workspace, ws_bytes, stream);
}
