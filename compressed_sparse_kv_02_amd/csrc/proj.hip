// Projections around the core attention, gfx950.
//
// "Paper Breakdown: DeepSeek-V4", section 4, CSA §2.3.1: the indexer queries
// are low-rank, projected from a latent c_t^Q shared with the attention
// queries; the core attention is followed by a grouped output projection
// (HCA §2.3.2: the same MQA + grouped projection). The pages give no shapes:
//  * cskv_lowrank_proj: out[t] = c^Q_t W (one call per projection, for the
//    attention queries [H * d] and the indexer queries [H_I * d_I]);
//  * cskv_grouped_out_proj: the H heads form G contiguous groups; group g's
//    concatenated outputs are projected by its own W_g [(H/G) d, d_g] into
//    mid[t, g] (stored bf16), then y[t] = concat_g mid[t, g] @ W_o.
//
// Both are bf16 products with fp32 accumulation on one batched GEMM kernel:
//  * 512 threads, a 256 x 256 output tile per workgroup (one per CU: each
//    byte brought into LDS feeds 128 flops), 4 x 2 waves of 64 x 128 (2 x 4
//    tiles of v_mfma_f32_32x32x16_bf16, accumulators in the accumulation
//    registers);
//  * the matrix cores compute C^T = B^T A^T, so that each lane ends with 4
//    consecutive columns of a row of C per group and stores them as one 8-byte
//    write (C = A B directly would leave one column per lane);
//  * K advances 64 at a time through double-buffered LDS tiles staged in
//    registers (the next tile's loads are in flight during this tile's math);
//  * A (row-major, M x K) rows are padded to 72 elements: the 32 rows of an
//    operand read start 36 banks apart, distinct groups of 4 among 128 banks;
//  * B (row-major, K x N) is kept as stored; its operand (8 k-values of one
//    column per lane) comes from two gfx950 transpose reads
//    (ds_read_b64_tr_b16), with rows padded to 144 elements so that the four
//    rows of one read start 72 banks apart (no conflicts);
//  * the finished tile is staged through LDS (8-byte writes, conflict-free
//    with 264-element rows) so that the global stores are whole 512-byte rows;
//  * workgroups are numbered so that each XCD takes a contiguous run of output
//    tiles, which mostly share their A rows in that XCD's L2.
#include "device_common.h"
#include "abi_common.h"

namespace cskv {

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* C;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;  // batch strides (elements)
  int tiles_m, tiles_n, batch;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i16 lds_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
}

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int GWM = 4, GWN = 2;              // waves along M and N
constexpr int GNT = GWM * GWN * 64;          // threads
constexpr int TI = GBM / GWM / 32, TJ = GBN / GWN / 32;  // 32 x 32 tiles per wave
constexpr int AROW = GBK + 8;    // padded A row in LDS (elements)
constexpr int BROW = GBN + 16;   // padded B row in LDS (elements)
constexpr int CROW = GBN + 8;    // padded row of the staged C tile (elements)
constexpr int A_ELEMS = GBM * AROW, B_ELEMS = GBK * BROW;
constexpr int SMEM = 2 * (A_ELEMS + B_ELEMS) > GBM * CROW ? 2 * (A_ELEMS + B_ELEMS) : GBM * CROW;

__global__ __launch_bounds__(GNT) void gemm_bf16(GemmArgs g) {
  // two stages of (A tile, B tile); after the last stage the same memory stages the C tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];
  auto As = [&](int buf) { return smem + buf * (A_ELEMS + B_ELEMS); };
  auto Bs = [&](int buf) { return smem + buf * (A_ELEMS + B_ELEMS) + A_ELEMS; };

  // workgroup -> (batch, tile): each XCD (flat id mod 8) gets a contiguous run of tiles
  const int64_t nwg = (int64_t)gridDim.x;
  const int64_t flat = blockIdx.x;
  const int64_t per = nwg / 8;
  const int64_t L = (nwg % 8 == 0) ? (flat % 8) * per + flat / 8 : flat;
  const int64_t per_batch = (int64_t)g.tiles_m * g.tiles_n;
  const int64_t bz = L / per_batch;
  const int64_t tl = L % per_batch;
  const int64_t m0 = (tl / g.tiles_n) * GBM, n0 = (tl % g.tiles_n) * GBN;
  const uint16_t* A = g.A + bz * g.sA;
  const uint16_t* B = g.B + bz * g.sB;
  uint16_t* C = g.C + bz * g.sC;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / GWN, wn = wave % GWN;  // this wave's (GBM/GWM) x (GBN/GWN) block

  // loader: A chunks (row, 8-element column group) and B chunks (k row, 8-column group)
  constexpr int ACH = GBM * GBK / 8 / GNT, BCH = GBK * GBN / 8 / GNT;  // 16-byte chunks per thread
  constexpr int ACR = GBK / 8, BCR = GBN / 8;                          // chunks per row
  u32x4 pa[ACH], pb[BCH];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + GNT * i;
      const int r = c / ACR, kc = c % ACR;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m0 + r < g.M) v = *reinterpret_cast<const u32x4*>(A + (m0 + r) * g.lda + k0 + 8 * kc);
      pa[i] = v;
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + GNT * i;
      const int kr = c / BCR, nc = c % BCR;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (n0 + 8 * nc < g.N) v = *reinterpret_cast<const u32x4*>(B + (k0 + kr) * g.ldb + n0 + 8 * nc);
      pb[i] = v;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + GNT * i;
      *reinterpret_cast<u32x4*>(As(buf) + (c / ACR) * AROW + 8 * (c % ACR)) = pa[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + GNT * i;
      *reinterpret_cast<u32x4*>(Bs(buf) + (c / BCR) * BROW + 8 * (c % BCR)) = pb[i];
    }
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

  // operand addresses: A^T lane (row of A l%32, k 8(l/32)..+7); B^T transpose reads of lane
  // group G: k rows 8(G/2) + e (+4 for the second read), columns 16(G%2) + 4(l%4)
  const int a_off = (wm * (GBM / GWM) + (lane & 31)) * AROW + 8 * (lane >> 5);
  const int G = lane >> 4, e = (lane & 15) >> 2;
  const int b_off = (8 * (G >> 1) + e) * BROW + wn * (GBN / GWN) + 16 * (G & 1) + 4 * (lane & 3);

  const int64_t nk = g.K / GBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nk) gload((kt + 1) * GBK);
    const uint16_t* as = As(buf);
    const uint16_t* bs = Bs(buf);
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8 av[TI], bv[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) av[i] = *reinterpret_cast<const bf16x8*>(as + a_off + i * 32 * AROW + 16 * ks);
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const uint16_t* p = bs + b_off + 16 * ks * BROW + 32 * j;
        const v4i16 h[2] = {lds_tr16(p), lds_tr16(p + 4 * BROW)};
        bv[j] = __builtin_bit_cast(bf16x8, h);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[j], av[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue, staged through LDS so that the global stores are whole rows: tile (i, j) of
  // C^T gives lane row l%32 of tile i and columns 8c + 4(l/32) .. +3 of tile j (c = 0..3)
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    uint16_t* crow = smem + (wm * (GBM / GWM) + i * 32 + (lane & 31)) * CROW + wn * (GBN / GWN) + 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint2 v;
        v.x = pack_bf16x2(acc[i][j][4 * c], acc[i][j][4 * c + 1]);
        v.y = pack_bf16x2(acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]);
        *reinterpret_cast<uint2*>(crow + j * 32 + 8 * c) = v;
      }
  }
  __syncthreads();
  constexpr int CCH = GBM * GBN / 8 / GNT;  // 16-byte chunks per thread
#pragma unroll
  for (int k = 0; k < CCH; ++k) {
    const int q = tid + GNT * k;
    const int r = q / (GBN / 8), cc = q % (GBN / 8);
    const int64_t row = m0 + r, col = n0 + 8 * cc;
    if (row < g.M && col < g.N)
      *reinterpret_cast<u32x4*>(C + row * g.ldc + col) = *reinterpret_cast<const u32x4*>(smem + r * CROW + 8 * cc);
  }
}

// C[b] = A[b] B[b] for b < batch; sizes validated by the callers.
static int launch_gemm(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int64_t lda,
                       int64_t ldb, int64_t ldc, int batch, int64_t sA, int64_t sB, int64_t sC,
                       hipStream_t st) {
  if (M == 0 || N == 0 || batch == 0) return CSKV_OK;
  GemmArgs g;
  g.A = (const uint16_t*)A;
  g.B = (const uint16_t*)B;
  g.C = (uint16_t*)C;
  g.M = M; g.N = N; g.K = K;
  g.lda = lda; g.ldb = ldb; g.ldc = ldc;
  g.sA = sA; g.sB = sB; g.sC = sC;
  g.tiles_m = (int)ceil_div(M, GBM);
  g.tiles_n = (int)ceil_div(N, GBN);
  g.batch = batch;
  const int64_t nwg = (int64_t)g.tiles_m * g.tiles_n * batch;
  if (nwg > 0x7fffffff) return CSKV_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(gemm_bf16, dim3((unsigned)nwg), dim3(GNT), 0, st, g);
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

}  // namespace cskv

using namespace cskv;

extern "C" int cskv_lowrank_proj(const void* cq, const void* W, void* out, int64_t T, int64_t r, int64_t n_out,
                                 int dtype, void* stream) {
  if (dtype != CSKV_BF16) return CSKV_ERR_BAD_DTYPE;
  if (T < 0 || r < GBK || r % GBK != 0 || n_out < 8 || n_out % 8 != 0) return CSKV_ERR_BAD_SHAPE;
  if (T > ((int64_t)1 << 31) || n_out > ((int64_t)1 << 31) || r > ((int64_t)1 << 20)) return CSKV_ERR_BAD_SHAPE;
  if (T == 0) return CSKV_OK;
  if (!cq || !W || !out) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(cq, W, out)) return CSKV_ERR_MISALIGNED;
  return launch_gemm(cq, W, out, T, n_out, r, r, n_out, n_out, 1, 0, 0, 0, (hipStream_t)stream);
}

extern "C" int cskv_grouped_out_proj(const void* o, const void* Wg, const void* Wo, void* mid, void* y, int64_t T,
                                     int H, int d, int G, int64_t dg, int64_t D, int dtype, void* stream) {
  if (dtype != CSKV_BF16) return CSKV_ERR_BAD_DTYPE;
  if (T < 0 || H < 1 || d < 1 || G < 1 || H % G != 0 || dg < 8 || D < 8) return CSKV_ERR_BAD_SHAPE;
  const int64_t kin = (int64_t)(H / G) * d;  // inputs per group
  if (kin % GBK != 0 || dg % 8 != 0 || (G * dg) % GBK != 0 || D % 8 != 0) return CSKV_ERR_BAD_SHAPE;
  if (T > ((int64_t)1 << 31) || (int64_t)H * d > ((int64_t)1 << 24) || G * dg > ((int64_t)1 << 24) ||
      D > ((int64_t)1 << 24))
    return CSKV_ERR_BAD_SHAPE;
  if (T == 0) return CSKV_OK;
  if (!o || !Wg || !Wo || !mid || !y) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(o, Wg, Wo, mid, y)) return CSKV_ERR_MISALIGNED;
  hipStream_t st = (hipStream_t)stream;
  // mid[:, g] = o[:, group g] @ Wg[g]: batch over groups, A rows strided by H*d
  int rc = launch_gemm(o, Wg, mid, T, dg, kin, (int64_t)H * d, dg, G * dg, G, kin, kin * dg, dg, st);
  if (rc != CSKV_OK) return rc;
  return launch_gemm(mid, Wo, y, T, D, G * dg, G * dg, D, D, 1, 0, 0, 0, st);
}
