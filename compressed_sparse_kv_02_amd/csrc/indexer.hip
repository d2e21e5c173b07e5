// Lightning-indexer scoring for gfx950.
//
// "Paper Breakdown: DeepSeek-V4", §2.3.1 "DSA on Compressed KV (lightning
// indexer + top-k)": every query scores every visible compressed indexer key,
//   I[t, s] = sum_h w[t, h] * ReLU(qI[t, h, :] . KI[s, :]),
// and keeps the k best entries ("How DeepSeek-V4 architecture and training
// work together", "Two compressed views of one history": k = 1024). The
// selection is in topk.hip; this file scores and holds the indexer_topk and
// indexer_scores entry points.
//
// Scoring (bf16): a dense Q.K^T contraction on the matrix cores
// (v_mfma_f32_32x32x16_bf16; M = 32 heads of one query, N = 32 keys,
// K = dI), fused with the ReLU and the weighted head-sum in registers. A
// workgroup of 8 waves holds QB queries (their q rows stay in registers as
// MFMA A operands) and streams a span of keys through double-buffered LDS
// tiles, copied straight from global memory into LDS (global_load_lds, no
// staging registers), so each key row fetched from HBM feeds QB queries. With QB = 1
// (decode) the 8 waves take different key blocks and many workgroups split
// the key range. Scores go to a caller workspace as fp32 rows.
#include "indexer.h"

namespace cskv {

// ----------------------------------------------------------------------------
// bf16 scoring on the matrix cores
// ----------------------------------------------------------------------------

// Prefill rows: 8 queries per workgroup, one per wave, sharing 256-key LDS tiles.
// Each 32-key sub-block runs in two phases of KS/2 k-steps. A phase issues the
// MFMAs of its first k-step, then the LDS reads of the next phase's B operands,
// then its remaining MFMAs, interleaved with half of the previous sub-block's
// ReLU / weighted head-sum; scheduling barriers keep the reads about one phase
// ahead of their use. The compiler waits for every LDS read in flight before a
// phase's first MFMA, so issuing the next reads after that point leaves it
// waiting only for reads made a phase earlier (1% faster than reads first).
template <int HT, int KS>
__global__ __launch_bounds__(512) void indexer_score_mfma(IdxArgs a) {
  constexpr int QB = 8;                // queries per workgroup (one per wave)
  constexpr int SUB = 8;               // 32-key sub-blocks per tile (even)
  constexpr int DI = 16 * KS;
  constexpr int KH = KS / 2;           // k-steps per phase
  constexpr int TILE = SUB * 32;       // keys per LDS tile
  constexpr int CPR = DI / 8;          // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;        // key rows per direct-to-LDS copy (64 lanes x 16 bytes)
  constexpr int IPW = 32 / RPI;        // copies per wave per tile (each wave copies 32 rows)
  constexpr int SH = CPR == 16 ? 1 : CPR == 8 ? 2 : 3;  // log2(32 / CPR)
  static_assert(SUB == 8 && CPR >= 4 && CPR <= 16, "tile shape");
  // Unpadded rows; chunk c of row r sits at position c ^ sw(r), sw(r) = (r >> SH) % CPR, so the
  // 32 rows of a 32-lane B read (one chunk each) hit 32 distinct 4-bank groups. Two arrays
  // (not one [2][...]) let the compiler see that a copy into one never feeds reads of the other.
  __shared__ __attribute__((aligned(16))) uint16_t kt0[TILE * DI], kt1[TILE * DI];

  const int tid = threadIdx.x, lane = tid & 63;
  const int qs = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.z;
  const int64_t qblk = (int64_t)gridDim.y - 1 - blockIdx.y;  // longest rows first
  const int64_t jr = qblk * QB + qs;                        // row within chunk
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
  const int nkeys = (int)(kend - kbeg);         // keys of this workgroup (< 2^31)
  // visible keys of this query within this workgroup's span
  const int vrel = (int)((vj < kbeg ? kbeg : (vj > kend ? kend : vj)) - kbeg);

  // A operands: lane holds head (lane % 32) of each 32-head tile, 8 dims per k-step.
  bf16x8 qa[HT][KS];
  float wv[HT][16];
  {
    const uint16_t* qp = (const uint16_t*)a.qI + ((int64_t)b * a.Tq + j) * a.HI * DI;
    const float* wp = a.wI + ((int64_t)b * a.Tq + j) * a.HI;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (qvalid && h < a.HI) v = *reinterpret_cast<const u32x4*>(qp + (int64_t)h * DI + ks * 16 + 8 * (lane >> 5));
        qa[ht][ks] = __builtin_bit_cast(bf16x8, v);
      }
      // accumulator rows held by this lane: 8*(i/4) + 4*(lane/32) + i%4
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hh = ht * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        wv[ht][i] = (qvalid && hh < a.HI) ? wp[hh] : 0.f;
      }
    }
  }

  const uint16_t* kbase = (const uint16_t*)a.KI + ((int64_t)b * a.N + kbeg) * DI;
  float* rowp = a.scores + ((int64_t)b * a.rows_ws + (qvalid ? jr : 0)) * a.ldS + kbeg;
  const int ntiles = (nkeys + TILE - 1) / TILE;

  // direct-to-LDS copy of tile t0 into buf: wave w copies rows 32 w .. 32 w + 31; lane l of a
  // copy lands at 16 l bytes past the copy's base, i.e. row l / CPR, position l % CPR, and
  // fetches the chunk stored there. Rows past the span fetch row 0 (their scores are dropped).
  auto dma = [&](int t0, uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int rr = 32 * qs + i * RPI + lane / CPR;
      const int c = (lane % CPR) ^ ((rr >> SH) % CPR);
      const int s = t0 + rr < nkeys ? t0 + rr : 0;
      __builtin_amdgcn_global_load_lds((const void*)(kbase + (int64_t)s * DI + c * 8),
                                       (__attribute__((address_space(3))) void*)(buf + (32 * qs + i * RPI) * DI), 16, 0,
                                       0);
    }
  };
  // B operand of k-step ks for the lane's key row: chunk 2 ks + (lane / 32) at its swizzled
  // position; bofs holds the lane's element offset of each k-step within a sub-block
  int bofs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) bofs[ks] = (lane & 31) * DI + (((2 * ks + (lane >> 5)) ^ (((lane & 31) >> SH) % CPR)) * 8);
  auto rdB = [&](const uint16_t* kp, int h, bf16x8 (&dst)[KH]) {
#pragma unroll
    for (int i = 0; i < KH; ++i) dst[i] = *reinterpret_cast<const bf16x8*>(kp + bofs[h * KH + i]);
  };
  auto mmaH = [&](const bf16x8 (&bv)[KH], int h, f32x16 (&acc)[HT], int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int ks = h * KH + i;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        acc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ht][ks], bv[i], ks == 0 ? f32x16{} : acc[ht], 0, 0, 0);
    }
  };
  // ReLU and head weights over accumulator entries [8h, 8h + 8) of every head tile
  auto epiH = [&](const f32x16 (&acc)[HT], int h, float part) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 8 * h; i < 8 * h + 8; ++i) part = __builtin_fmaf(relu_bits(acc[ht][i]), wv[ht][i], part);
    return part;
  };
  // sum of the two lane halves (the other 16 heads of each 32-head tile); lanes 0-31 store key
  // lane%32 through a buffer descriptor that covers this sub-block's keys of this row, so that the
  // hardware drops the stores of keys past the span (and of a padding query) without branches
  auto finish = [&](float part, int s0) {
    {  // lanes 0-31 receive lanes 32-63
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
      part += __uint_as_float(sw[1]);
    }
    const int left = nkeys - s0;
    const int nrec = (qvalid && left > 0) ? 4 * (left < 32 ? left : 32) : 0;  // 0: all dropped
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(rowp + s0, (short)0, nrec, 0x00020000);
    const float v = s0 + (lane & 31) < vrel ? part : -INFINITY;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, lane < 32 ? 4 * lane : 256, 0, 0);
  };

  // wait for this wave's copies, then a workgroup barrier (every copy of the tile has landed and
  // every wave is done with the other buffer)
  auto wait_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0);  // every counter at zero: the compiler's wait tracking sees it
    __syncthreads();
  };
  f32x16 acc[2][HT];
  bf16x8 b0[KH], b1[KH];
  auto tile = [&](int it, const uint16_t* kb) {
    const int t0 = it * TILE;
    const uint16_t* kp = kb;
    rdB(kp, 0, b0);
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      // the previous sub-block (of this tile, or the last of the previous tile) is epilogued here
      const bool prev = sb > 0 || it > 0;
      const int sp = t0 + sb * 32 - 32;
      // phase 0: its first k-step, then the reads of phase 1's operands, then the rest
      mmaH(b0, 0, acc[sb & 1], 0, 1);
      __builtin_amdgcn_sched_barrier(0);
      rdB(kp + sb * 32 * DI, 1, b1);
      __builtin_amdgcn_sched_barrier(0);
      mmaH(b0, 0, acc[sb & 1], 1, KH);
      float part = 0.f;
      if (prev) part = epiH(acc[(sb + 1) & 1], 0, 0.f);
      __builtin_amdgcn_sched_barrier(0);
      // phase 1
      mmaH(b1, 1, acc[sb & 1], 0, 1);
      __builtin_amdgcn_sched_barrier(0);
      if (sb + 1 < SUB) rdB(kp + (sb + 1) * 32 * DI, 0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mmaH(b1, 1, acc[sb & 1], 1, KH);
      if (prev) finish(epiH(acc[(sb + 1) & 1], 1, part), sp);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  dma(0, kt0);
  wait_barrier();
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    dma((it + 1) * TILE, kt1);
    tile(it, kt0);
    wait_barrier();
    dma((it + 2 < ntiles ? it + 2 : it) * TILE, kt0);  // unconditional (a join would cost a full wait)
    tile(it + 1, kt1);
    wait_barrier();
  }
  if (it < ntiles) tile(it, kt0);
  // last sub-block of the last tile
  finish(epiH(acc[(SUB - 1) & 1], 1, epiH(acc[(SUB - 1) & 1], 0, 0.f)), ntiles * TILE - 32);
}

// Decode-shaped rows (fewer than 64 queries in the call): row_waves waves score
// one query, wave r taking the 32-key blocks r, r + row_waves, r + 2 row_waves,
// ..., so the waves of a row read one contiguous, advancing window of keys
// (every HBM channel busy) rather than each streaming its own distant span. A
// key serves one query only, so waves share nothing: each loads its block with
// fully coalesced 16-byte loads (1 KiB per instruction) NB blocks ahead into
// registers, and turns it into the MFMA B layout through its own padded LDS
// rows (no workgroup barrier; a wave's LDS operations run in order). The K
// dimension is permuted the same way in A and B (lane half h, k-step ks: dims
// h*8*KS + 8*ks .. +8), so each lane reads one contiguous half row from LDS;
// every dot product is unchanged.
template <int HT, int KS>
__global__ __launch_bounds__(256) void indexer_score_stream(IdxArgs a) {
  constexpr int DI = 16 * KS;
  constexpr int NB = 2;  // key blocks in registers: the current one + 1 in flight
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, kl = lane & 31;
  const int b = blockIdx.z;
  const int64_t jr = blockIdx.y;
  const int64_t j = a.row0 + jr;
  const int64_t vj = visible_entries(a.pos0 + j, a.m, a.N);
  const int64_t wr = (int64_t)blockIdx.x * 4 + wave;  // this wave's rank in the row
  const int64_t row_blk = (vj + 31) / 32;
  if (wr >= row_blk) return;  // per wave: the kernel has no workgroup barrier
  const int nblk = (int)((row_blk - wr + a.row_waves - 1) / a.row_waves);  // blocks of this wave

  bf16x8 qa[HT][KS];
  float wv[HT][16];
  {
    const uint16_t* qp = (const uint16_t*)a.qI + ((int64_t)b * a.Tq + j) * a.HI * DI + half * 8 * KS;
    const float* wp = a.wI + ((int64_t)b * a.Tq + j) * a.HI;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 32 + kl;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (h < a.HI) v = *reinterpret_cast<const u32x4*>(qp + (int64_t)h * DI + 8 * ks);
        qa[ht][ks] = __builtin_bit_cast(bf16x8, v);
      }
      // accumulator rows held by this lane: 8*(i/4) + 4*(lane/32) + i%4
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hh = ht * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        wv[ht][i] = hh < a.HI ? wp[hh] : 0.f;
      }
    }
  }

  const uint16_t* kbase = (const uint16_t*)a.KI + (int64_t)b * a.N * DI + half * 8 * KS;
  float* srow = a.scores + ((int64_t)b * a.rows_ws + jr) * a.ldS;
  auto key_of = [&](int blk) { return (wr + (int64_t)blk * a.row_waves) * 32 + kl; };
  constexpr int RB = 32 * KS;  // bytes per key row
  constexpr int RS = RB + 16;  // padded LDS row
  __shared__ __attribute__((aligned(16))) uint8_t kst[4][32 * RS];
  uint8_t* my = kst[wave];
  const uint8_t* kb0 = (const uint8_t*)a.KI + (int64_t)b * a.N * RB;
  u32x4 kb[NB][KS];
  auto load = [&](int blk, u32x4 (&dst)[KS]) {
    if (blk >= nblk) return;
    const int64_t key0 = (wr + (int64_t)blk * a.row_waves) * 32;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int off = i * 1024 + lane * 16;
      int64_t r = key0 + off / RB;
      if (r > vj - 1) r = vj - 1;
      dst[i] = *reinterpret_cast<const u32x4*>(kb0 + r * RB + (off % RB));
    }
  };
  auto step = [&](int blk, const u32x4 (&src)[KS]) {
    if (blk >= nblk) return;
    // wave-scope fences: the previous block's LDS reads precede these writes, which
    // precede the reads below (other lanes' rows)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int off = i * 1024 + lane * 16;
      *reinterpret_cast<u32x4*>(my + (off / RB) * RS + (off % RB)) = src[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    u32x4 bop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bop[ks] = *reinterpret_cast<const u32x4*>(my + kl * RS + (half * KS + ks) * 16);
    f32x16 acc[HT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 bv = __builtin_bit_cast(bf16x8, bop[ks]);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        acc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ht][ks], bv, ks == 0 ? f32x16{} : acc[ht], 0, 0, 0);
    }
    float part = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 0; i < 16; ++i) part = __builtin_fmaf(relu_bits(acc[ht][i]), wv[ht][i], part);
    part += __shfl_xor(part, 32, 64);
    const int64_t s = key_of(blk);
    if (lane < 32 && s < vj) srow[s] = part;
    if (a.bm_fused) {  // the block's maximum key, for the selection
      const uint32_t mk = max_key32(s < vj ? score_key(part) : 0u);
      if (lane == 0) a.bm[((int64_t)b * a.bm_rows + jr) * a.bm_ld + (s >> 5)] = mk;
    }
  };

#pragma unroll
  for (int p = 0; p < NB; ++p) load(p, kb[p]);
  for (int it = 0; it < nblk; it += NB) {
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      step(it + p, kb[p]);
      load(it + p + NB, kb[p]);
    }
  }
}

// ----------------------------------------------------------------------------
// fp32 scoring on the vector ALUs (fp32 mode: small shapes, correctness)
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void indexer_score_f32(IdxArgs a) {
  extern __shared__ float qsh[];  // [HI * dI + HI]
  const int b = blockIdx.z;
  const int64_t jr = blockIdx.y;
  const int64_t j = a.row0 + jr;
  const float* qp = (const float*)a.qI + ((int64_t)b * a.Tq + j) * a.HI * a.dI;
  const float* wp = a.wI + ((int64_t)b * a.Tq + j) * a.HI;
  for (int i = threadIdx.x; i < a.HI * a.dI; i += blockDim.x) qsh[i] = qp[i];
  for (int i = threadIdx.x; i < a.HI; i += blockDim.x) qsh[a.HI * a.dI + i] = wp[i];
  __syncthreads();
  const int64_t vj = visible_entries(a.pos0 + j, a.m, a.N);
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= vj) return;
  const float* kp = (const float*)a.KI + ((int64_t)b * a.N + s) * a.dI;
  float tot = 0.f;
  for (int h = 0; h < a.HI; ++h) {
    float dot = 0.f;
    for (int c = 0; c < a.dI; ++c) dot = fmaf(qsh[h * a.dI + c], kp[c], dot);
    tot += qsh[a.HI * a.dI + h] * fmaxf(dot, 0.f);
  }
  a.scores[((int64_t)b * a.rows_ws + jr) * a.ldS + s] = tot;
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
static constexpr int64_t SCORE_CHUNK_BYTES = (int64_t)128 << 20;
static constexpr int64_t STREAM_WAVES = 4096;  // decode scoring: waves over the whole call

IdxPlan plan_indexer(int batch, int64_t Tq, int64_t N, int dtype) {
  IdxPlan p;
  p.ldS = round_up(N > 0 ? N : 1, 64);
  p.qb = (dtype != CSKV_F32 && Tq >= 64) ? 8 : 1;
  int64_t rows = SCORE_CHUNK_BYTES / (p.ldS * 4 * (batch > 0 ? batch : 1));
  // enough rows per chunk to fill the GPU with selection workgroups
  if (rows < 2048 / (batch > 0 ? batch : 1)) rows = 2048 / (batch > 0 ? batch : 1);
  if (rows < p.qb) rows = p.qb;
  rows = (rows / p.qb) * p.qb;
  if (rows > 32768) rows = 32768;
  if (rows > Tq) rows = Tq;
  p.rows_ws = rows > 0 ? rows : 1;
  return p;
}

// STREAM = false: indexer_score_mfma (512 threads), true: indexer_score_stream (256 threads).
template <int HT, int KS, bool STREAM>
static void launch_mfma(const IdxArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (STREAM)
    hipLaunchKernelGGL((indexer_score_stream<HT, KS>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((indexer_score_mfma<HT, KS>), grid, dim3(512), 0, st, a);
}

template <int HT, bool STREAM>
static bool dispatch_ks(int ks, const IdxArgs& a, dim3 grid, hipStream_t st) {
  switch (ks) {
    case 2: launch_mfma<HT, 2, STREAM>(a, grid, st); return true;
    case 4: launch_mfma<HT, 4, STREAM>(a, grid, st); return true;
    case 8: launch_mfma<HT, 8, STREAM>(a, grid, st); return true;
    default: return false;
  }
}

template <bool STREAM>
static bool dispatch_mfma(int ht, int ks, const IdxArgs& a, dim3 grid, hipStream_t st) {
  switch (ht) {
    case 1: return dispatch_ks<1, STREAM>(ks, a, grid, st);
    case 2: return dispatch_ks<2, STREAM>(ks, a, grid, st);
    case 4: return dispatch_ks<4, STREAM>(ks, a, grid, st);
    default: return false;
  }
}

static bool mfma_shape_ok(int HI, int dI) {
  const int ht = HI <= 32 ? 1 : (HI <= 64 ? 2 : 4);
  const int ks = dI / 16;
  if (dI % 16 != 0) return false;
  (void)ht;
  return ks == 2 || ks == 4 || ks == 8;
}


// Launch the scoring kernel for rows [a.row0, a.row0 + a.nrows) into a.scores.
int launch_scores(IdxArgs& a, int batch, int qb, int dtype, hipStream_t st) {
  const int64_t last = a.pos0 + a.row0 + a.nrows - 1;
  int64_t vmax = (last + 1) / a.m;
  if (vmax > a.N) vmax = a.N;
  if (vmax <= 0) return CSKV_OK;
  if (dtype == CSKV_BF16) {
    const int ht = a.HI <= 32 ? 1 : (a.HI <= 64 ? 2 : 4);
    bool ok;
    if (qb == 8) {
      // key spans (multiples of 128 keys) so that about 1024 workgroups run
      const int64_t qblocks = ceil_div(a.nrows, (int64_t)8);
      int64_t splits = ceil_div(1024, qblocks * batch);
      if (splits < 1) splits = 1;
      a.span = round_up(ceil_div(vmax, splits), (int64_t)128);
      splits = ceil_div(vmax, a.span);
      dim3 grid((unsigned)splits, (unsigned)qblocks, (unsigned)batch);
      ok = dispatch_mfma<false>(ht, a.dI / 16, a, grid, st);
    } else {
      // about STREAM_WAVES waves in all, at least 4 blocks of 32 keys per wave
      const int64_t rows = a.nrows * batch;
      int64_t per_row = ceil_div(STREAM_WAVES, rows);
      const int64_t cap = ceil_div(vmax, (int64_t)128);
      if (per_row > cap) per_row = cap;
      a.row_waves = round_up(per_row, (int64_t)4);
      dim3 grid((unsigned)(a.row_waves / 4), (unsigned)a.nrows, (unsigned)batch);
      ok = dispatch_mfma<true>(ht, a.dI / 16, a, grid, st);
    }
    if (!ok) return CSKV_ERR_UNSUPPORTED;
  } else {
    dim3 grid((unsigned)ceil_div(vmax, 256), (unsigned)a.nrows, (unsigned)batch);
    const size_t shm = ((size_t)a.HI * a.dI + a.HI) * 4;
    hipLaunchKernelGGL(indexer_score_f32, grid, dim3(256), shm, st, a);
  }
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

static int check_indexer_shape(int batch, int64_t Tq, int64_t N, int HI, int dI, int64_t pos0, int m, int dtype) {
  if (dtype != CSKV_BF16 && dtype != CSKV_F32) return CSKV_ERR_BAD_DTYPE;
  if (batch < 0 || Tq < 0 || N < 0 || pos0 < 0 || m < 1) return CSKV_ERR_BAD_SHAPE;
  if (HI < 1 || HI > CSKV_MAX_HEADS || dI < 16 || dI % 16 != 0) return CSKV_ERR_BAD_SHAPE;
  if (N > ((int64_t)1 << 31) - 64) return CSKV_ERR_BAD_SHAPE;
  if (dtype == CSKV_BF16 && !mfma_shape_ok(HI, dI)) return CSKV_ERR_UNSUPPORTED;
  if (dtype == CSKV_F32 && ((int64_t)HI * dI + HI) * 4 > 48 * 1024) return CSKV_ERR_UNSUPPORTED;
  return CSKV_OK;
}

}  // namespace cskv

using namespace cskv;

extern "C" size_t cskv_indexer_workspace_size(int batch, int64_t Tq, int64_t N, int HI, int k,
                                              int dtype) {
  (void)HI;
  if (batch <= 0 || Tq <= 0) return 0;
  IdxPlan p = plan_indexer(batch, Tq, N, dtype);
  return (size_t)(batch * p.rows_ws * p.ldS * 4) + split_ws_bytes((int64_t)batch * p.rows_ws, N, k);
}

extern "C" int indexer_topk(const void* qI, const float* wI, const void* KI, int batch, int64_t Tq,
                            int64_t N, int HI, int dI, int64_t pos0, int m, int k,
                            int32_t* out_idx, void* workspace, size_t ws_bytes, int dtype,
                            void* stream) {
  int st = check_indexer_shape(batch, Tq, N, HI, dI, pos0, m, dtype);
  if (st) return st;
  if (k < 1) return CSKV_ERR_BAD_SHAPE;
  if (k > CSKV_MAX_TOPK) return CSKV_ERR_UNSUPPORTED;
  if (batch == 0 || Tq == 0) return CSKV_OK;
  if (!qI || !wI || !out_idx || (N > 0 && !KI)) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(qI, wI, KI, out_idx, workspace)) return CSKV_ERR_MISALIGNED;
  IdxPlan p = plan_indexer(batch, Tq, N, dtype);
  const size_t score_bytes = (size_t)(batch * p.rows_ws * p.ldS * 4);
  const size_t split_bytes = split_ws_bytes((int64_t)batch * p.rows_ws, N, k);
  const size_t need_ws = score_bytes + split_bytes;
  if (!workspace || ws_bytes < need_ws) return CSKV_ERR_WORKSPACE;
  // the selection area follows the score rows (score_bytes is a multiple of 256: ldS % 64 == 0)
  uint8_t* sel_ws = split_bytes ? (uint8_t*)workspace + score_bytes : nullptr;
  const size_t sel_bytes = split_bytes;

  hipStream_t hs = (hipStream_t)stream;
  IdxArgs a{};
  a.qI = qI; a.wI = wI; a.KI = KI; a.scores = (float*)workspace; a.out = out_idx;
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
    // into the rows' selection workspace
    a.bm_fused = dtype == CSKV_BF16 && p.qb == 1 && split_bytes && bm_route(vmin, vmax, k);
    if (a.bm_fused) {
      a.bm = reinterpret_cast<uint32_t*>(sel_ws);
      a.bm_ld = topk_sel_stride() / 4;
      a.bm_rows = a.nrows;
    }
    if (vmax > k) {  // rows with V_t <= k need no scores
      st = launch_scores(a, batch, (int)p.qb, dtype, hs);
      if (st) return st;
    }
    st = launch_select(a, batch, sel_ws, sel_bytes, hs);
    if (st) return st;
  }
  return CSKV_OK;
}

extern "C" int indexer_scores(const void* qI, const float* wI, const void* KI, int batch, int64_t Tq,
                              int64_t N, int HI, int dI, int64_t pos0, int m, float* scores,
                              int64_t ld, uint32_t* block_max, int64_t bm_ld, int dtype, void* stream) {
  int st = check_indexer_shape(batch, Tq, N, HI, dI, pos0, m, dtype);
  if (st) return st;
  if (ld < N || ld % 4 != 0) return CSKV_ERR_BAD_SHAPE;
  if (block_max && dtype != CSKV_BF16) return CSKV_ERR_UNSUPPORTED;
  if (block_max && (bm_ld < ceil_div(N, (int64_t)32) || bm_ld % 4 != 0)) return CSKV_ERR_BAD_SHAPE;
  if (batch == 0 || Tq == 0) return CSKV_OK;
  if (!qI || !wI || !scores || (N > 0 && !KI)) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(qI, wI, KI, scores, block_max)) return CSKV_ERR_MISALIGNED;
  IdxArgs a{};
  a.qI = qI; a.wI = wI; a.KI = KI; a.scores = scores;
  a.Tq = Tq; a.N = N; a.pos0 = pos0; a.ldS = ld; a.rows_ws = Tq; a.row0 = 0; a.nrows = Tq;
  a.HI = HI; a.dI = dI; a.m = m;
  const int qb = (dtype == CSKV_BF16 && Tq >= 64) ? 8 : 1;
  if (block_max && qb == 1) {  // the one-query-per-workgroup scorer writes the block maxima
    a.bm = block_max;
    a.bm_ld = bm_ld;
    a.bm_rows = Tq;
    a.bm_fused = 1;
  }
  return launch_scores(a, batch, qb, dtype, (hipStream_t)stream);
}
