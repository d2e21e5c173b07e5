// Per-query exact top-k selection for gfx950.
//
// "Paper Breakdown: DeepSeek-V4", §2.3.1 "DSA on Compressed KV (lightning
// indexer + top-k)": each query keeps the k compressed entries of largest
// indexer score ("How DeepSeek-V4 architecture and training work together",
// "Two compressed views of one history": k = 1024). The pages leave ties and
// order open; here the smaller index wins among equal scores and the list is
// ascending, -1 padded when fewer than k entries are visible.
//
// Scores are compared through an order-preserving uint32 key, so the
// selection is integer work and deterministic.
//
// Many rows (prefill): one 512-thread workgroup per row (three fit a compute
// unit). A sample of the row (64 runs of 32 consecutive entries) gives a
// threshold that about 3k entries exceed; one vectorised pass, each wave over
// its own contiguous share of the row, keeps those entries (in index order)
// in LDS, an exact 3-pass radix
// select (11 + 11 + 10 bits) finds the k-th largest among them, and an
// in-order pick with block prefix sums writes the result without a sort.
// Should the sample miss, the row falls back to the exact radix select over
// global memory.
//
// Few long rows (decode): the row is cut into parts selected by separate
// workgroups, then merged (topk_part / topk_merge below).
#include "indexer.h"

namespace cskv {

// ----------------------------------------------------------------------------
// Exact top-k per row
// ----------------------------------------------------------------------------
constexpr int TOPK_THREADS = 512;
constexpr int TOPK_CAP = 5632;      // candidate (key, index) pairs held in LDS: 53 KiB per workgroup, three per CU
constexpr int TOPK_SAMPLES = 2048;     // sample of a long row, for the candidate threshold
constexpr int TOPK_SAMPLE_RUNS = 64;   // ... taken as runs of 32 consecutive entries

// Exclusive prefix sum over the workgroup; also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TOPK_THREADS / 64; ++w) {
    const int x = wsum[w];
    if (w < wave) pre += x;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return pre + incl - v;
}

// Exclusive prefix count of a flag over the workgroup (ballots and popcounts: no shuffle chain);
// also returns the total.
__device__ __forceinline__ int block_exclusive_count(bool f, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(f);
  const int before = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(m);
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TOPK_THREADS / 64; ++w) {
    const int x = wsum[w];
    if (w < wave) pre += x;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return pre + before;
}

// Four consecutive entries per lane, in lane order: how many flagged entries precede this lane's
// first one in the wave, and how many the wave holds (four ballots, no shuffle chain).
__device__ __forceinline__ void wave_count4(const bool (&fl)[4], int& before, int& tot) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  before = 0;
  tot = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint64_t m = __ballot(fl[e]);
    before += __popcll(m & below);
    tot += __popcll(m);
  }
}

struct TopkShared {
  int hist[2048];
  int wsum[TOPK_THREADS / 64];
  int wcnt[TOPK_THREADS / 64];  // candidates found by each wave
  int sel_bin, sel_above, count;
};

// Radix select (11 + 11 + 10 bits): the kk-th largest of n keys read through key_at.
// Returns it in tau; `need` = how many keys equal to tau belong to the top kk.
template <typename KeyAt>
__device__ void radix_select(KeyAt key_at, int64_t n, int kk, TopkShared& sh, uint32_t& tau, int& need) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  need = kk;
  const int shifts[3] = {21, 10, 0};
  const int nbits[3] = {11, 11, 10};
  for (int p = 0; p < 3; ++p) {
    const int nb = 1 << nbits[p];
    const uint32_t bmask = (uint32_t)nb - 1u;
    for (int i = tid; i < 2048; i += TOPK_THREADS) sh.hist[i] = 0;
    __syncthreads();
    for (int64_t s = tid; s < n; s += TOPK_THREADS) {
      const uint32_t key = key_at(s);
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shifts[p]) & bmask], 1);
    }
    __syncthreads();
    const int bpt = nb / TOPK_THREADS;  // bins per thread, descending
    int cnt[2048 / TOPK_THREADS] = {}, loc = 0;
    for (int q = 0; q < bpt; ++q) {
      cnt[q] = sh.hist[nb - 1 - (tid * bpt + q)];
      loc += cnt[q];
    }
    int total;
    int above = block_exclusive_scan(loc, sh.wsum, total);
    for (int q = 0; q < bpt; ++q) {
      if (above < need && need <= above + cnt[q]) {
        sh.sel_bin = nb - 1 - (tid * bpt + q);
        sh.sel_above = above;
      }
      above += cnt[q];
    }
    __syncthreads();
    need -= sh.sel_above;
    prefix |= (uint32_t)sh.sel_bin << shifts[p];
    pmask |= bmask << shifts[p];
    __syncthreads();
  }
  tau = prefix;
}

// Emits, in index order, the entries with key > tau plus the first `need` with key == tau:
// emit(position among the emitted, s).
template <typename KeyAt, typename Emit>
__device__ void ordered_pick(KeyAt key_at, Emit emit, int64_t n, uint32_t tau, int need, TopkShared& sh) {
  const int tid = threadIdx.x;
  int eq_taken = 0, written = 0;
  for (int64_t base = 0; base < n; base += TOPK_THREADS) {
    const int64_t s = base + tid;
    uint32_t key = 0;
    if (s < n) key = key_at(s);
    const bool gt = s < n && key > tau;
    const bool eq = s < n && key == tau;
    int eq_tot;
    const int eq_rank = block_exclusive_count(eq, sh.wsum, eq_tot);
    const bool sel = gt || (eq && (eq_taken + eq_rank) < need);
    int sel_tot;
    const int pos = block_exclusive_count(sel, sh.wsum, sel_tot);
    if (sel) emit(written + pos, s);
    eq_taken += eq_tot;
    written += sel_tot;
  }
}

// Exact top-k of one row straight from global memory (3 radix passes + in-order pick).
__device__ void select_row_global(const float* row, int64_t V, int k, int32_t* out, TopkShared& sh) {
  uint32_t tau;
  int need;
  auto key_at = [&](int64_t s) { return score_key(row[s]); };
  radix_select(key_at, V, k, sh, tau, need);
  ordered_pick(key_at, [&](int pos, int64_t s) { out[pos] = (int32_t)s; }, V, tau, need, sh);
}

// One workgroup per query row.
//  * V <= CAP: the whole row becomes the candidate set.
//  * otherwise: the (3k * S / V)-th largest of S sampled entries gives a
//    threshold tau0; one vectorised pass over the row keeps every entry with
//    key >= tau0, in index order, as candidates (about 3k of them).
//  * exact radix select among the candidates, then an in-order pick.
// If the candidates do not hold at least k entries (or overflow LDS), the
// row falls back to the exact 3-pass radix select over global memory. Both
// routes return the same, exact set.
__global__ __launch_bounds__(TOPK_THREADS) void topk_select(IdxArgs a) {
  __shared__ uint32_t ckey[TOPK_CAP];
  __shared__ int32_t cidx[TOPK_CAP];
  __shared__ TopkShared sh;
  uint32_t* samp = reinterpret_cast<uint32_t*>(cidx);  // the sample is done before candidates exist
  static_assert(TOPK_SAMPLES <= TOPK_CAP, "sample buffer aliases the candidate indices");

  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int64_t jr = blockIdx.x;
  const int64_t j = a.row0 + jr;
  const int k = a.k;
  int32_t* out = a.out + ((int64_t)b * a.Tq + j) * k;
  const int64_t V = visible_entries(a.pos0 + j, a.m, a.N);
  if (V <= k) {
    for (int i = tid; i < k; i += TOPK_THREADS) out[i] = i < V ? i : -1;
    return;
  }
  const float* row = a.scores + ((int64_t)b * a.rows_ws + jr) * a.ldS;
  int n_cand = 0;
  if (V <= TOPK_CAP) {
    for (int64_t s = tid; s < V; s += TOPK_THREADS) {
      ckey[s] = score_key(row[s]);
      cidx[s] = (int32_t)s;
    }
    n_cand = (int)V;
    __syncthreads();
  } else {
    // threshold from a sample: TOPK_SAMPLE_RUNS runs of consecutive entries spread evenly
    // over the row (whole cache lines, 16-byte loads)
    constexpr int RUN = TOPK_SAMPLES / TOPK_SAMPLE_RUNS;
    static_assert(RUN % 4 == 0 && TOPK_SAMPLES % (4 * TOPK_THREADS) == 0, "sample runs are read as float4");
    for (int i = 4 * tid; i < TOPK_SAMPLES; i += 4 * TOPK_THREADS) {
      const int run = i / RUN;
      const int64_t start = ((int64_t)run * (V - RUN) / (TOPK_SAMPLE_RUNS - 1)) & ~(int64_t)3;
      const float4 v = *reinterpret_cast<const float4*>(row + start + (i - run * RUN));
      samp[i] = score_key(v.x);
      samp[i + 1] = score_key(v.y);
      samp[i + 2] = score_key(v.z);
      samp[i + 3] = score_key(v.w);
    }
    __syncthreads();
    int r = (int)(((int64_t)3 * k * TOPK_SAMPLES + V - 1) / V);
    if (r > TOPK_SAMPLES) r = TOPK_SAMPLES;
    uint32_t tau0;
    int need0;
    radix_select([&](int64_t s) { return samp[s]; }, TOPK_SAMPLES, r, sh, tau0, need0);
    __syncthreads();  // the sample (aliasing cidx) is consumed
    // one pass: keep key >= tau0 in index order. Wave w scans its own contiguous
    // eighth of the row (4 consecutive entries per lane per 256-entry chunk, UNR
    // chunks loaded before any is scanned) and appends to its own LDS segment of SEG
    // slots with a wave-level prefix sum: no workgroup barrier inside the pass.
    constexpr int NWAVE = TOPK_THREADS / 64;
    constexpr int SEG = TOPK_CAP / NWAVE;
    constexpr int UNR = 6;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t len = ((V + NWAVE - 1) / NWAVE + 3) & ~(int64_t)3;  // a multiple of 4
    const int64_t lo = wave * len;
    const int64_t hi = lo + len < V ? lo + len : V;
    uint32_t* wkey = ckey + wave * SEG;
    int32_t* widx = cidx + wave * SEG;
    int cnt = 0;
    for (int64_t base = lo; base < hi; base += UNR * 256) {
      float4 v[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int64_t s0 = base + u * 256 + 4 * lane;
        v[u] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (s0 < hi) v[u] = *reinterpret_cast<const float4*>(row + s0);  // rows are padded to 64 entries
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int64_t s0 = base + u * 256 + 4 * lane;
        const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        uint32_t kk4[4];
        bool fl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kk4[e] = score_key(vv[e]);
          fl[e] = s0 + e < hi && kk4[e] >= tau0;
        }
        int before, tot;
        wave_count4(fl, before, tot);
        int pos = cnt + before;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (fl[e]) {
            if (pos < SEG) {
              wkey[pos] = kk4[e];
              widx[pos] = (int32_t)(s0 + e);
            }
            ++pos;
          }
        }
        cnt += tot;
      }
    }
    if (lane == 0) sh.wcnt[wave] = cnt;
    __syncthreads();
    // segments -> one contiguous list in index order (gather to registers, then scatter)
    int cw[NWAVE], off[NWAVE], total = 0;
    bool overflow = false;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      cw[w] = sh.wcnt[w];
      off[w] = total;
      total += cw[w];
      overflow |= cw[w] > SEG;
    }
    n_cand = overflow ? TOPK_CAP + 1 : total;  // an overflowing segment sends the row to the fallback
    if (n_cand >= k && n_cand <= TOPK_CAP) {
      constexpr int SPT = TOPK_CAP / TOPK_THREADS;
      uint32_t kr[SPT];
      int32_t ir[SPT];
      int dst[SPT];
#pragma unroll
      for (int q = 0; q < SPT; ++q) {
        const int slot = q * TOPK_THREADS + tid;
        const int w = slot / SEG, e = slot - w * SEG;
        dst[q] = -1;
#pragma unroll
        for (int ww = 0; ww < NWAVE; ++ww)  // static indexing of cw/off
          if (ww == w && e < cw[ww]) dst[q] = off[ww] + e;
        if (dst[q] >= 0) {
          kr[q] = ckey[slot];
          ir[q] = cidx[slot];
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < SPT; ++q)
        if (dst[q] >= 0) {
          ckey[dst[q]] = kr[q];
          cidx[dst[q]] = ir[q];
        }
      __syncthreads();
    }
  }
  if (n_cand >= k && n_cand <= TOPK_CAP) {
    uint32_t tau;
    int need;
    radix_select([&](int64_t s) { return ckey[s]; }, n_cand, k, sh, tau, need);
    ordered_pick([&](int64_t s) { return ckey[s]; }, [&](int pos, int64_t s) { out[pos] = cidx[s]; }, n_cand,
                 tau, need, sh);
  } else {
    select_row_global(row, V, k, out, sh);
  }
}

// Few long rows (decode): one workgroup per row would leave most of the GPU idle,
// so each row is cut into parts of part_len entries.
//  * topk_part (one workgroup per part): the part's kp best entries (exact, by
//    key then smaller index), in index order, go to the row's candidate list at
//    slot p * kp, with a record {count, kp-th key, truncated}.
//  * topk_merge (one workgroup per row): the exact top-k of the concatenated
//    candidates (index order is kept, parts being consecutive ranges). An entry
//    a truncated part dropped has a key <= that part's kp-th key; if every such
//    key is below the candidates' k-th key, at least k kept entries beat every
//    dropped one, so the candidates hold the row's exact top-k. Otherwise the
//    row falls back to the exact select over global memory.
constexpr int TOPK_MAX_PARTS = 128;
// Part length and candidate capacity of the two-kernel route (few workgroups, so their LDS
// size does not limit occupancy; larger than TOPK_CAP so that k up to 2048 still splits).
constexpr int TOPK_SPLIT_CAP = 8192;
constexpr int64_t TOPK_SEL_STRIDE = (int64_t)TOPK_SPLIT_CAP * 8 + TOPK_MAX_PARTS * 16;

__global__ __launch_bounds__(TOPK_THREADS) void topk_part(IdxArgs a) {
  __shared__ uint32_t ckey[TOPK_SPLIT_CAP];
  __shared__ TopkShared sh;
  const int tid = threadIdx.x;
  const int p = blockIdx.x;
  const int64_t jr = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t V = visible_entries(a.pos0 + a.row0 + jr, a.m, a.N);
  if (V <= a.k) return;
  uint8_t* ws = a.sel_ws + ((int64_t)b * a.nrows + jr) * TOPK_SEL_STRIDE;
  uint32_t* wkey = reinterpret_cast<uint32_t*>(ws) + (int64_t)p * a.kp;
  int32_t* widx = reinterpret_cast<int32_t*>(ws + (int64_t)TOPK_SPLIT_CAP * 4) + (int64_t)p * a.kp;
  int4* rec = reinterpret_cast<int4*>(ws + (int64_t)TOPK_SPLIT_CAP * 8) + p;
  const int64_t s0 = (int64_t)p * a.part_len;
  const int n = (int)(V - s0 < a.part_len ? (V - s0 > 0 ? V - s0 : 0) : a.part_len);
  if (n == 0) {
    if (tid == 0) *rec = make_int4(0, 0, 0, 0);
    return;
  }
  const float* row = a.scores + ((int64_t)b * a.rows_ws + jr) * a.ldS + s0;
  for (int i = 4 * tid; i < n; i += 4 * TOPK_THREADS) {  // s0 % 4 == 0; rows are padded to 64 entries
    const float4 v = *reinterpret_cast<const float4*>(row + i);
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i + e < n) ckey[i + e] = score_key(vv[e]);
  }
  __syncthreads();
  if (n <= a.kp) {
    for (int i = tid; i < n; i += TOPK_THREADS) {
      wkey[i] = ckey[i];
      widx[i] = (int32_t)(s0 + i);
    }
    if (tid == 0) *rec = make_int4(n, 0, 0, 0);
    return;
  }
  uint32_t tau;
  int need;
  radix_select([&](int64_t s) { return ckey[s]; }, n, a.kp, sh, tau, need);
  ordered_pick([&](int64_t s) { return ckey[s]; },
               [&](int pos, int64_t s) {
                 wkey[pos] = ckey[s];
                 widx[pos] = (int32_t)(s0 + s);
               },
               n, tau, need, sh);
  if (tid == 0) *rec = make_int4(a.kp, (int)tau, 1, 0);
}

__global__ __launch_bounds__(TOPK_THREADS) void topk_merge(IdxArgs a) {
  __shared__ uint32_t ckey[TOPK_SPLIT_CAP];
  __shared__ int32_t cidx[TOPK_SPLIT_CAP];
  __shared__ int pcnt[TOPK_MAX_PARTS], poff[TOPK_MAX_PARTS];
  __shared__ TopkShared sh;
  const int tid = threadIdx.x;
  const int64_t jr = blockIdx.x;
  const int b = blockIdx.y;
  const int k = a.k;
  int32_t* out = a.out + ((int64_t)b * a.Tq + a.row0 + jr) * k;
  const int64_t V = visible_entries(a.pos0 + a.row0 + jr, a.m, a.N);
  if (V <= k) {
    for (int i = tid; i < k; i += TOPK_THREADS) out[i] = i < V ? i : -1;
    return;
  }
  const uint8_t* ws = a.sel_ws + ((int64_t)b * a.nrows + jr) * TOPK_SEL_STRIDE;
  const uint32_t* wkey = reinterpret_cast<const uint32_t*>(ws);
  const int32_t* widx = reinterpret_cast<const int32_t*>(ws + (int64_t)TOPK_SPLIT_CAP * 4);
  const int4* rec = reinterpret_cast<const int4*>(ws + (int64_t)TOPK_SPLIT_CAP * 8);
  const int P = (int)((V + a.part_len - 1) / a.part_len);
  const int4 r = tid < P ? rec[tid] : make_int4(0, 0, 0, 0);
  int n_cand;
  const int off = block_exclusive_scan(r.x, sh.wsum, n_cand);
  if (tid < P) {
    pcnt[tid] = r.x;
    poff[tid] = off;
  }
  __syncthreads();
  for (int i = tid; i < P * a.kp; i += TOPK_THREADS) {
    const int p = i / a.kp, e = i - p * a.kp;
    if (e < pcnt[p]) {
      ckey[poff[p] + e] = wkey[i];
      cidx[poff[p] + e] = widx[i];
    }
  }
  __syncthreads();
  const float* row = a.scores + ((int64_t)b * a.rows_ws + jr) * a.ldS;
  if (n_cand < k) {
    select_row_global(row, V, k, out, sh);
    return;
  }
  uint32_t tau;
  int need;
  radix_select([&](int64_t s) { return ckey[s]; }, n_cand, k, sh, tau, need);
  const bool unsafe = tid < P && r.z != 0 && (uint32_t)r.y >= tau;
  if (__syncthreads_or(unsafe)) {
    select_row_global(row, V, k, out, sh);
    return;
  }
  ordered_pick([&](int64_t s) { return ckey[s]; }, [&](int pos, int64_t s) { out[pos] = cidx[s]; }, n_cand,
               tau, need, sh);
}

// Rows of at most BM_MAX_BLOCKS blocks of 32 entries: selection through block maxima.
//  * the largest key of every block of 32 entries of the row (entries past V count as absent):
//    written by the bf16 one-query-per-workgroup scorer as it stores the scores (indexer_topk
//    on decode rows), or else by topk_blockmax (many workgroups) from the score rows.
//  * topk_bm_select (one workgroup per row): tau_b = a lower bound of the k-th largest block
//    maximum (0 when the row has at most k blocks). Each block maximum is an entry's key, so at
//    least k entries reach tau_b: the k-th largest key of the row is >= tau_b, and every entry
//    at or above it sits in a block whose maximum is >= tau_b. The entries >= tau_b of those
//    blocks (about k of them on continuous scores) are gathered in index order, and the exact
//    top-k among them (radix select + in-order pick) is the row's exact top-k, ties included.
//    Should they overflow LDS (many equal scores), the row falls back to the exact select over
//    global memory.
constexpr int BM_CAP = 8192;  // gathered candidates held in LDS

__global__ __launch_bounds__(256) void topk_blockmax(IdxArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t jr = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t V = visible_entries(a.pos0 + a.row0 + jr, a.m, a.N);
  if (V <= a.k) return;
  const int nb = (int)((V + 31) / 32);
  const float* row = a.scores + ((int64_t)b * a.rows_ws + jr) * a.ldS;
  uint32_t* bm = a.bm + ((int64_t)b * a.bm_rows + jr) * a.bm_ld;
  // this workgroup: blocks [256 x, 256 x + 256); wave w: 64 of them, 8 per load (8 lanes per block)
  const int blk0 = blockIdx.x * 256 + wave * 64;
  float4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t e0 = (int64_t)(blk0 + 8 * i) * 32 + 4 * lane;  // rows are padded to 64 entries
    v[i] = e0 < V ? *reinterpret_cast<const float4*>(row + e0) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t e0 = (int64_t)(blk0 + 8 * i) * 32 + 4 * lane;
    const float vv[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t mk = 0;  // absent entries: below every score's key
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e0 + e < V) mk = max(mk, score_key(vv[e]));
    mk = max(mk, (uint32_t)__shfl_xor((int)mk, 1, 64));
    mk = max(mk, (uint32_t)__shfl_xor((int)mk, 2, 64));
    mk = max(mk, (uint32_t)__shfl_xor((int)mk, 4, 64));
    const int blk = blk0 + 8 * i + (lane >> 3);
    if ((lane & 7) == 0 && blk < nb) bm[blk] = mk;
  }
}

// A lower bound of the kk-th largest of the keys held 16 per thread (bk; 0 = absent), 1 <= kk <=
// the number present. The keys between the smallest and the largest present key share every bit
// above the highest bit in which those two differ (hb), so one 2048-bin histogram of the 11 bits
// below and at hb spreads them (few collisions on the same LDS counter); the lower edge of the bin
// that holds the kk-th largest is <= it, and within 2^(hb - 10) of it.
__device__ uint32_t kth_lower_bound(const uint32_t (&bk)[16], int kk, TopkShared& sh) {
  constexpr int NWAVE = TOPK_THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (bk[q]) {
      mx = max(mx, bk[q]);
      mn = min(mn, bk[q]);
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
  }
  if (lane == 0) {
    sh.wsum[wave] = (int)mx;
    sh.wcnt[wave] = (int)mn;
  }
  for (int i = tid; i < 2048; i += TOPK_THREADS) sh.hist[i] = 0;
  __syncthreads();
  mx = 0u;
  mn = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    mx = max(mx, (uint32_t)sh.wsum[w]);
    mn = min(mn, (uint32_t)sh.wcnt[w]);
  }
  if (mx == mn) return mx;  // one distinct key: it is the kk-th largest
  const int hb = 31 - __clz(mx ^ mn);
  const int shift = hb >= 10 ? hb - 10 : 0;
  const uint32_t high = hb >= 31 ? 0u : (mx >> (hb + 1)) << (hb + 1);  // the shared bits above hb
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (bk[q]) atomicAdd(&sh.hist[(bk[q] >> shift) & 2047u], 1);
  __syncthreads();
  constexpr int BPT = 2048 / TOPK_THREADS;
  int cnt[BPT], loc = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    cnt[q] = sh.hist[2047 - (tid * BPT + q)];
    loc += cnt[q];
  }
  int total;
  int above = block_exclusive_scan(loc, sh.wsum, total);
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    if (above < kk && kk <= above + cnt[q]) sh.sel_bin = 2047 - (tid * BPT + q);
    above += cnt[q];
  }
  __syncthreads();
  const uint32_t lb = high | ((uint32_t)sh.sel_bin << shift);
  __syncthreads();
  return lb;
}

__global__ __launch_bounds__(TOPK_THREADS) void topk_bm_select(IdxArgs a) {
  static_assert(BM_MAX_BLOCKS == 16 * TOPK_THREADS, "16 block maxima per thread");
  __shared__ int32_t cblk[BM_MAX_BLOCKS];
  __shared__ uint32_t ckey[BM_CAP];
  __shared__ int32_t cidx[BM_CAP];
  __shared__ TopkShared sh;
  constexpr int NWAVE = TOPK_THREADS / 64;
  constexpr int SEG = BM_CAP / NWAVE;
  constexpr int GB = 16;  // gather loads in flight per lane (8 blocks of 32 entries per wave load)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t jr = blockIdx.x;
  const int b = blockIdx.y;
  const int k = a.k;
  int32_t* out = a.out + ((int64_t)b * a.Tq + a.row0 + jr) * k;
  const int64_t V = visible_entries(a.pos0 + a.row0 + jr, a.m, a.N);
  if (V <= k) {
    for (int i = tid; i < k; i += TOPK_THREADS) out[i] = i < V ? i : -1;
    return;
  }
  const float* row = a.scores + ((int64_t)b * a.rows_ws + jr) * a.ldS;
  const uint32_t* bm = a.bm + ((int64_t)b * a.bm_rows + jr) * a.bm_ld;
  const int nb = (int)((V + 31) / 32);
  // thread t holds block maxima 16 t .. 16 t + 15 (4 vector loads, none past the row's nb
  // blocks, which bm_ld, a multiple of 4, covers; past nb: absent)
  uint32_t bk[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = 16 * tid + 4 * q < nb ? *reinterpret_cast<const uint4*>(bm + 16 * tid + 4 * q) : uint4{0u, 0u, 0u, 0u};
    bk[4 * q] = v.x;
    bk[4 * q + 1] = v.y;
    bk[4 * q + 2] = v.z;
    bk[4 * q + 3] = v.w;
  }
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (16 * tid + q >= nb) bk[q] = 0u;
  // tau_b <= the kb-th largest block maximum (0: every block, when the row has at most k blocks)
  const int kb = k < nb ? k : nb;
  const uint32_t tau_b = kb == nb ? 0u : kth_lower_bound(bk, kb, sh);
  // candidate blocks (maximum >= tau_b) in index order
  int f = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) f += (16 * tid + q < nb && bk[q] >= tau_b) ? 1 : 0;
  int n_cb;
  int pos = block_exclusive_scan(f, sh.wsum, n_cb);
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (16 * tid + q < nb && bk[q] >= tau_b) cblk[pos++] = 16 * tid + q;
  __syncthreads();
  // gather the entries >= tau_b of the candidate blocks: wave w takes candidate blocks
  // [c0, c1), 8 per wave load (8 lanes per block, 4 entries per lane, so lane order is index
  // order), GB loads issued before any is used, and appends to its own LDS segment
  const int L = (n_cb + NWAVE - 1) / NWAVE;
  const int c0 = wave * L, c1 = c0 + L < n_cb ? c0 + L : n_cb;
  uint32_t* wkey = ckey + wave * SEG;
  int32_t* widx = cidx + wave * SEG;
  int cnt = 0;
  for (int c = c0; c < c1; c += 8 * GB) {
    float4 v[GB];
    int64_t e0[GB];
#pragma unroll
    for (int u = 0; u < GB; ++u) {
      const int cc = c + 8 * u + (lane >> 3);
      e0[u] = cc < c1 ? (int64_t)cblk[cc] * 32 + 4 * (lane & 7) : V;
      v[u] = e0[u] < V ? *reinterpret_cast<const float4*>(row + e0[u]) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < GB; ++u) {
      const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t kk4[4];
      bool fl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kk4[e] = score_key(vv[e]);
        fl[e] = e0[u] + e < V && kk4[e] >= tau_b;
      }
      int before, tot;
      wave_count4(fl, before, tot);
      int p = cnt + before;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (fl[e]) {
          if (p < SEG) {
            wkey[p] = kk4[e];
            widx[p] = (int32_t)(e0[u] + e);
          }
          ++p;
        }
      }
      cnt += tot;
    }
  }
  if (lane == 0) sh.wcnt[wave] = cnt;
  __syncthreads();
  int cw[NWAVE], off[NWAVE], total = 0;
  bool overflow = false;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    cw[w] = sh.wcnt[w];
    off[w] = total;
    total += cw[w];
    overflow |= cw[w] > SEG;
  }
  if (overflow || total < k) {  // (total >= k always holds without overflow)
    select_row_global(row, V, k, out, sh);
    return;
  }
  // segments -> one contiguous list in index order
  constexpr int SPT = BM_CAP / TOPK_THREADS;
  uint32_t kr[SPT];
  int32_t ir[SPT];
  int dst[SPT];
#pragma unroll
  for (int q = 0; q < SPT; ++q) {
    const int slot = q * TOPK_THREADS + tid;
    const int w = slot / SEG, e = slot - w * SEG;
    dst[q] = -1;
#pragma unroll
    for (int ww = 0; ww < NWAVE; ++ww)
      if (ww == w && e < cw[ww]) dst[q] = off[ww] + e;
    if (dst[q] >= 0) {
      kr[q] = ckey[slot];
      ir[q] = cidx[slot];
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < SPT; ++q)
    if (dst[q] >= 0) {
      ckey[dst[q]] = kr[q];
      cidx[dst[q]] = ir[q];
    }
  __syncthreads();
  uint32_t tau;
  int need;
  radix_select([&](int64_t s) { return ckey[s]; }, total, k, sh, tau, need);
  ordered_pick([&](int64_t s) { return ckey[s]; }, [&](int p, int64_t s) { out[p] = cidx[s]; }, total, tau, need,
               sh);
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
// Parts for the two-kernel selection: rows of at least 4 parts of TOPK_SPLIT_CAP entries, and
// at most 64 rows in the call (more rows fill the GPU one workgroup per row).
struct SplitPlan {
  int parts, kp;
};

static bool plan_split(int64_t rows, int64_t vmax, int k, SplitPlan& sp) {
  if (rows > 64) return false;
  const int64_t P = ceil_div(vmax, (int64_t)TOPK_SPLIT_CAP);
  if (P < 4 || P > TOPK_MAX_PARTS) return false;
  int64_t kp = round_up(ceil_div(4 * (int64_t)k, P), (int64_t)64);
  if (P * kp > TOPK_SPLIT_CAP) return false;
  sp.parts = (int)P;
  sp.kp = (int)kp;
  return true;
}

int64_t topk_sel_stride() { return TOPK_SEL_STRIDE; }

size_t split_ws_bytes(int64_t rows, int64_t vmax, int k) {
  SplitPlan sp;
  return plan_split(rows, vmax, k, sp) ? (size_t)(rows * TOPK_SEL_STRIDE) : 0;
}

// Selection for rows [a.row0, a.row0 + a.nrows); sel_ws/sel_bytes: optional workspace
// for the two-kernel route.
int launch_select(IdxArgs& a, int batch, void* sel_ws, size_t sel_bytes, hipStream_t st) {
  const int64_t last = a.pos0 + a.row0 + a.nrows - 1;
  int64_t vmax = (last + 1) / a.m;
  if (vmax > a.N) vmax = a.N;
  SplitPlan sp;
  const int64_t rows = (int64_t)batch * a.nrows;
  int64_t vmin = (a.pos0 + a.row0 + 1) / a.m;
  if (vmin > a.N) vmin = a.N;
  if (a.bm_fused) {  // the scorer wrote the block maxima (set only where bm_route holds)
    hipLaunchKernelGGL(topk_bm_select, dim3((unsigned)a.nrows, (unsigned)batch), dim3(TOPK_THREADS), 0, st, a);
    return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
  }
  const bool ws_ok = sel_ws && plan_split(rows, vmax, a.k, sp) && sel_bytes >= (size_t)(rows * TOPK_SEL_STRIDE);
  if (ws_ok && bm_route(vmin, vmax, a.k)) {
    static_assert((int64_t)BM_MAX_BLOCKS * 4 <= TOPK_SEL_STRIDE, "block maxima fit a row's workspace");
    a.sel_ws = (uint8_t*)sel_ws;
    a.bm = reinterpret_cast<uint32_t*>(sel_ws);
    a.bm_ld = TOPK_SEL_STRIDE / 4;
    a.bm_rows = a.nrows;
    hipLaunchKernelGGL(topk_blockmax, dim3((unsigned)ceil_div(ceil_div(vmax, (int64_t)32), (int64_t)256),
                                           (unsigned)a.nrows, (unsigned)batch),
                       dim3(256), 0, st, a);
    hipLaunchKernelGGL(topk_bm_select, dim3((unsigned)a.nrows, (unsigned)batch), dim3(TOPK_THREADS), 0, st, a);
  } else if (ws_ok) {
    a.sel_ws = (uint8_t*)sel_ws;
    a.part_len = TOPK_SPLIT_CAP;
    a.kp = sp.kp;
    hipLaunchKernelGGL(topk_part, dim3((unsigned)sp.parts, (unsigned)a.nrows, (unsigned)batch),
                       dim3(TOPK_THREADS), 0, st, a);
    hipLaunchKernelGGL(topk_merge, dim3((unsigned)a.nrows, (unsigned)batch), dim3(TOPK_THREADS), 0, st, a);
  } else {
    hipLaunchKernelGGL(topk_select, dim3((unsigned)a.nrows, (unsigned)batch), dim3(TOPK_THREADS), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? CSKV_OK : CSKV_ERR_HIP;
}

}  // namespace cskv

using namespace cskv;

extern "C" size_t cskv_topk_workspace_size(int batch, int64_t Tq, int64_t N, int k) {
  if (batch <= 0 || Tq <= 0 || k < 1) return 0;
  return split_ws_bytes((int64_t)batch * Tq, N, k);
}

extern "C" int topk_select(const float* scores, int64_t ld, const uint32_t* block_max, int64_t bm_ld, int batch,
                           int64_t Tq, int64_t N, int64_t pos0, int m, int k, int32_t* out_idx, void* workspace,
                           size_t ws_bytes, void* stream) {
  if (batch < 0 || Tq < 0 || N < 0 || pos0 < 0 || m < 1 || ld < N) return CSKV_ERR_BAD_SHAPE;
  if (ld % 4 != 0) return CSKV_ERR_BAD_SHAPE;
  if (block_max && (bm_ld < ceil_div(N, (int64_t)32) || bm_ld % 4 != 0)) return CSKV_ERR_BAD_SHAPE;
  if (k < 1) return CSKV_ERR_BAD_SHAPE;
  if (k > CSKV_MAX_TOPK) return CSKV_ERR_UNSUPPORTED;
  if (batch == 0 || Tq == 0) return CSKV_OK;
  if (!out_idx || (N > 0 && !scores)) return CSKV_ERR_INVALID_ARG;
  if (!aligned16(scores, out_idx, workspace, block_max)) return CSKV_ERR_MISALIGNED;
  IdxArgs a{};
  a.scores = (float*)scores; a.out = out_idx;
  a.Tq = Tq; a.N = N; a.pos0 = pos0; a.ldS = ld; a.rows_ws = Tq; a.row0 = 0; a.nrows = Tq;
  a.m = m; a.k = k;
  int64_t vmin = (pos0 + 1) / m, vmax = (pos0 + Tq) / m;
  if (vmin > N) vmin = N;
  if (vmax > N) vmax = N;
  if (block_max && Tq < 64 && bm_route(vmin, vmax, k)) {  // block maxima written by indexer_scores
    a.bm = const_cast<uint32_t*>(block_max);
    a.bm_ld = bm_ld;
    a.bm_rows = Tq;
    a.bm_fused = 1;
  }
  return launch_select(a, batch, workspace, workspace ? ws_bytes : 0, (hipStream_t)stream);
}
