// indexer.hip -- Lightning-Indexer scores and exact top-k selection.
//
// QbitAI rewrite (futuo-fx-trading.com), lightning indexer + top-k step: a
// light indexer scores every compressed KV block against each query token and
// only the best blocks are kept; "深度解析 DeepSeek-V4", CSA Step 2 Select;
// "DeepSeek V4的4个技巧", 技巧1: the top 2048 blocks.  Score of entry j for
// query t (visible only when j < floor(t/m), strict causality):
//     s[j] = sum_h w[h] * max(0, q[h] . K[j]).
//
// Score kernel (bf16).  One query's H_I x d_I block against 32 keys is one
// tile of v_mfma_f32_32x32x16_bf16 per (32 heads, 16 dims): the heads are the
// M side (A operand, kept in VGPRs for the whole sweep), the keys the N side
// (B operand, streamed from HBM), the indexer dim the K side.  Because the
// contraction order is free, each lane reads one contiguous half-row of its
// key (d_I bytes), so a wave consumes whole 128-byte lines.  The ReLU and the
// w-weighted head sum run on the accumulator in place: a lane holds one key
// and 16 of the 32 heads, so one cross-half shuffle finishes the head sum.
// Scores go to workspace as fp32.
//
// Top-k.  Keys are the order-preserving uint32 images of the fp32 scores.
//  * Row-wise path (many rows, or short rows): one workgroup per row runs a
//    4-pass MSD radix select (8-bit digits, LDS histograms with wave-level
//    aggregation of equal digits), then one ordered pass that keeps every key
//    above the threshold and the lowest-index keys equal to it, written in
//    ascending index order through a block-wide prefix count.
//  * Split path (few long rows, e.g. decode at 1M tokens): many workgroups
//    per row build a 12-bit histogram, then filter their chunks (keys above
//    the threshold bucket go straight to the selection, keys in it become
//    candidates), and one workgroup per row resolves the candidates with the
//    same radix select, breaks ties by index and sorts the final set
//    (bitonic, in LDS) into ascending index order.
// Both paths give the same set: first min(k, n_vis) under (score desc, index
// asc).  Deterministic: no floating-point atomics, ordered output.
#include "lac_internal.h"

namespace lac {

namespace {

constexpr int kTopkThreads = 512;
constexpr int kSplitChunk = 4096;      // scores per workgroup in the split path
constexpr int kHistBins = 4096;        // 12-bit first digit of the split path

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct ScoreArgs {
  const void* q;
  const float* w;
  const void* K;
  float* scores;          // [R, Np]
  int B, Tq, HI, dI, N, m;
  int64_t Np;
  int tiles_per_wave;     // 32-key tiles per wave
  uint32_t* hist;         // [R, kHistBins] 12-bit key histogram (split path) or null
  Positions qpos;
};

// Wave-aggregated LDS histogram add: lanes with equal digits add once.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool on, uint32_t d) {
  uint64_t active = __ballot(on);
  while (active) {
    const int leader = __ffsll((unsigned long long)active) - 1;
    const uint32_t dl = __shfl(d, leader);
    const uint64_t same = __ballot(on && d == dl) & active;
    if (lane_id() == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(same));
    active &= ~same;
  }
}

// ---------------------------------------------------------------- fp32 scores (VALU)
__global__ void __launch_bounds__(256) score_f32_kernel(ScoreArgs a) {
  extern __shared__ float sq[];   // [HI * dI] query + [HI] weights
  const int row = blockIdx.y;
  const int b = row / a.Tq, i = row - b * a.Tq;
  const int64_t t = (int64_t)a.qpos.v[b] + i;
  const int64_t nv = n_visible(t, a.N, a.m);
  const float* q = static_cast<const float*>(a.q) + (int64_t)row * a.HI * a.dI;
  for (int e = threadIdx.x; e < a.HI * a.dI; e += blockDim.x) sq[e] = q[e];
  for (int e = threadIdx.x; e < a.HI; e += blockDim.x) sq[a.HI * a.dI + e] = a.w[(int64_t)row * a.HI + e];
  __syncthreads();
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= nv) return;
  const float* kr = static_cast<const float*>(a.K) + ((int64_t)b * a.N + j) * a.dI;
  float s = 0.f;
  for (int h = 0; h < a.HI; ++h) {
    float dot = 0.f;
    for (int c = 0; c < a.dI; ++c) dot = fmaf(sq[h * a.dI + c], kr[c], dot);
    s = fmaf(sq[a.HI * a.dI + h], fmaxf(dot, 0.f), s);
  }
  a.scores[row * a.Np + j] = s;
  if (a.hist) atomicAdd(&a.hist[(int64_t)row * kHistBins + (score_key(s) >> 20)], 1u);
}

// ---------------------------------------------------------------- bf16 scores (MFMA)
// Block = 4 waves.  RW waves along rows (each with QPW consecutive queries of
// one sequence), 4/RW waves along keys.  Grid: x = key chunks, y = row groups.
//
// Keys reach the MFMA through a per-wave LDS tile: every global load
// instruction reads 1 KB of consecutive key rows (fully used 128-byte lines),
// written to LDS with the 16-byte chunks of each row XOR-swizzled by the row
// index, so the MFMA-layout reads (one chunk of 32 different rows per half
// wave) are free of bank conflicts.  The next tile is loaded into VGPRs while
// the current one is consumed from LDS.
template <int HT, int KS, int QPW, int RW>
__global__ void __launch_bounds__(256) score_bf16_kernel(ScoreArgs a) {
  constexpr int kRowsPerBlock = RW * QPW;
  constexpr int KW = 4 / RW;
  constexpr int dI = KS * 16;
  constexpr int HI = HT * 32;
  constexpr int CH = dI / 8;                 // 16-byte chunks per key row
  constexpr int ROWB = dI * 2;               // bytes per key row
  constexpr int TILEB = 32 * ROWB;           // bytes per 32-key tile
  constexpr int NLD = TILEB / 1024;          // 1 KB load instructions per tile
  __shared__ float sw[kRowsPerBlock][HI];
  __shared__ __align__(16) uint8_t ktile[4][TILEB];
  __shared__ uint32_t lhist[kHistBins];
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int hf = l >> 5, ln = l & 31;
  const int wr = wave % RW, wk = wave / RW;
  const bool do_hist = a.hist != nullptr;

  // Rows of this block: consecutive queries of one sequence.
  const int groups_per_seq = (a.Tq + kRowsPerBlock - 1) / kRowsPerBlock;
  const int b = blockIdx.y / groups_per_seq;
  const int i0 = (blockIdx.y - b * groups_per_seq) * kRowsPerBlock;
  const int n_rows_blk = min(kRowsPerBlock, a.Tq - i0);
  const int64_t t_last = (int64_t)a.qpos.v[b] + i0 + n_rows_blk - 1;
  const int64_t nv_max = n_visible(t_last, a.N, a.m);

  for (int e = threadIdx.x; e < kRowsPerBlock * HI; e += 256) {
    const int rr = e / HI, h = e - rr * HI;
    const int i = min(i0 + rr, a.Tq - 1);
    sw[rr][h] = a.w[((int64_t)b * a.Tq + i) * HI + h];
  }
  if (do_hist)
    for (int e = threadIdx.x; e < kHistBins; e += 256) lhist[e] = 0u;
  __syncthreads();

  const int64_t tile_lo = ((int64_t)blockIdx.x * KW + wk) * a.tiles_per_wave;
  int64_t tile_hi = tile_lo + a.tiles_per_wave;
  const int64_t n_tiles = (nv_max + 31) / 32;
  if (tile_hi > n_tiles) tile_hi = n_tiles;

  if (tile_lo < tile_hi) {
    // Query fragments: lane (ln, hf) holds head ht*32+ln, dims hf*dI/2 + s*8 .. +8.
    bf16x8 qf[QPW][HT][KS];
    int64_t nv_row[QPW];
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
      const int rr = wr * QPW + qi;
      const int i = min(i0 + rr, a.Tq - 1);
      nv_row[qi] = (i0 + rr < a.Tq) ? n_visible((int64_t)a.qpos.v[b] + i, a.N, a.m) : 0;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const __bf16* qp = static_cast<const __bf16*>(a.q) +
                           ((((int64_t)b * a.Tq + i) * HI) + ht * 32 + ln) * dI + hf * (dI / 2);
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[qi][ht][s] = *reinterpret_cast<const bf16x8*>(qp + s * 8);
      }
    }

    const uint8_t* Kb = static_cast<const uint8_t*>(a.K) + (int64_t)b * a.N * ROWB;
    uint8_t* kt = ktile[wave];
    // Load instruction u of a tile: lane l takes 16 bytes at u*1024 + l*16 of
    // the tile in LDS order, i.e. row kk, swizzled chunk slot cs, which holds
    // the row's chunk cs ^ (kk % CH).
    auto load_tile = [&](int64_t tile, uint4* st) {
#pragma unroll
      for (int u = 0; u < NLD; ++u) {
        const int o = u * 1024 + l * 16;
        const int kk = o / ROWB, cs = (o % ROWB) / 16;
        int64_t j = tile * 32 + kk;
        if (j > a.N - 1) j = a.N - 1;
        st[u] = ld_stream16(Kb + j * ROWB + ((cs ^ (kk % CH)) * 16));
      }
    };
    auto store_tile = [&](const uint4* st) {
#pragma unroll
      for (int u = 0; u < NLD; ++u) *reinterpret_cast<uint4*>(kt + u * 1024 + l * 16) = st[u];
    };

    uint4 stage[NLD];
    load_tile(tile_lo, stage);
    for (int64_t tile = tile_lo; tile < tile_hi; ++tile) {
      store_tile(stage);
      __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): LDS writes done
      __builtin_amdgcn_wave_barrier();
      if (tile + 1 < tile_hi) load_tile(tile + 1, stage);
      bf16x8 kf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int c = hf * (CH / 2) + s;
        kf[s] = *reinterpret_cast<const bf16x8*>(kt + ln * ROWB + ((c ^ (ln % CH)) * 16));
      }
      const int64_t j = tile * 32 + ln;
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        const int rr = wr * QPW + qi;
        float part = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          f32x16 acc = {};
#pragma unroll
          for (int s = 0; s < KS; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[qi][ht][s], kf[s], acc, 0, 0, 0);
          // acc[v] is head ht*32 + 8*(v/4) + 4*hf + v%4 against key j.
#pragma unroll
          for (int v = 0; v < 16; ++v)
            part = fmaf(sw[rr][ht * 32 + 8 * (v >> 2) + 4 * hf + (v & 3)], fmaxf(acc[v], 0.f), part);
        }
        part += __shfl_xor(part, 32);
        const bool live = hf == 0 && j < nv_row[qi];
        if (live) a.scores[((int64_t)b * a.Tq + i0 + rr) * a.Np + j] = part;
        if (do_hist) hist_add(lhist, live, score_key(part) >> 20);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);      // LDS reads of this tile done
      __builtin_amdgcn_wave_barrier();
    }
  }

  if (do_hist) {
    __syncthreads();
    // Only the decode shape (one row per block) keeps a histogram.
    uint32_t* gh = a.hist + ((int64_t)b * a.Tq + i0) * kHistBins;
    for (int e = threadIdx.x; e < kHistBins; e += 256)
      if (lhist[e]) atomicAdd(&gh[e], lhist[e]);
  }
}

// ---------------------------------------------------------------- radix select
// Finds, from the top digit down, the digit where the running count reaches
// `need`.  Run by wave 0 only, over a 256-bin histogram.  Writes
// out[0] = digit, out[1] = count of all digits above it, out[2] = its count.
__device__ void find_digit(const uint32_t* hist, uint32_t need, uint32_t* out) {
  const int l = lane_id();
  uint32_t c[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) { c[q] = hist[255 - 4 * l - q]; sum += c[q]; }
  uint32_t incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_up(incl, o);
    if (l >= o) incl += v;
  }
  const uint64_t hit = __ballot(incl >= need);
  const int L = __ffsll((unsigned long long)hit) - 1;
  if (l == L) {
    uint32_t cum = incl - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (cum + c[q] >= need) {
        out[0] = 255 - 4 * l - q;
        out[1] = cum;
        out[2] = c[q];
        break;
      }
      cum += c[q];
    }
  }
}

// Block-wide MSD radix select over n elements.  keyf(e, &u) returns whether
// element e takes part and its key.  Result: thr = key of the need-th largest
// element, need_eq = how many elements equal to thr belong to the top `need`,
// cnt_eq = how many elements equal thr.
template <class KeyFn>
__device__ void radix_select(int n, uint32_t need, KeyFn keyf, uint32_t* hist, uint32_t* bc,
                             uint32_t& thr, uint32_t& need_eq, uint32_t& cnt_eq) {
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int e = threadIdx.x; e < 256; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int n_iter = (n + blockDim.x - 1) / blockDim.x;
    for (int it = 0; it < n_iter; ++it) {
      const int e = it * blockDim.x + threadIdx.x;
      uint32_t u = 0;
      const bool on = e < n && keyf(e, &u) && (u & mask) == prefix;
      hist_add(hist, on, (u >> shift) & 255u);
    }
    __syncthreads();
    if (threadIdx.x < 64) find_digit(hist, need, bc);
    __syncthreads();
    need -= bc[1];
    prefix |= bc[0] << shift;
    mask |= 255u << shift;
    cnt_eq = bc[2];
    __syncthreads();
  }
  thr = prefix;
  need_eq = need;
}

// Block-wide exclusive prefix counts of two flags, in thread order.
__device__ __forceinline__ void block_count2(bool f0, bool f1, uint32_t* lds, uint32_t& ex0,
                                             uint32_t& ex1, uint32_t& tot0, uint32_t& tot1) {
  const int l = lane_id(), wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint64_t b0 = __ballot(f0), b1 = __ballot(f1);
  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
  if (l == 0) { lds[wv] = (uint32_t)__popcll(b0); lds[32 + wv] = (uint32_t)__popcll(b1); }
  __syncthreads();
  uint32_t p0 = 0, p1 = 0, s0 = 0, s1 = 0;
  for (int w = 0; w < nw; ++w) {
    const uint32_t c0 = lds[w], c1 = lds[32 + w];
    if (w < wv) { p0 += c0; p1 += c1; }
    s0 += c0; s1 += c1;
  }
  ex0 = p0 + (uint32_t)__popcll(b0 & below);
  ex1 = p1 + (uint32_t)__popcll(b1 & below);
  tot0 = s0; tot1 = s1;
  __syncthreads();
}

struct TopkArgs {
  const float* scores;    // [R, Np]
  int64_t Np;
  int B, Tq, N, m, k;
  int32_t* idx;           // [R, k]
  float* score_out;       // [R, k] or null
  uint32_t* hist;         // split path: [R, kHistBins]
  uint32_t* cnt;          // split path: [R, 4] (selected, candidates)
  int32_t* sel;           // split path: [R, k]
  uint2* cand;            // split path: [R, Np] (key, index)
  int chunks;             // split path: workgroups per row
  Positions qpos;
};

__device__ __forceinline__ int64_t row_nvis(const TopkArgs& a, int row) {
  const int b = row / a.Tq, i = row - b * a.Tq;
  return n_visible((int64_t)a.qpos.v[b] + i, a.N, a.m);
}

// Writes 0..nv-1 and pads: the case k >= n_vis.
__device__ void write_all_visible(const TopkArgs& a, int row, int nv) {
  const float* s = a.scores + (int64_t)row * a.Np;
  for (int e = threadIdx.x; e < a.k; e += blockDim.x) {
    a.idx[(int64_t)row * a.k + e] = e < nv ? e : -1;
    if (a.score_out) a.score_out[(int64_t)row * a.k + e] = e < nv ? s[e] : -INFINITY;
  }
}

__global__ void __launch_bounds__(kTopkThreads) topk_rowwise_kernel(TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bc[4];
  __shared__ uint32_t cnt[64];
  const int row = blockIdx.x;
  const int nv = (int)row_nvis(a, row);
  const int keff = min(a.k, nv);
  if (keff == nv) { write_all_visible(a, row, nv); return; }
  const float* s = a.scores + (int64_t)row * a.Np;
  uint32_t thr, need_eq, cnt_eq;
  radix_select(nv, (uint32_t)keff,
               [&](int e, uint32_t* u) { *u = score_key(s[e]); return true; }, hist, bc, thr,
               need_eq, cnt_eq);
  (void)cnt_eq;
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < nv; base += blockDim.x) {
    const int e = base + threadIdx.x;
    const uint32_t u = e < nv ? score_key(s[e]) : 0u;
    const bool gt = e < nv && u > thr, eq = e < nv && u == thr;
    uint32_t ex_gt, ex_eq, tot_gt, tot_eq;
    block_count2(gt, eq, cnt, ex_gt, ex_eq, tot_gt, tot_eq);
    const uint32_t eq_before = run_eq + ex_eq;
    if (gt || (eq && eq_before < need_eq)) {
      const uint32_t pos = run_gt + ex_gt + min(eq_before, need_eq);
      a.idx[(int64_t)row * a.k + pos] = e;
      if (a.score_out) a.score_out[(int64_t)row * a.k + pos] = s[e];
    }
    run_gt += tot_gt;
    run_eq += tot_eq;
  }
  for (int e = keff + threadIdx.x; e < a.k; e += blockDim.x) {
    a.idx[(int64_t)row * a.k + e] = -1;
    if (a.score_out) a.score_out[(int64_t)row * a.k + e] = -INFINITY;
  }
}

// ---------------------------------------------------------------- split path
__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The 12-bit bucket holding the keff-th largest key, and the count above it.
__device__ void split_threshold(const uint32_t* gh, uint32_t need, uint32_t* lds,
                                uint32_t* bucket, uint32_t* above) {
  // Thread t covers buckets 4095-16t .. 4080-16t (descending).
  const int t = threadIdx.x;
  uint32_t c[16], sum = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) { c[q] = gh[kHistBins - 1 - 16 * t - q]; sum += c[q]; }
  // block inclusive scan over 256 threads
  const int l = lane_id(), wv = t >> 6;
  uint32_t incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_up(incl, o);
    if (l >= o) incl += v;
  }
  if (l == 63) lds[wv] = incl;
  __syncthreads();
  for (int w = 0; w < wv; ++w) incl += lds[w];
  const uint32_t excl = incl - sum;
  if (excl < need && incl >= need) {
    uint32_t cum = excl;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (cum + c[q] >= need) {
        lds[8] = kHistBins - 1 - 16 * t - q;
        lds[9] = cum;
        break;
      }
      cum += c[q];
    }
  }
  __syncthreads();
  *bucket = lds[8];
  *above = lds[9];
  __syncthreads();
}

// Block-wide exclusive prefix sums of two per-thread counts (256 threads).
__device__ __forceinline__ void block_scan2(uint32_t v0, uint32_t v1, uint32_t* lds, uint32_t& ex0,
                                            uint32_t& ex1, uint32_t& tot0, uint32_t& tot1) {
  const int l = lane_id(), wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t i0 = v0, i1 = v1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t a0 = __shfl_up(i0, o), a1 = __shfl_up(i1, o);
    if (l >= o) { i0 += a0; i1 += a1; }
  }
  if (l == 63) { lds[wv] = i0; lds[16 + wv] = i1; }
  __syncthreads();
  uint32_t p0 = 0, p1 = 0, s0 = 0, s1 = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wv) { p0 += lds[w]; p1 += lds[16 + w]; }
    s0 += lds[w]; s1 += lds[16 + w];
  }
  ex0 = p0 + i0 - v0;
  ex1 = p1 + i1 - v1;
  tot0 = s0; tot1 = s1;
  __syncthreads();
}

__global__ void __launch_bounds__(256) topk_filter_kernel(TopkArgs a) {
  constexpr int kPer = kSplitChunk / 256;
  __shared__ uint32_t lds[40];
  const int row = blockIdx.y;
  const int nv = (int)row_nvis(a, row);
  const int keff = min(a.k, nv);
  if (keff == nv) return;
  const int lo = blockIdx.x * kSplitChunk;
  if (lo >= nv) return;
  const int hi = min(nv, lo + kSplitChunk);
  uint32_t bucket, above;
  split_threshold(a.hist + (int64_t)row * kHistBins, (uint32_t)keff, lds, &bucket, &above);
  const float* s = a.scores + (int64_t)row * a.Np;
  uint32_t key[kPer];
  uint32_t n_up = 0, n_in = 0;
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int e = lo + it * 256 + threadIdx.x;
    key[it] = e < hi ? score_key(s[e]) : 0u;
    n_up += (e < hi && (key[it] >> 20) > bucket);
    n_in += (e < hi && (key[it] >> 20) == bucket);
  }
  uint32_t ex_up, ex_in, tot_up, tot_in;
  block_scan2(n_up, n_in, lds, ex_up, ex_in, tot_up, tot_in);
  uint32_t* cnt = a.cnt + (int64_t)row * 4;
  if (threadIdx.x == 0) {
    lds[32] = tot_up ? atomicAdd(&cnt[0], tot_up) : 0u;
    lds[33] = tot_in ? atomicAdd(&cnt[1], tot_in) : 0u;
  }
  __syncthreads();
  uint32_t pu = lds[32] + ex_up, pi = lds[33] + ex_in;
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int e = lo + it * 256 + threadIdx.x;
    if (e >= hi) continue;
    const uint32_t bk = key[it] >> 20;
    if (bk > bucket) a.sel[(int64_t)row * a.k + pu++] = e;
    else if (bk == bucket) a.cand[(int64_t)row * a.Np + pi++] = make_uint2(key[it], (uint32_t)e);
  }
}

// Bitonic sort of n (power of two) int32 in LDS, ascending.
__device__ void bitonic_sort(int32_t* v, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += blockDim.x) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int32_t x = v[lo], y = v[hi];
        if ((x > y) == up) { v[lo] = y; v[hi] = x; }
      }
      __syncthreads();
    }
  }
}

constexpr int kCandLds = 6144;         // candidates staged in LDS by the resolve step

__global__ void __launch_bounds__(1024) topk_resolve_kernel(TopkArgs a) {
  extern __shared__ __align__(16) uint8_t rsm[];
  uint2* lcand = reinterpret_cast<uint2*>(rsm);                 // [kCandLds]
  int32_t* list = reinterpret_cast<int32_t*>(lcand + kCandLds);  // [next_pow2(k)]
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bc[4];
  __shared__ uint32_t n_list;
  const int row = blockIdx.x;
  const int nv = (int)row_nvis(a, row);
  const int keff = min(a.k, nv);
  if (keff == nv) { write_all_visible(a, row, nv); return; }
  const uint32_t* cnt = a.cnt + (int64_t)row * 4;
  const uint32_t n_sel = cnt[0], n_cand = cnt[1];
  const uint2* gcand = a.cand + (int64_t)row * a.Np;
  const bool in_lds = n_cand <= (uint32_t)kCandLds;
  int pow2 = 1;
  while (pow2 < keff) pow2 <<= 1;
  for (int e = threadIdx.x; e < pow2; e += blockDim.x)
    list[e] = e < (int)n_sel ? a.sel[(int64_t)row * a.k + e] : INT32_MAX;
  if (in_lds)
    for (int e = threadIdx.x; e < (int)n_cand; e += blockDim.x) lcand[e] = gcand[e];
  if (threadIdx.x == 0) n_list = n_sel;
  __syncthreads();
  const uint2* cand = in_lds ? lcand : gcand;
  const uint32_t need = (uint32_t)keff - n_sel;
  uint32_t thr, need_eq, cnt_eq;
  radix_select((int)n_cand, need,
               [&](int e, uint32_t* u) { *u = cand[e].x; return true; }, hist, bc, thr, need_eq,
               cnt_eq);
  // Ties at the threshold: keep the need_eq lowest indices (largest ~index).
  uint32_t thr2 = 0;
  if (cnt_eq > need_eq) {
    uint32_t ne2, ce2;
    radix_select((int)n_cand, need_eq,
                 [&](int e, uint32_t* u) {
                   const uint2 c = cand[e];
                   *u = ~c.y;
                   return c.x == thr;
                 },
                 hist, bc, thr2, ne2, ce2);
  }
  for (int e = threadIdx.x; e < (int)n_cand; e += blockDim.x) {
    const uint2 c = cand[e];
    if (c.x > thr || (c.x == thr && ~c.y >= thr2)) {
      const uint32_t pos = atomicAdd(&n_list, 1u);
      if (pos < (uint32_t)pow2) list[pos] = (int32_t)c.y;
    }
  }
  __syncthreads();
  bitonic_sort(list, pow2);
  const float* s = a.scores + (int64_t)row * a.Np;
  for (int e = threadIdx.x; e < a.k; e += blockDim.x) {
    const int32_t j = e < keff ? list[e] : -1;
    a.idx[(int64_t)row * a.k + e] = j;
    if (a.score_out) a.score_out[(int64_t)row * a.k + e] = j >= 0 ? s[j] : -INFINITY;
  }
}

// ---------------------------------------------------------------- plan
struct Plan {
  int64_t Np;
  bool split;
  int chunks;
  size_t off_scores, off_hist, off_cnt, off_sel, off_cand, total;
};

Plan make_plan(int B, int Tq, int N, int k) {
  Plan p{};
  const int64_t R = (int64_t)B * Tq;
  p.Np = round_up(N > 0 ? N : 1, 64);
  p.split = R <= 64 && N > 16384;
  p.chunks = (int)((N + kSplitChunk - 1) / kSplitChunk);
  size_t off = 0;
  p.off_scores = off;
  off += round_up(R * p.Np * 4, 256);
  if (p.split) {
    p.off_hist = off;
    off += round_up(R * kHistBins * 4, 256);
    p.off_cnt = off;
    off += round_up(R * 16, 256);
    p.off_sel = off;
    off += round_up(R * (int64_t)k * 4, 256);
    p.off_cand = off;
    off += round_up(R * p.Np * 8, 256);
  }
  p.total = off;
  return p;
}

template <int HT, int KS, int QPW, int RW>
hipError_t launch_score(const ScoreArgs& sa, int64_t key_chunks, int row_groups, hipStream_t st) {
  hipLaunchKernelGGL((score_bf16_kernel<HT, KS, QPW, RW>), dim3((unsigned)key_chunks, row_groups),
                     dim3(256), 0, st, sa);
  return hipGetLastError();
}

}  // namespace

size_t indexer_workspace_bytes(int B, int Tq, int N, int k) { return make_plan(B, Tq, N, k).total; }

hipError_t launch_indexer_topk(const IndexerArgs& a, void* ws, hipStream_t st) {
  const Plan p = make_plan(a.B, a.Tq, a.N, a.k);
  const int R = a.B * a.Tq;
  if (R == 0) return hipSuccess;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  float* scores = reinterpret_cast<float*>(w8 + p.off_scores);
  hipError_t err = hipSuccess;

  TopkArgs ta{};
  ta.scores = scores; ta.Np = p.Np; ta.B = a.B; ta.Tq = a.Tq; ta.N = a.N; ta.m = a.m; ta.k = a.k;
  ta.idx = a.topk_idx; ta.score_out = a.topk_score; ta.qpos = a.qpos; ta.chunks = p.chunks;
  if (p.split) {
    ta.hist = reinterpret_cast<uint32_t*>(w8 + p.off_hist);
    ta.cnt = reinterpret_cast<uint32_t*>(w8 + p.off_cnt);
    ta.sel = reinterpret_cast<int32_t*>(w8 + p.off_sel);
    ta.cand = reinterpret_cast<uint2*>(w8 + p.off_cand);
    // The score kernel accumulates into the histogram: clear it (and the
    // adjacent counters) first, with a kernel rather than a memset.
    const int64_t n_clear = (int64_t)(p.off_sel - p.off_hist) / 4;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n_clear + 255) / 256)), dim3(256), 0, st,
                       ta.hist, n_clear);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }

  // Largest visible count over all rows sizes the key sweep.
  int64_t nv_max = 0;
  for (int b = 0; b < a.B; ++b) {
    const int64_t t = (int64_t)a.qpos.v[b] + a.Tq - 1;
    int64_t nv = t >= 0 ? t / a.m : 0;
    if (nv > a.N) nv = a.N;
    if (nv > nv_max) nv_max = nv;
  }

  ScoreArgs sa{};
  sa.q = a.q; sa.w = a.w; sa.K = a.K; sa.scores = scores;
  sa.B = a.B; sa.Tq = a.Tq; sa.HI = a.HI; sa.dI = a.dI; sa.N = a.N; sa.m = a.m;
  sa.Np = p.Np; sa.qpos = a.qpos; sa.hist = ta.hist;
  if (nv_max > 0) {
    TimedLaunch tl(kKernelIndexerScore, st);
    if (a.fmt == kF32) {
      const size_t lds = (size_t)(a.HI * a.dI + a.HI) * 4;
      hipLaunchKernelGGL(score_f32_kernel, dim3((unsigned)((nv_max + 255) / 256), R), dim3(256),
                         lds, st, sa);
      err = hipGetLastError();
    } else {
      const int64_t n_tiles = (nv_max + 31) / 32;
      const int HT = a.HI / 32, KS = a.dI / 16;
      if (a.Tq >= 8 && !p.split) {
        // Prefill: 4 waves x 2 queries share each key sweep.
        sa.tiles_per_wave = 64;
        const int64_t chunks = (n_tiles + sa.tiles_per_wave - 1) / sa.tiles_per_wave;
        const int groups = a.B * ((a.Tq + 7) / 8);
#define LAC_SCORE_CASE(ht, ks) \
  if (HT == ht && KS == ks) err = launch_score<ht, ks, 2, 4>(sa, chunks, groups, st);
        LAC_SCORE_CASE(1, 4) LAC_SCORE_CASE(1, 8) LAC_SCORE_CASE(2, 4) LAC_SCORE_CASE(2, 8)
        LAC_SCORE_CASE(4, 4) LAC_SCORE_CASE(4, 8)
#undef LAC_SCORE_CASE
      } else {
        // Decode: one query per block, 4 waves split the keys.
        sa.tiles_per_wave = 8;
        const int64_t chunks = (n_tiles + 4 * sa.tiles_per_wave - 1) / (4 * sa.tiles_per_wave);
        const int groups = a.B * a.Tq;
#define LAC_SCORE_CASE(ht, ks) \
  if (HT == ht && KS == ks) err = launch_score<ht, ks, 1, 1>(sa, chunks, groups, st);
        LAC_SCORE_CASE(1, 4) LAC_SCORE_CASE(1, 8) LAC_SCORE_CASE(2, 4) LAC_SCORE_CASE(2, 8)
        LAC_SCORE_CASE(4, 4) LAC_SCORE_CASE(4, 8)
#undef LAC_SCORE_CASE
      }
    }
    if (err != hipSuccess) return err;
  }

  if (!p.split) {
    TimedLaunch tl(kKernelTopk, st);
    hipLaunchKernelGGL(topk_rowwise_kernel, dim3(R), dim3(kTopkThreads), 0, st, ta);
    return hipGetLastError();
  }
  {
    TimedLaunch tl(kKernelTopk, st);
    hipLaunchKernelGGL(topk_filter_kernel, dim3(p.chunks, R), dim3(256), 0, st, ta);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  int pow2 = 1;
  while (pow2 < a.k) pow2 <<= 1;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&topk_resolve_kernel),
      hipFuncAttributeMaxDynamicSharedMemorySize, kCandLds * 8 + 8192 * 4);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(topk_resolve_kernel, dim3(R), dim3(1024),
                     (size_t)kCandLds * 8 + (size_t)pow2 * 4, st, ta);
  return hipGetLastError();
}

}  // namespace lac
