// score.hip -- Lightning-Indexer scores.
//
// QbitAI rewrite (futuo-fx-trading.com), lightning indexer + top-k step: a
// light indexer scores every compressed KV block against each query token;
// "深度解析 DeepSeek-V4", CSA Step 2 Select.  Score of entry j for query t
// (visible only when j < floor(t/m), strict causality):
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
#include <algorithm>

#include "lac_internal.h"

namespace lac {

namespace {

constexpr int kHistBins = kScoreHistBins;
// Decode score launches: tile stages in flight per wave (bf16 keys, E4M3
// keys) and the blocks the grid spreads over (bf16, E4M3 queries).
constexpr int kStagesBF16 = 2, kStagesF8 = 2, kStagesFP4 = 4;
constexpr int kDecodeBlocksBF16 = 512, kDecodeBlocksF8 = 768, kDecodeBlocksFP4 = 512;

// E4M3 key tiles in LDS (E4M3 queries): a row is d_I bytes, its 16-byte
// chunks XOR-swizzled by f8_swz(row), chosen so that the MFMA-layout reads
// (one 16-byte chunk of each of 8 consecutive rows per LDS pass) hit distinct
// bank groups: with d_I = 64 two rows share a 128-byte line, so the swizzle
// follows the line index.
template <int dI>
__device__ __forceinline__ int f8_swz(int row) {
  static_assert(dI == 64 || dI == 128, "E4M3 score tiles take d_I of 64 or 128");
  return (row / (128 / dI)) % (dI / 16);
}
// The byte offset in the HBM tile of the 16 bytes at LDS offset o of a
// swizzled E4M3 tile: physical chunk p of row kk holds its chunk p ^ f8_swz(kk).
template <int dI>
__device__ __forceinline__ int f8_src(int o) {
  const int kk = o / dI, p = (o % dI) / 16;
  return kk * dI + ((p ^ f8_swz<dI>(kk)) * 16);
}
// Fragments 2c and 2c + 1 of a lane (8 codes each) from its row's logical
// 16-byte chunk c of a swizzled E4M3 tile.
template <int dI>
__device__ __forceinline__ void f8_pair(const uint8_t* kt, int row, int c, long* f) {
  const uint4 v = *reinterpret_cast<const uint4*>(kt + row * dI + ((c ^ f8_swz<dI>(row)) * 16));
  f[0] = (long)((uint64_t)v.x | ((uint64_t)v.y << 32));
  f[1] = (long)((uint64_t)v.z | ((uint64_t)v.w << 32));
}

struct ScoreArgs {
  const void* q;
  const float* w;
  const void* K;
  float* scores;          // [R, Np]
  int B, Tq, HI, dI, N, m;
  int64_t Np;
  int tiles_per_wave;     // 32-key tiles per wave (static schedule)
  uint32_t* hist;         // [R, kHistBins] 12-bit key histogram (split path) or null
  uint32_t* tile_ctr;     // [R, 16 * 32] zeroed tile counters (dynamic schedule) or null
  int n_static;           // dynamic schedule: strided tiles per wave before the counters
  int n_groups;           // dynamic schedule: counters per row (<= 16)
  int round_bf16;         // scores rounded to bf16 (ties to even) before they are stored
  Positions qpos;
};

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
  if (a.round_bf16) s = round_bf16(s);
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
template <int HT, int KS, int QPW, int RW, bool DYN, int KF>
__global__ void __launch_bounds__(256) score_bf16_kernel(ScoreArgs a) {
  constexpr int kRowsPerBlock = RW * QPW;
  constexpr int KW = 4 / RW;
  constexpr int dI = KS * 16;
  constexpr int HI = HT * 32;
  constexpr int CH = dI / 8;                 // 16-byte chunks per key row
  constexpr int ROWB = dI * 2;               // bytes per key row
  constexpr int TILEB = 32 * ROWB;           // bytes per 32-key tile
  // Keys in HBM: bf16 rows (2 d_I bytes) or E4M3 rows (d_I bytes).  With
  // bf16 queries (kMixed) E4M3 keys are widened to the bf16 layout in LDS;
  // with E4M3 queries (kE4M3) they stay E4M3 in LDS (f8_swz) and feed the
  // FP8 MFMA.
  constexpr bool F8 = KF == kE4M3;
  // MXFP4 keys (kMXFP4): rows of d_I/2 bytes of E2M1 codes and d_I/32 scale
  // bytes; a tile is copied as bytes to a per-wave LDS area and widened from
  // there to the bf16 layout.
  constexpr bool FP4 = KF == kMXFP4;
  // MXFP4 keys against E4M3 queries (kMX4E4): no LDS at all.  Each lane loads
  // its MFMA operands straight from the key rows: the 16 code bytes of the
  // 32-dim blocks hf and 2 + hf of key ln (one per 64-dim product step) and
  // the row's scale word, and the scaled FP4 product consumes the codes and
  // scales as stored.
  constexpr bool FP4D = KF == kMX4E4;
  static_assert(!FP4D || dI == 128, "direct MXFP4 keys take d_I = 128");
  constexpr int KROWB = FP4 || FP4D ? dI / 2 + dI / 32 : KF == kMixed || F8 ? dI : ROWB;
  constexpr int KTILEB = 32 * KROWB;
  constexpr int NLD = FP4D ? 3 : (KTILEB + 1023) / 1024;   // 16-byte registers per lane per tile
  constexpr int kLPR = dI / 8;               // E4M3: lanes per key (8 codes each)
  constexpr int kRPI = 64 / kLPR;            // E4M3: keys per 8-byte load
  __shared__ float sw[kRowsPerBlock][HI];
  __shared__ __align__(16) uint8_t ktile[4][FP4D ? 16 : F8 ? KTILEB : TILEB];
  __shared__ __align__(16) uint8_t kraw[4][FP4 ? NLD * 1024 : 16];
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

  // The head weights are requested first: loads complete in order, so the
  // LDS store of w below does not wait for the key tiles requested after it.
  constexpr int kWPer = (kRowsPerBlock * HI + 255) / 256;
  float wreg[kWPer];
#pragma unroll
  for (int u = 0; u < kWPer; ++u) {
    const int e = threadIdx.x + 256 * u;
    const int rr = e / HI, h = e - rr * HI;
    const int i = min(i0 + rr, a.Tq - 1);
    wreg[u] = e < kRowsPerBlock * HI ? a.w[((int64_t)b * a.Tq + i) * HI + h] : 0.f;
  }

  // Wave gw of the row's nw key waves takes tiles gw, gw + nw, gw + 2nw, ...:
  // at any moment the waves of a row stream one contiguous stretch of keys,
  // which spreads their loads over all memory channels.
  const int64_t gw = (int64_t)blockIdx.x * KW + wk, nw = (int64_t)gridDim.x * KW;
  const int64_t n_tiles = (nv_max + 31) / 32;
  const int64_t n_mine = gw < n_tiles ? std::min<int64_t>(a.tiles_per_wave, (n_tiles - gw + nw - 1) / nw) : 0;
  // Dynamic schedule: the one-query decode shape with tile counters (two
  // stages per wave); otherwise each wave takes its n_mine strided tiles.
  constexpr bool dynamic = DYN && QPW == 1;
  uint32_t* ctr = dynamic ? a.tile_ctr + ((int64_t)b * a.Tq + i0) * (16 * 32) : nullptr;

  const uint8_t* Kb = static_cast<const uint8_t*>(a.K) + (int64_t)b * a.N * KROWB;
  uint8_t* kt = ktile[wave];
  // Load instruction u of a tile: lane l takes 16 bytes at u*1024 + l*16 of
  // the tile in LDS order, i.e. row kk, swizzled chunk slot cs, which holds
  // the row's chunk cs ^ (kk % CH).  The loads go through a buffer resource
  // based at the tile and bounded by its rows below N, so rows past the end
  // read as zeros and a lane's offsets are the same for every tile.
  auto load_tile = [&](int64_t tile_any, uint4* st) {
    // (the tile is the same in every lane: say so, so that the resource
    // stays in scalar registers)
    const int64_t tile = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(tile_any >> 32)) << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane((int)tile_any));
    const int64_t rows = a.N - tile * 32;
    const int nrec = rows >= 32 ? KTILEB : rows > 0 ? (int)rows * KROWB : 0;
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Kb + tile * KTILEB), 0, nrec,
                                                        0x00020000);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      if constexpr (KF == kMixed) {
        // two 8-byte loads: 8 codes (one bf16 chunk) of key kk8(h) each
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 2 * u + h;
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, (kRPI * j + l / kLPR) * dI + (l % kLPR) * 8, 0, 2);
          if (h == 0) { st[u].x = v[0]; st[u].y = v[1]; } else { st[u].z = v[0]; st[u].w = v[1]; }
        }
      } else if constexpr (FP4D) {
        // u = 0, 1: code bytes of block 2u + hf of key ln; u = 2: its scale word
        if (u < 2) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, ln * KROWB + 16 * (2 * u + hf), 0, 2);
          st[u] = make_uint4(v.x, v.y, v.z, v.w);
        } else {
          st[u].x = __builtin_amdgcn_raw_buffer_load_b32(rsrc, ln * KROWB + dI / 2, 0, 2);
        }
      } else if constexpr (FP4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, u * 1024 + l * 16, 0, 2);
        st[u] = make_uint4(v.x, v.y, v.z, v.w);
      } else if constexpr (F8) {
        const int src = f8_src<dI>(u * 1024 + l * 16);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, src, 0, 2);
        st[u] = make_uint4(v.x, v.y, v.z, v.w);
      } else {
        const int o = u * 1024 + l * 16;
        const int kk = o / ROWB, cs = (o % ROWB) / 16;
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, kk * ROWB + ((cs ^ (kk % CH)) * 16), 0, 2);
        st[u] = make_uint4(v.x, v.y, v.z, v.w);
      }
    }
  };
  uint4 cur[FP4D ? NLD : 1];
  auto store_tile = [&](const uint4* st) {
    if constexpr (FP4D) {
#pragma unroll
      for (int u = 0; u < NLD; ++u) cur[u] = st[u];
      return;
    }
    if constexpr (FP4) {
      // bytes of the tile to the wave's raw area, then lane l widens chunks
      // l, l + 64, ... (key kk = o / CH, 8 dims c = o % CH): 4 code bytes and
      // the scale byte of their 32-dim block, into the swizzled bf16 row
      uint8_t* raw = kraw[wave];
#pragma unroll
      for (int u = 0; u < NLD; ++u) *reinterpret_cast<uint4*>(raw + u * 1024 + l * 16) = st[u];
      __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 32 * CH / 64; ++i) {
        const int o = l + 64 * i, kk = o / CH, c = o % CH;
        const uint8_t* p = raw + kk * KROWB + 4 * c;   // 2-byte aligned (KROWB even)
        const uint32_t codes = (uint32_t)*reinterpret_cast<const uint16_t*>(p) |
                               ((uint32_t)*reinterpret_cast<const uint16_t*>(p + 2) << 16);
        const uint32_t sc = raw[kk * KROWB + dI / 2 + c / 4];
        *reinterpret_cast<uint4*>(kt + kk * ROWB + ((c ^ (kk % CH)) * 16)) = e2m1x8_to_bf16x8(codes, sc);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      if constexpr (KF == kMixed) {
        // 8 E4M3 codes of key kk -> bf16 chunk c of its swizzled LDS row
        // (exact widening); the lanes of one load cover whole rows, so each
        // store instruction writes whole rows of the tile.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kk = kRPI * (2 * u + h) + l / kLPR, c = l % kLPR;
          *reinterpret_cast<uint4*>(kt + kk * ROWB + ((c ^ (kk % CH)) * 16)) =
              h == 0 ? e4m3x8_to_bf16x8(st[u].x, st[u].y) : e4m3x8_to_bf16x8(st[u].z, st[u].w);
        }
      } else {
        *reinterpret_cast<uint4*>(kt + u * 1024 + l * 16) = st[u];
      }
    }
  };

  // The query fragments and the first tiles are requested before anything
  // else, so their latency overlaps the set-up below.  PF tiles are in
  // flight per wave (two for the one-query decode shape, whose registers
  // allow it); the stages alternate.
  constexpr int PF = QPW == 1 ? (FP4D ? kStagesFP4 : F8 ? kStagesF8 : kStagesBF16) : 1;
  uint4 stage[PF][NLD];
  // Query fragments first: lane (ln, hf) holds head ht*32+ln, dims
  // hf*dI/2 + s*8 .. +8.  (They come from L2 for all but the first waves of
  // a row, so the first tile's compute need not wait for the second tile.)
  typedef typename std::conditional<F8 || FP4D, long, bf16x8>::type QFrag;
  QFrag qf[QPW][HT][KS];
  int64_t nv_row[QPW];
  __amdgpu_buffer_rsrc_t srow[QPW];
  {
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
      const int rr = wr * QPW + qi;
      const int i = min(i0 + rr, a.Tq - 1);
      nv_row[qi] = (i0 + rr < a.Tq) ? n_visible((int64_t)a.qpos.v[b] + i, a.N, a.m) : 0;
      srow[qi] = __builtin_amdgcn_make_buffer_rsrc(a.scores + ((int64_t)b * a.Tq + i) * a.Np, 0,
                                                   (int)(nv_row[qi] * 4), 0x00020000);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const int64_t qrow = (((int64_t)b * a.Tq + i) * HI) + ht * 32 + ln;
        if constexpr (FP4D) {
          // step u, fragment r: the query bytes that meet the key dims
          // 64u + 32(r/2) + 16hf + 8(r%2) .. +8 in the scaled FP4 product
          const uint8_t* qp = static_cast<const uint8_t*>(a.q) + qrow * dI;
#pragma unroll
          for (int s = 0; s < KS; ++s)
            qf[qi][ht][s] = *reinterpret_cast<const long*>(
                qp + 64 * (s >> 2) + 32 * ((s >> 1) & 1) + 16 * hf + 8 * (s & 1));
        } else if constexpr (F8) {
          const uint8_t* qp = static_cast<const uint8_t*>(a.q) + qrow * dI + hf * (dI / 2);
#pragma unroll
          for (int s = 0; s < KS; ++s) qf[qi][ht][s] = *reinterpret_cast<const long*>(qp + s * 8);
        } else {
          const __bf16* qp = static_cast<const __bf16*>(a.q) + qrow * dI + hf * (dI / 2);
#pragma unroll
          for (int s = 0; s < KS; ++s) qf[qi][ht][s] = *reinterpret_cast<const bf16x8*>(qp + s * 8);
        }
      }
    }
  }
  // (Unconditional, so that the compiler can count them: a tile past the end
  // reads zeros and is not used.)
#pragma unroll
  for (int f = 0; f < PF; ++f) load_tile(gw + f * nw, stage[f]);

#pragma unroll
  for (int u = 0; u < kWPer; ++u) {
    const int e = threadIdx.x + 256 * u;
    if (e < kRowsPerBlock * HI) sw[e / HI][e % HI] = wreg[u];
  }
  if (do_hist)
    for (int e = threadIdx.x; e < kHistBins; e += 256) lhist[e] = 0u;
  __syncthreads();

  // Work on one tile held in LDS: scores of the wave's query rows.
  auto compute = [&](int64_t tile) {
    QFrag kf[KS];
    if constexpr (F8) {
      // fragments s, s + 1 hold dims hf * d_I / 2 + 8 s .. + 16: one 16-byte read
#pragma unroll
      for (int s = 0; s < KS; s += 2) f8_pair<dI>(kt, ln, hf * (dI / 32) + s / 2, &kf[s]);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (FP4D) {
        kf[s] = 0;                           // unused: the operands are in cur
      } else if constexpr (F8) {
        // read above
      } else {
        const int c = hf * (CH / 2) + s;
        kf[s] = *reinterpret_cast<const bf16x8*>(kt + ln * ROWB + ((c ^ (ln % CH)) * 16));
      }
    }
    const int64_t j = tile * 32 + ln;
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
      const int rr = wr * QPW + qi;
      float part = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x16 acc = {};
        if constexpr (FP4D) {
          // E4M3 queries (unit scales) x MXFP4 keys with their own block
          // scales: step u covers dims 64u .. 64u + 63; this lane's key
          // block is 2u + hf, whose scale is byte 2u + hf of the scale word.
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            i32x8 kb = {};
            kb[0] = (int)cur[u].x; kb[1] = (int)cur[u].y; kb[2] = (int)cur[u].z; kb[3] = (int)cur[u].w;
            acc = mfma_scaled_32x32x64<0, 4>(
                cat4(qf[qi][ht][4 * u], qf[qi][ht][4 * u + 1], qf[qi][ht][4 * u + 2], qf[qi][ht][4 * u + 3]),
                kb, acc, 127, (int)(cur[2].x >> (8 * (2 * u + hf))));
          }
        } else if constexpr (F8) {
          // E4M3 x E4M3 on the 64-deep scaled FP8 product (unit scales):
          // fragments 4u .. 4u+3 of a lane are 32 bytes of its row, in the
          // same order for queries and keys, so every dim meets its partner.
#pragma unroll
          for (int u = 0; u < KS / 4; ++u)
            acc = mfma_scaled_32x32x64<0, 0>(
                cat4(qf[qi][ht][4 * u], qf[qi][ht][4 * u + 1], qf[qi][ht][4 * u + 2], qf[qi][ht][4 * u + 3]),
                cat4(kf[4 * u], kf[4 * u + 1], kf[4 * u + 2], kf[4 * u + 3]), acc, 127, 127);
        } else {
#pragma unroll
          for (int s = 0; s < KS; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[qi][ht][s], kf[s], acc, 0, 0, 0);
        }
        // acc[v] is head ht*32 + 8*(v/4) + 4*hf + v%4 against key j.
#pragma unroll
        for (int v = 0; v < 16; ++v)
          part = fmaf(sw[rr][ht * 32 + 8 * (v >> 2) + 4 * hf + (v & 3)], relu(acc[v]), part);
      }
      part += __shfl_xor(part, 32);
      const float pr = round_bf16(part);
      part = a.round_bf16 ? pr : part;
      const bool live = hf == 0 && j < nv_row[qi];
      // through the row's buffer resource: a lane that is not live stores out
      // of range and its store is dropped, so the store is issued on every path
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(part), srow[qi], live ? (int)j * 4 : 0x7fffffff,
                                            0, 0);
      if (do_hist) hist_add(lhist, live, score_key(part) >> 20);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);      // LDS reads of this tile done
    __builtin_amdgcn_wave_barrier();
  };
  auto stage_in = [&](const uint4* st) {
    store_tile(st);
    __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): LDS writes done
    __builtin_amdgcn_wave_barrier();
  };

  if constexpr (dynamic) {
    // The first n_static tiles of a wave are its strided ones; the rest of
    // the row's tiles are handed out by counters, so that waves that stream
    // faster take more of them and all finish together.  Each of the row's
    // n_groups counters (one per group of eight consecutive blocks, which
    // spans every XCD) serves the tiles n_static * nw + c * n_groups + g:
    // a device-scope atomic on one address costs tens of nanoseconds, so
    // the load is spread over several addresses and only the tail of the
    // sweep is dynamic.  Stage f holds tile t[f] (the wave's sequence
    // number k + f); its ticket r[f], drawn by lane 0 when stage f was last
    // refilled, names the tile that refills it next, PF tiles later, so the
    // atomic's latency is hidden like a load's.
    const int g = (int)((blockIdx.x >> 3) % (unsigned)a.n_groups);
    uint32_t* gctr = ctr + 32 * g;
    const int64_t ns = a.n_static, dyn0 = ns * nw;
    auto tile_of = [&](int64_t k, uint32_t ticket) {
      return k < ns ? gw + k * nw : dyn0 + (int64_t)ticket * a.n_groups + g;
    };
    int64_t t[PF];
    uint32_t r[PF];
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      t[f] = gw + f * nw;
      r[f] = 0u;
      if (l == 0 && t[f] < n_tiles && f + PF >= ns) r[f] = atomicAdd(gctr, 1u);
    }
    int64_t k = 0;                 // sequence number of the tile in stage 0
    for (;; k += PF) {
#pragma unroll
      for (int f = 0; f < PF; ++f) {
        if (t[f] >= n_tiles) goto done;
        stage_in(stage[f]);
        const int64_t kn = k + f + PF;
        const int64_t nt = tile_of(kn, kn >= ns ? __builtin_amdgcn_readfirstlane(r[f]) : 0u);
        if (nt < n_tiles) {
          load_tile(nt, stage[f]);
          if (l == 0 && kn + PF >= ns) r[f] = atomicAdd(gctr, 1u);
        }
        compute(t[f]);
        t[f] = nt;
      }
    }
  done:;
  } else if (n_mine > 0) {
    // Whole rounds of PF tiles first.  Every load and store in them is issued
    // on every path (a refill past the wave's share loads a tile with no rows,
    // which reads nothing), so the compiler's memory-counter waits are exact
    // and only the oldest stage is waited for: a refill issued under a branch
    // would make it wait for every load in flight at each stage.
    const int64_t none = (a.N + 31) / 32;      // a tile with no rows
    int64_t it = 0;
    for (; it + PF <= n_mine; it += PF) {
#pragma unroll
      for (int f = 0; f < PF; ++f) {
        const int64_t k = it + f;
        stage_in(stage[f]);
        load_tile(k + PF < n_mine ? gw + (k + PF) * nw : none, stage[f]);
        compute(gw + k * nw);
      }
    }
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      if (it + f < n_mine) {
        stage_in(stage[f]);
        compute(gw + (it + f) * nw);
      }
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

// Prefill score kernel.  A block of eight waves holds 8 * QPW consecutive
// queries of one sequence (QPW per wave, fragments in VGPRs) and sweeps all
// keys the block can see, one 32-key tile at a time: the 512 threads load a
// tile cooperatively (one 16-byte load each, XOR-swizzled into LDS, two
// tiles ahead in registers) and every wave reads it from LDS, so each key
// tile crosses HBM once per 8 * QPW queries and all waves of a compute unit
// share it.
template <int HT, int KS, int QPW, int KF>
__global__ void __launch_bounds__(512) score_prefill_kernel(ScoreArgs a) {
  constexpr int QB = 8 * QPW;                // queries per block
  constexpr int dI = KS * 16;
  constexpr int HI = HT * 32;
  constexpr int CH = dI / 8;                 // 16-byte chunks per key row
  constexpr int ROWB = dI * 2;               // bytes per key row
  constexpr int TILEB = 32 * ROWB;           // bytes per 32-key tile
  // Keys in HBM: bf16 rows or E4M3 rows (widened to bf16 in LDS for bf16
  // queries, kept E4M3 in LDS for E4M3 queries).
  constexpr bool F8 = KF == kE4M3;
  // MXFP4 keys against E4M3 queries (kMX4E4, d_I = 128): a tile is 32 rows
  // of 64 code bytes and a 4-byte scale word; every thread loads one of its
  // 544 words (the first 32 threads a second) and puts it in LDS as 32 rows
  // of 64 code bytes followed by the 32 scale words, so that the operand
  // reads are aligned 16-byte reads.
  constexpr bool FP4D = KF == kMX4E4;
  static_assert(!FP4D || dI == 128, "MXFP4 keys against E4M3 queries take d_I = 128");
  constexpr int KROWB = FP4D ? dI / 2 + dI / 32 : KF == kMixed || F8 ? dI : ROWB;
  constexpr int LBYTES = FP4D ? 4 : KF == kMixed ? 8 : 16;    // bytes each loader reads
  constexpr int LOADERS = FP4D ? 512 : 32 * KROWB / LBYTES;
  constexpr int FP4W = 32 * KROWB / 4;       // words per MXFP4 tile (544)
  __shared__ float sw[QB][HI];
  __shared__ __align__(16) uint8_t ktile[2][FP4D ? 32 * KROWB : F8 ? 32 * dI : TILEB];
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int hf = l >> 5, ln = l & 31;
  const int blocks_per_seq = (a.Tq + QB - 1) / QB;
  const int b = blockIdx.x / blocks_per_seq;
  const int i0 = (blockIdx.x - b * blocks_per_seq) * QB;
  const int n_rows_blk = min(QB, a.Tq - i0);
  const int64_t t_last = (int64_t)a.qpos.v[b] + i0 + n_rows_blk - 1;
  const int64_t nv_max = n_visible(t_last, a.N, a.m);
  const int64_t n_tiles = (nv_max + 31) / 32;

  // Head weights first (loads complete in order; see the decode kernel).
  constexpr int kWPer = (QB * HI + 511) / 512;
  float wreg[kWPer];
#pragma unroll
  for (int u = 0; u < kWPer; ++u) {
    const int e = threadIdx.x + 512 * u;
    const int rr = e / HI, h = e - rr * HI;
    const int i = min(i0 + rr, a.Tq - 1);
    wreg[u] = e < QB * HI ? a.w[((int64_t)b * a.Tq + i) * HI + h] : 0.f;
  }

  const uint8_t* Kb = static_cast<const uint8_t*>(a.K) + (int64_t)b * a.N * KROWB;
  // bf16: loader thread t takes 16 bytes at t*16 of the tile in LDS order:
  // row kk, swizzled slot cs, which holds the row's chunk cs ^ (kk % CH).
  // E4M3 widened: loader t takes the 8 codes of chunk cs of key kk (t*8 of
  // the tile in HBM order) and writes them widened into that chunk's slot, so
  // the loaders of one key fill its whole LDS row.  E4M3 kept: loader t fills
  // the 16 bytes at t*16 of the swizzled tile (f8_src).
  const bool loader = (int)threadIdx.x < LOADERS;
  const int lo_off = threadIdx.x * LBYTES;
  const int lo_kk = lo_off / KROWB, lo_cs = (lo_off % KROWB) / LBYTES;
  const int lo_src8 = F8 ? f8_src<dI>(lo_off) % dI : 0;   // byte in its row
  auto load_tile = [&](int64_t tile) {
    if constexpr (FP4D) {
      // words t and 512 + t of the tile (rows past N read row N - 1)
      uint4 r = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int wd = (int)threadIdx.x + 512 * h;
        if (wd < FP4W) {
          int64_t j = tile * 32 + wd / 17;
          if (j > a.N - 1) j = a.N - 1;
          const uint32_t v = *reinterpret_cast<const uint32_t*>(Kb + j * KROWB + 4 * (wd % 17));
          if (h == 0) r.x = v; else r.y = v;
        }
      }
      return r;
    }
    int64_t j = tile * 32 + lo_kk;
    if (j > a.N - 1) j = a.N - 1;
    if constexpr (KF == kMixed) {
      const uint2 v = ld_stream8(Kb + j * KROWB + lo_cs * 8);
      return make_uint4(v.x, v.y, 0u, 0u);
    } else if constexpr (F8) {
      return ld_stream16(Kb + j * dI + lo_src8);
    } else {
      return ld_stream16(Kb + j * ROWB + ((lo_cs ^ (lo_kk % CH)) * 16));
    }
  };
  auto put_tile = [&](uint8_t* kt, const uint4& st) {
    if constexpr (FP4D) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int wd = (int)threadIdx.x + 512 * h;
        if (wd < FP4W) {
          const int kk = wd / 17, c = wd % 17;
          *reinterpret_cast<uint32_t*>(kt + (c < 16 ? kk * 64 + 4 * c : 32 * 64 + 4 * kk)) =
              h == 0 ? st.x : st.y;
        }
      }
      return;
    }
    if constexpr (KF == kMixed)
      *reinterpret_cast<uint4*>(kt + lo_kk * ROWB + ((lo_cs ^ (lo_kk % CH)) * 16)) =
          e4m3x8_to_bf16x8(st.x, st.y);
    else
      *reinterpret_cast<uint4*>(kt + lo_off) = st;
  };
  uint4 stage[2];
  if (loader) {
    if (n_tiles > 0) stage[0] = load_tile(0);
    if (n_tiles > 1) stage[1] = load_tile(1);
  }

  // Query fragments: lane (ln, hf) holds head ht*32+ln, dims hf*dI/2 + s*8 .. +8.
  // Scores are written through a buffer resource per query row: a masked
  // lane (hidden key, second half-wave, row past Tq) stores out of range and
  // the store is dropped, so every store instruction is issued unconditionally
  // and the memory counter stays exact for the prefetch waits.
  typedef typename std::conditional<F8 || FP4D, long, bf16x8>::type QFrag;
  QFrag qf[QPW][HT][KS];
  int64_t nv_row[QPW];
  __amdgpu_buffer_rsrc_t srow[QPW];
#pragma unroll
  for (int qi = 0; qi < QPW; ++qi) {
    const int rr = wave * QPW + qi;
    const int i = min(i0 + rr, a.Tq - 1);
    nv_row[qi] = (i0 + rr < a.Tq) ? n_visible((int64_t)a.qpos.v[b] + i, a.N, a.m) : 0;
    srow[qi] = __builtin_amdgcn_make_buffer_rsrc(a.scores + ((int64_t)b * a.Tq + i) * a.Np, 0,
                                                 (int)(nv_row[qi] * 4), 0x00020000);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int64_t qrow = (((int64_t)b * a.Tq + i) * HI) + ht * 32 + ln;
      if constexpr (FP4D) {
        // step u, fragment r: the query bytes that meet the key dims
        // 64u + 32(r/2) + 16hf + 8(r%2) .. +8 in the scaled FP4 product
        const uint8_t* qp = static_cast<const uint8_t*>(a.q) + qrow * dI;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          qf[qi][ht][s] = *reinterpret_cast<const long*>(
              qp + 64 * (s >> 2) + 32 * ((s >> 1) & 1) + 16 * hf + 8 * (s & 1));
      } else if constexpr (F8) {
        const uint8_t* qp = static_cast<const uint8_t*>(a.q) + qrow * dI + hf * (dI / 2);
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[qi][ht][s] = *reinterpret_cast<const long*>(qp + s * 8);
      } else {
        const __bf16* qp = static_cast<const __bf16*>(a.q) + qrow * dI + hf * (dI / 2);
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[qi][ht][s] = *reinterpret_cast<const bf16x8*>(qp + s * 8);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kWPer; ++u) {
    const int e = threadIdx.x + 512 * u;
    if (e < QB * HI) sw[e / HI][e % HI] = wreg[u];
  }

  // One step per tile; the loop is unrolled by two so that the staging
  // registers and LDS buffers are indexed statically (a runtime index would
  // force the prefetch to complete when it is issued).
  auto step = [&](int64_t tile, uint4& st, uint8_t* kt) {
    if (loader) {
      put_tile(kt, st);
      if (tile + 2 < n_tiles) st = load_tile(tile + 2);
    }
    __syncthreads();             // tile visible; every wave is done with tile - 1
    QFrag kf[KS];
    // MXFP4: this lane's code blocks 2u + hf of key ln, and its scale word
    uint4 kc[2];
    uint32_t ksc = 0;
    if constexpr (FP4D) {
#pragma unroll
      for (int u = 0; u < 2; ++u) kc[u] = *reinterpret_cast<const uint4*>(kt + ln * 64 + 16 * (2 * u + hf));
      ksc = *reinterpret_cast<const uint32_t*>(kt + 32 * 64 + 4 * ln);
    }
    if constexpr (F8) {
      // fragments s, s + 1 hold dims hf * d_I / 2 + 8 s .. + 16: one 16-byte read
#pragma unroll
      for (int s = 0; s < KS; s += 2) f8_pair<dI>(kt, ln, hf * (dI / 32) + s / 2, &kf[s]);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (FP4D) {
        kf[s] = 0;                           // unused: the operands are in kc
      } else if constexpr (F8) {
        // read above
      } else {
        const int c = hf * (CH / 2) + s;
        kf[s] = *reinterpret_cast<const bf16x8*>(kt + ln * ROWB + ((c ^ (ln % CH)) * 16));
      }
    }
    const int64_t j = tile * 32 + ln;
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
      const int rr = wave * QPW + qi;
      float part = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x16 acc = {};
        if constexpr (FP4D) {
          // E4M3 queries (unit scales) x MXFP4 keys with their block scales,
          // as in the decode kernel
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            i32x8 kb = {};
            kb[0] = (int)kc[u].x; kb[1] = (int)kc[u].y; kb[2] = (int)kc[u].z; kb[3] = (int)kc[u].w;
            acc = mfma_scaled_32x32x64<0, 4>(
                cat4(qf[qi][ht][4 * u], qf[qi][ht][4 * u + 1], qf[qi][ht][4 * u + 2], qf[qi][ht][4 * u + 3]),
                kb, acc, 127, (int)(ksc >> (8 * (2 * u + hf))));
          }
        } else if constexpr (F8) {
          // E4M3 x E4M3 on the 64-deep scaled FP8 product (unit scales):
          // fragments 4u .. 4u+3 of a lane are 32 bytes of its row, in the
          // same order for queries and keys, so every dim meets its partner.
#pragma unroll
          for (int u = 0; u < KS / 4; ++u)
            acc = mfma_scaled_32x32x64<0, 0>(
                cat4(qf[qi][ht][4 * u], qf[qi][ht][4 * u + 1], qf[qi][ht][4 * u + 2], qf[qi][ht][4 * u + 3]),
                cat4(kf[4 * u], kf[4 * u + 1], kf[4 * u + 2], kf[4 * u + 3]), acc, 127, 127);
        } else {
#pragma unroll
          for (int s = 0; s < KS; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[qi][ht][s], kf[s], acc, 0, 0, 0);
        }
        // acc[v] is head ht*32 + 8*(v/4) + 4*hf + v%4 against key j.
#pragma unroll
        for (int v = 0; v < 16; ++v)
          part = fmaf(sw[rr][ht * 32 + 8 * (v >> 2) + 4 * hf + (v & 3)], relu(acc[v]), part);
      }
      part += __shfl_xor(part, 32);
      const float pr = round_bf16(part);
      part = a.round_bf16 ? pr : part;
      const int off = hf == 0 ? (int)j * 4 : 0x7fffffff;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(part), srow[qi], off, 0, 2);   // nt
    }
  };
  for (int64_t tile = 0; tile < n_tiles; tile += 2) {
    step(tile, stage[0], ktile[0]);
    if (tile + 1 < n_tiles) step(tile + 1, stage[1], ktile[1]);
  }
}

template <int HT, int KS, int QPW, int RW, int KF>
hipError_t launch_score(const ScoreArgs& sa, int64_t key_chunks, int row_groups, hipStream_t st) {
  if (sa.tile_ctr != nullptr)
    hipLaunchKernelGGL((score_bf16_kernel<HT, KS, QPW, RW, true, KF>),
                       dim3((unsigned)key_chunks, row_groups), dim3(256), 0, st, sa);
  else
    hipLaunchKernelGGL((score_bf16_kernel<HT, KS, QPW, RW, false, KF>),
                       dim3((unsigned)key_chunks, row_groups), dim3(256), 0, st, sa);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerArgs& a, const ScoreBuffers& sb, int64_t nv_max,
                                 hipStream_t st) {
  const int R = a.B * a.Tq;
  if (R == 0 || nv_max <= 0) return hipSuccess;
  hipError_t err = hipSuccess;
  ScoreArgs sa{};
  sa.q = a.q; sa.w = a.w; sa.K = a.K; sa.scores = sb.scores;
  sa.B = a.B; sa.Tq = a.Tq; sa.HI = a.HI; sa.dI = a.dI; sa.N = a.N; sa.m = a.m;
  sa.Np = sb.Np; sa.qpos = a.qpos; sa.hist = sb.hist;
  sa.tile_ctr = sb.tile_ctr;
  sa.round_bf16 = a.round_bf16;
  {
    TimedLaunch tl(kKernelIndexerScore, st);
    if (a.fmt == kF32) {
      const size_t lds = (size_t)(a.HI * a.dI + a.HI) * 4;
      hipLaunchKernelGGL(score_f32_kernel, dim3((unsigned)((nv_max + 255) / 256), R), dim3(256),
                         lds, st, sa);
      err = hipGetLastError();
    } else {
      const int64_t n_tiles = (nv_max + 31) / 32;
      const int HT = a.HI / 32, KS = a.dI / 16;
      // kBF16: bf16 queries and keys; kMixed: bf16 queries, E4M3 keys;
      // kE4M3: E4M3 queries and keys (FP8 MFMA); kMXFP4: bf16 queries, MXFP4
      // keys (the decode kernel for every shape); kMX4E4: E4M3 queries, MXFP4
      // keys (scaled FP4 MFMA)
      const int kf = a.fmt;
      if (a.Tq >= 8 && !sb.split && kf == kMX4E4 && KS == 8) {
        // MXFP4 keys against E4M3 queries: d_I = 128 (the ABI refuses others)
        // one query per wave (HT > 1): 109 VGPRs, two blocks per compute unit
        const int qpw = HT == 1 ? 2 : 1;
        const int blocks = a.B * ((a.Tq + 8 * qpw - 1) / (8 * qpw));
        if (HT == 1)
          hipLaunchKernelGGL((score_prefill_kernel<1, 8, 2, kMX4E4>), dim3(blocks), dim3(512), 0, st, sa);
        else if (HT == 2)
          hipLaunchKernelGGL((score_prefill_kernel<2, 8, 1, kMX4E4>), dim3(blocks), dim3(512), 0, st, sa);
        else
          hipLaunchKernelGGL((score_prefill_kernel<4, 8, 1, kMX4E4>), dim3(blocks), dim3(512), 0, st, sa);
        err = hipGetLastError();
      } else if (a.Tq >= 8 && !sb.split && kf == kE4M3 && HT == 2 && KS == 8) {
        // E4M3 queries and keys, 64 heads x 128: one query per wave as well
        // (low register use, two blocks per compute unit)
        const int blocks = a.B * ((a.Tq + 7) / 8);
        hipLaunchKernelGGL((score_prefill_kernel<2, 8, 1, kE4M3>), dim3(blocks), dim3(512), 0, st, sa);
        err = hipGetLastError();
      } else if (a.Tq >= 8 && !sb.split && kf != kMXFP4 && kf != kMX4E4) {
        // Prefill: a block of eight waves shares each key tile among 8 * QPW
        // queries and sweeps all the keys they see.
#define LAC_SCORE_CASE(ht, ks, qpw)                                                        \
  if (HT == ht && KS == ks) {                                                              \
    const int blocks = a.B * ((a.Tq + 8 * qpw - 1) / (8 * qpw));                           \
    if (kf == kE4M3)                                                                       \
      hipLaunchKernelGGL((score_prefill_kernel<ht, ks, qpw, kE4M3>), dim3(blocks), dim3(512), 0, st, sa); \
    else if (kf == kMixed)                                                                 \
      hipLaunchKernelGGL((score_prefill_kernel<ht, ks, qpw, kMixed>), dim3(blocks), dim3(512), 0, st, sa); \
    else                                                                                   \
      hipLaunchKernelGGL((score_prefill_kernel<ht, ks, qpw, kBF16>), dim3(blocks), dim3(512), 0, st, sa); \
    err = hipGetLastError();                                                               \
  }
        LAC_SCORE_CASE(1, 4, 2) LAC_SCORE_CASE(1, 8, 2) LAC_SCORE_CASE(2, 4, 2)
        LAC_SCORE_CASE(2, 8, 2) LAC_SCORE_CASE(4, 4, 2) LAC_SCORE_CASE(4, 8, 1)
#undef LAC_SCORE_CASE
      } else {
        // Decode: one query per block, 4 waves split the keys.  The grid is
        // one round of the 512 resident blocks (two blocks of 4 waves per
        // compute unit at this kernel's register use), so no partial second
        // round trails the sweep.
        const int64_t per_row = std::max<int64_t>(
            1, (kf == kE4M3 ? kDecodeBlocksF8 : kf == kMX4E4 ? kDecodeBlocksFP4 : kDecodeBlocksBF16) / R);
        sa.tiles_per_wave = (int)std::max<int64_t>(2, (n_tiles + 4 * per_row - 1) / (4 * per_row));
        const int64_t chunks = (n_tiles + 4 * sa.tiles_per_wave - 1) / (4 * sa.tiles_per_wave);
        // dynamic schedule: about the last quarter of the sweep
        sa.n_static = std::max(2, sa.tiles_per_wave * 3 / 4);
        sa.n_groups = (int)std::min<int64_t>(16, std::max<int64_t>(1, chunks / 8));
        // E4M3 and MXFP4 keys: the sweep is bound by each tile's MFMA and
        // ReLU-weighting work rather than by HBM, so every wave takes its
        // strided share (its rounds of tiles keep exact prefetch waits); the
        // counters only pay for bf16 keys, whose waves stream at different rates.
        if (kf == kE4M3 || kf == kMX4E4) sa.tile_ctr = nullptr;
        const int groups = a.B * a.Tq;
#define LAC_SCORE_CASE(ht, ks)                                                      \
  if (HT == ht && KS == ks)                                                         \
    err = kf == kE4M3    ? launch_score<ht, ks, 1, 1, kE4M3>(sa, chunks, groups, st)  \
          : kf == kMixed ? launch_score<ht, ks, 1, 1, kMixed>(sa, chunks, groups, st) \
          : kf == kMXFP4 ? launch_score<ht, ks, 1, 1, kMXFP4>(sa, chunks, groups, st) \
                         : launch_score<ht, ks, 1, 1, kBF16>(sa, chunks, groups, st);
        if (kf == kMX4E4) {
          // d_I = 128 only (the ABI refuses other widths for this format)
          if (KS == 8)
            err = HT == 1   ? launch_score<1, 8, 1, 1, kMX4E4>(sa, chunks, groups, st)
                  : HT == 2 ? launch_score<2, 8, 1, 1, kMX4E4>(sa, chunks, groups, st)
                            : launch_score<4, 8, 1, 1, kMX4E4>(sa, chunks, groups, st);
        } else {
        LAC_SCORE_CASE(1, 4) LAC_SCORE_CASE(1, 8) LAC_SCORE_CASE(2, 4) LAC_SCORE_CASE(2, 8)
        LAC_SCORE_CASE(4, 4) LAC_SCORE_CASE(4, 8)
        }
#undef LAC_SCORE_CASE
      }
    }
    if (err != hipSuccess) return err;
  }

  return hipSuccess;
}

}  // namespace lac
