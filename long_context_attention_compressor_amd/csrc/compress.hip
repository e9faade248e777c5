// compress.hip -- block-softmax KV compression (CSA m = 4, HCA m' = 128).
//
// "深度解析 DeepSeek-V4" (learnblockchain.cn), section "CSA：Compressed Sparse
// Attention", Step 1 Compress: every m consecutive KV entries merge into one
// entry with learned softmax weights; section "HCA：Heavily Compressed
// Attention": the same with m' = 128.  Per channel c of entry j:
//   out[j, c] = sum_i softmax_i(logits[j*m + i, c]) * kv[j*m + i, c],
// then the last r dims are rotated at the block start j*m (partial RoPE of the
// QbitAI rewrite).
//
// The kernel is a pure HBM stream: each thread owns 8 consecutive channels
// (one 16-byte bf16 load per token row, coalesced across the row) of one
// entry and walks its share of the block's tokens with an online softmax
// (running max, denominator and weighted sum in fp32), with up to eight
// tokens' loads in flight before any is used.  When a block has many tokens
// (HCA), S threads split the tokens and merge their partial states through
// LDS in a log2(S)-level tree, so short sequences still spread over many
// lanes.  The rotation table is built while the first loads are in flight.
//
// Optional RMSNorm of each entry before its rotation ("深度解析 DeepSeek-V4",
// section "Attention Sink": RMSNorm of the queries and compressed KV entries
// before core attention): the block then holds all channel groups of an
// entry, whose GB threads are consecutive lanes of one wave, and the entry's
// sum of squares is reduced across them with lane shuffles.
#include <algorithm>
#include <type_traits>

#include "lac_internal.h"

namespace lac {

namespace {

// Raw 8-channel slice of one token row: bf16 in one 16-byte word, f32 in two.
template <int IN>
struct Raw8 {
  uint4 w[IN == kF32 ? 2 : 1];
};

template <int IN>
__device__ __forceinline__ Raw8<IN> load_raw8(const void* base, int64_t elem) {
  Raw8<IN> r;
  if constexpr (IN == kF32) {
    const float* p = static_cast<const float*>(base) + elem;
    r.w[0] = ld_stream16(p);
    r.w[1] = ld_stream16(p + 4);
  } else {
    r.w[0] = ld_stream16(static_cast<const uint16_t*>(base) + elem);
  }
  return r;
}

template <int IN>
__device__ __forceinline__ void unpack8(const Raw8<IN>& r, float* v) {
  if constexpr (IN == kF32) {
    const uint32_t w[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w, r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  } else {
    const uint32_t w[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
}

template <int IN>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float* v) {
  if constexpr (IN == kF32) {
    const float* p = static_cast<const float*>(base) + elem;
    const uint4 a = ld_stream16(p), b = ld_stream16(p + 4);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  } else {
    const uint4 a = ld_stream16(static_cast<const uint16_t*>(base) + elem);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
}

template <int IN>
__device__ __forceinline__ void softmax_step(const float* xv, const float* zv, float* mx, float* den,
                                             float* acc) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float nm = fmaxf(mx[c], zv[c]);
    const float sc = __expf(mx[c] - nm);          // 0 on the first token
    const float p = __expf(zv[c] - nm);
    den[c] = den[c] * sc + p;
    acc[c] = acc[c] * sc + p * xv[c];
    mx[c] = nm;
  }
}

// One call as the kernel reads it.  A launch carries up to kCompressGroup
// independent calls (CLaunch): its workgroups are the calls' workgroups one
// after another, and a call's positions and rotation table sit in the
// launch's pools, so that the whole launch fits one kernel argument.
struct CompressK {
  const void* kv;
  const void* logits;
  void* out;
  const float* norm_gain;   // [D] or null: RMSNorm of each entry before its rotation
  int64_t kv_bstride, z_bstride, out_bstride;   // rows
  int out_fmt, D, m, r, overlap, N;
  int per, gb, s, epb, tokn;   // tokens per thread; block (gb, s, epb); loads in flight
  int gx, gy;                  // workgroups per sequence: entry groups x channel slices
  uint32_t mul_gb, mul_gbs;    // t / gb and t / (gb * s) for t < 512: (t * mul) >> 20
  int pos_off, freq_off;       // pos0 and the rotation table in the pools
  float norm_eps;
};

constexpr int kCompressGroup = 4;
constexpr int kCompressPos = 384;
constexpr int kCompressTables = 2;

struct CLaunch {
  CompressK c[kCompressGroup];
  uint32_t blk_end[kCompressGroup];   // workgroups of calls 0 .. i
  int n;
  // clearing jobs after the calls' workgroups: job i zeroes clr_words[i]
  // words at clr[i] with the workgroups up to clr_end[i] (cumulative, after
  // the calls'); blk_total = all workgroups of the launch
  int n_clr;
  uint32_t* clr[kCompressGroup];
  uint64_t clr_words[kCompressGroup];
  uint32_t clr_end[kCompressGroup];
  uint32_t blk_total;
  int32_t pos[kCompressPos];
  double freq[kCompressTables * kMaxRopePairs];
};

// A launch's whole argument is one kernel argument: keep it within 4 KB.
static_assert(sizeof(CLaunch) <= 4096, "kernel argument above 4 KB");

// Thread (x, y, z) of a call's block (GB, S, epb) owns channel group
// slice * GB + x of entry group * epb + z and token share y of its block; a
// call's workgroups run (entry groups, channel slices, sequences), fastest
// first.  A single call launches exactly that grid and block (MULTI false:
// its arguments sit at fixed offsets and its indices come straight from the
// hardware).  A launch of several calls (MULTI true) has a flat grid of their
// workgroups one call after another and a flat block as large as its largest
// call's; the extra threads of a smaller call only take part in the barriers.
// OUT: the output format of a single call, or -1 (MULTI: each call's own).
template <int IN, int TOKN, int OUT>
__global__ void __launch_bounds__(512) compress_kernel(CLaunch L) {
  constexpr bool MULTI = OUT < 0;
  extern __shared__ float part[];                  // [threads][25] when S > 1
  __shared__ double freq[kMaxRopePairs];
  int ci = 0;
  uint32_t lb = 0;
  if constexpr (MULTI) {
    const uint32_t wg = blockIdx.y * gridDim.x + blockIdx.x;
    if (wg >= L.blk_total) return;            // the grid's rounding
    const uint32_t calls_end = L.n ? L.blk_end[L.n - 1] : 0u;
    if (wg >= calls_end) {
      // a clearing workgroup: 16 bytes per thread of its job's words
      int q = 0;
      while (q + 1 < L.n_clr && wg >= L.clr_end[q]) ++q;
      const uint32_t first = q ? L.clr_end[q - 1] : calls_end;
      const uint64_t v = ((uint64_t)(wg - first) * blockDim.x + threadIdx.x) * 4;
      if (v < L.clr_words[q]) *reinterpret_cast<uint4*>(L.clr[q] + v) = make_uint4(0u, 0u, 0u, 0u);
      return;
    }
    while (ci + 1 < L.n && wg >= L.blk_end[ci]) ++ci;
    lb = wg - (ci ? L.blk_end[ci - 1] : 0u);
  }
  const CompressK& a = L.c[ci];
  const int GB = a.gb, S = a.s;
  int t, tx, s, tz, eg, slice, b, nthr;
  if constexpr (MULTI) {
    // (x, y, z) of thread t: exact reciprocal multiplies (t < 512, divisors <= 512)
    t = threadIdx.x;
    const int ty_all = (int)(((uint32_t)t * a.mul_gb) >> 20);
    tz = (int)(((uint32_t)t * a.mul_gbs) >> 20);
    tx = t - ty_all * GB;
    s = ty_all - tz * S;
    eg = (int)(lb % (uint32_t)a.gx);
    slice = (int)((lb / (uint32_t)a.gx) % (uint32_t)a.gy);
    b = (int)(lb / ((uint32_t)a.gx * (uint32_t)a.gy));
    nthr = blockDim.x;
  } else {
    tx = threadIdx.x; s = threadIdx.y; tz = threadIdx.z;
    t = (tz * S + s) * GB + tx;
    eg = blockIdx.x; slice = blockIdx.y; b = blockIdx.z;
    nthr = GB * S * a.epb;
  }
  const int g = slice * GB + tx;
  const int j = eg * a.epb + tz;
  const bool act = tz < a.epb;
  const bool live = act && j < a.N;
  // a single call's positions and table sit at the start of the pools
  const double* tab = L.freq + (MULTI ? a.freq_off : 0);
  const int64_t pos0 = L.pos[(MULTI ? a.pos_off : 0) + b];
  auto fill_freq = [&]() {
    for (int i = t; i < a.r / 2; i += nthr) freq[i] = tab[i];
  };

  float mx[8], den[8], acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) { mx[c] = -INFINITY; den[c] = 0.f; acc[c] = 0.f; }
  // the gains of this thread's 8 channels, requested first
  float4 gain0 = make_float4(1.f, 1.f, 1.f, 1.f), gain1 = gain0;
  if (a.norm_gain && act) {
    gain0 = *reinterpret_cast<const float4*>(a.norm_gain + g * 8);
    gain1 = *reinterpret_cast<const float4*>(a.norm_gain + g * 8 + 4);
  }

  if (live) {
    // The entry's window: with an overlap o, positions [max(0, p_j - o),
    // p_j + m) of the rows that start min(o, pos0) before the first block;
    // this thread takes tokens s * per .. of it.
    const int per = a.per;
    const int64_t pj = pos0 + (int64_t)j * a.m;
    const int64_t lead = min((int64_t)a.overlap, pos0);
    const int64_t back = min((int64_t)a.overlap, pj);
    const int cnt = a.m + (int)back;                       // window tokens
    const int mine = max(0, min(per, cnt - s * per));      // this thread's tokens
    const int64_t row0 = lead + (int64_t)j * a.m - back + (int64_t)s * per;
    const int64_t xb = (b * a.kv_bstride + row0) * a.D + g * 8;
    const int64_t zb = (b * a.z_bstride + row0) * a.D + g * 8;
    // TOK tokens' loads in flight before any of them is used, kept packed
    // until used (rows past the thread's share re-read its last row and are
    // not used); TOKN = 4 when every call's share is at most 4 tokens (the
    // launch's calls share TOKN, which sets the kernel's registers).
    {
      constexpr int TOK = IN == kF32 ? (TOKN < 4 ? TOKN : 4) : TOKN;
      for (int i = 0; i < mine; i += TOK) {
        Raw8<IN> xr[TOK], zr[TOK];
#pragma unroll
        for (int u = 0; u < TOK; ++u) {
          const int64_t row = min(i + u, mine - 1);
          xr[u] = load_raw8<IN>(a.kv, xb + row * a.D);
          zr[u] = load_raw8<IN>(a.logits, zb + row * a.D);
        }
        if (i == 0) fill_freq();
#pragma unroll
        for (int u = 0; u < TOK; ++u) {
          if (i + u < mine) {
            float xv[8], zv[8];
            unpack8<IN>(xr[u], xv);
            unpack8<IN>(zr[u], zv);
            softmax_step<IN>(xv, zv, mx, den, acc);
          }
        }
      }
    }
    if (mine == 0) fill_freq();
  } else {
    fill_freq();
  }
  __syncthreads();                   // rotation table complete

  if (S > 1) {
    // Tree merge: at level o, thread s < o absorbs thread s + o.
    float* mine = part + t * 25;
    for (int o = S >> 1; o >= 1; o >>= 1) {
      if (act && s < 2 * o) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          mine[c] = mx[c];
          mine[8 + c] = den[c];
          mine[16 + c] = acc[c];
        }
      }
      __syncthreads();
      if (act && s < o) {
        const float* other = part + (t + o * GB) * 25;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float om = other[c];
          const float nm = fmaxf(mx[c], om);
          const float s0 = nm == -INFINITY ? 0.f : __expf(mx[c] - nm);
          const float s1 = nm == -INFINITY ? 0.f : __expf(om - nm);
          den[c] = den[c] * s0 + other[8 + c] * s1;
          acc[c] = acc[c] * s0 + other[16 + c] * s1;
          mx[c] = nm;
        }
      }
      __syncthreads();
    }
    if (s != 0) return;
  }
  if (!live) return;

  float o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = acc[c] / den[c];
  if (a.norm_gain) {
    // RMSNorm over the entry's D channels: its GB (a power of two, at most
    // 64) threads are lanes t .. t + GB - 1 of one wave, aligned to GB.
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) ss = fmaf(o[c], o[c], ss);
    for (int off = 1; off < GB; off <<= 1) ss += __shfl_xor(ss, off);
    const float inv = 1.0f / sqrtf(ss / (float)a.D + a.norm_eps);
    const float gv[8] = {gain0.x, gain0.y, gain0.z, gain0.w, gain1.x, gain1.y, gain1.z, gain1.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = o[c] * inv * gv[c];
  }

  const int c0 = g * 8;
  const int nope = a.D - a.r;
  if (c0 >= nope) {
    const double pos = (double)pos0 + (double)j * a.m;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pair = (c0 - nope) / 2 + q;
      float cs, sn;
      rope_cos_sin(pos, freq[pair], &cs, &sn);
      const float x0 = o[2 * q], x1 = o[2 * q + 1];
      o[2 * q] = x0 * cs - x1 * sn;
      o[2 * q + 1] = x0 * sn + x1 * cs;
    }
  }

  const int64_t orow = (int64_t)b * a.out_bstride + j;
  uint8_t* out = static_cast<uint8_t*>(a.out);
  const int out_fmt = MULTI ? a.out_fmt : OUT;
  if (out_fmt == kF32) {
    float4* p = reinterpret_cast<float4*>(out + (orow * a.D + c0) * 4);
    p[0] = make_float4(o[0], o[1], o[2], o[3]);
    p[1] = make_float4(o[4], o[5], o[6], o[7]);
  } else if (out_fmt == kBF16) {
    uint4* p = reinterpret_cast<uint4*>(out + (orow * a.D + c0) * 2);
    *p = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                    pack_bf16x2(o[6], o[7]));
  } else if (out_fmt == kMXFP4) {
    // MXFP4 (no rotated dims): the 4 threads of a 32-channel block are lanes
    // 4k .. 4k+3 (GB is a multiple of 4), and share the block's exponent
    // e = floor(log2 max|o|) - 2; each value becomes the nearest E2M1 code of
    // o / 2^e (ties to even, saturating at 6), sign bit for o < 0.
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(o[c]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int e = amax > 0.f ? min(127, max(-127, ilogbf(amax) - 2)) : 0;
    uint32_t codes = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float x = ldexpf(o[c], -e);
      const float ax = fabsf(x);
      const uint32_t q = ax <= 0.25f ? 0u : ax < 0.75f ? 1u : ax <= 1.25f ? 2u : ax < 1.75f ? 3u
                       : ax <= 2.5f ? 4u : ax < 3.5f ? 5u : ax <= 5.f ? 6u : 7u;
      codes |= (q | (x < 0.f ? 8u : 0u)) << (4 * c);
    }
    uint8_t* rp = out + orow * (int64_t)(a.D / 2 + a.D / 32);
    *reinterpret_cast<uint32_t*>(rp + c0 / 2) = codes;
    if ((g & 3) == 0) rp[a.D / 2 + c0 / 32] = (uint8_t)(e + 127);
  } else {
    const int64_t rowb = (int64_t)a.D + a.r;
    uint8_t* rp = out + orow * rowb;
    if (c0 < nope) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lo |= f32_to_e4m3(o[c]) << (8 * c);
        hi |= f32_to_e4m3(o[4 + c]) << (8 * c);
      }
      *reinterpret_cast<uint2*>(rp + c0) = make_uint2(lo, hi);
    } else {
      uint2* p = reinterpret_cast<uint2*>(rp + nope + 2 * (c0 - nope));
      p[0] = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      p[1] = make_uint2(pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
    }
  }
}

// The block decomposition of one call.  Split a block's tokens over S
// threads until each thread has at most 8 (a bf16 thread's loads are then
// all in flight at once), then give a block at most 256 threads: GB channel
// groups of one entry, or whole entries when an entry needs fewer threads.
// With RMSNorm the block keeps all G channel groups of an entry (G is a
// power of two, at most 64 with the norm), and the token split shrinks to
// fit: a long block (m' = 128) is then streamed by one compute unit.
// Returns the call's threads per workgroup.
int plan_call(const CompressArgs& a, CompressK* k) {
  const int G = a.D / 8;
  int S = 1;
  const int L = a.m + a.overlap;                 // tokens per window
  // Few entries (a decode step's newest block): up to kFewPer tokens per
  // thread and kFewGB channel groups per block, so that a long block spreads
  // over more workgroups.
  constexpr int kFewPer = 4, kFewGB = 4;
  const bool few = a.norm_gain == nullptr && (int64_t)a.B * (a.T / a.m) * G < 4096;
  const int per_max = few ? kFewPer : 8;
  while ((L + S - 1) / S > per_max && S < 256 && (a.overlap > 0 || a.m % (2 * S) == 0)) S *= 2;
  int GB = G;
  if (a.norm_gain == nullptr)
    while ((GB * S > 256 || (few && GB > kFewGB)) && GB % 2 == 0) GB /= 2;
  if (a.out_fmt == kMXFP4 && GB % 4) GB = 4;   // a 32-channel block's threads share one block
  if (GB * S > 512) {           // few channel groups and a long block: fewer splits
    while (GB * S > 512) S /= 2;
  }
  const int threads = GB * S <= 256 ? (GB == G ? 256 : GB * S) : GB * S;
  const int epb = threads / (GB * S);
  *k = CompressK{};
  k->kv = a.kv; k->logits = a.logits; k->out = a.out; k->norm_gain = a.norm_gain;
  k->kv_bstride = a.kv_bstride; k->z_bstride = a.z_bstride; k->out_bstride = a.out_bstride;
  k->out_fmt = a.out_fmt; k->D = a.D; k->m = a.m; k->r = a.r; k->overlap = a.overlap;
  k->N = a.T / a.m;
  k->per = (L + S - 1) / S;
  k->tokn = k->per <= 4 ? 4 : 8;
  k->gb = GB; k->s = S; k->epb = epb;
  k->gx = (k->N + epb - 1) / epb;
  k->gy = G / GB;
  // floor(t / d) = (t * ceil(2^20 / d)) >> 20 for t < 512 and d <= 512: the
  // error t * (ceil(2^20 / d) * d - 2^20) / (d * 2^20) < 512 / 2^20 < 1/d
  k->mul_gb = (uint32_t)(((1u << 20) + GB - 1) / GB);
  k->mul_gbs = (uint32_t)(((1u << 20) + GB * S - 1) / (GB * S));
  k->norm_eps = a.norm_eps;
  return GB * S * epb;
}

template <int IN, int TOKN, int OUT>
hipError_t set_lds_limit() {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&compress_kernel<IN, TOKN, OUT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 512 * 25 * (int)sizeof(float));
  return attr;
}

template <int IN, int TOKN>
hipError_t launch_one(const CLaunch& L, int threads, bool tree, int B, hipStream_t st) {
  const size_t lds = tree ? (size_t)threads * 25 * sizeof(float) : 0;
  hipError_t e;
  TimedLaunch tl(kKernelCompress, st);
  if (L.n == 1 && L.n_clr == 0) {
    const CompressK& k = L.c[0];
    const dim3 grid(k.gx, k.gy, B), block(k.gb, k.s, k.epb);
    auto one = [&](auto out_c) {
      constexpr int OUT = decltype(out_c)::value;
      hipError_t e1 = set_lds_limit<IN, TOKN, OUT>();
      if (e1 != hipSuccess) return e1;
      hipLaunchKernelGGL((compress_kernel<IN, TOKN, OUT>), grid, block, lds, st, L);
      return hipGetLastError();
    };
    switch (k.out_fmt) {
      case kF32: return one(std::integral_constant<int, kF32>{});
      case kBF16: return one(std::integral_constant<int, kBF16>{});
      case kMXFP4: return one(std::integral_constant<int, kMXFP4>{});
      default: return one(std::integral_constant<int, kMixed>{});
    }
  }
  if ((e = set_lds_limit<IN, TOKN, -1>()) != hipSuccess) return e;
  // (x, y) grid of at least the launch's workgroups, x fastest
  const uint32_t total = L.blk_total;
  const uint32_t gx = std::min<uint32_t>(total, 65536u);
  hipLaunchKernelGGL((compress_kernel<IN, TOKN, -1>), dim3(gx, (total + gx - 1) / gx),
                     dim3(threads), lds, st, L);
  return hipGetLastError();
}

}  // namespace

// Calls of one input format and one loads-in-flight count go into launches
// of up to kCompressGroup calls, in call order, as long as their positions
// and rotation tables fit the launch's pools.  Clearing jobs ride on the
// first launch (up to kCompressGroup of them; the rest, and jobs with no
// compress call to join, take launches of their own).
hipError_t launch_compress_group(const CompressArgs* calls, int n, hipStream_t st,
                                 const ClearJob* clears, int n_clears) {
  int clr_next = 0;
  // append the pending clearing jobs (up to the launch's capacity) after the
  // calls' workgroups of L, whose workgroups have `threads` threads
  auto add_clears = [&](CLaunch& L, int threads) {
    uint32_t end = L.n ? L.blk_end[L.n - 1] : 0u;
    while (clr_next < n_clears && L.n_clr < kCompressGroup) {
      const ClearJob& c = clears[clr_next++];
      if (c.words == 0) continue;
      L.clr[L.n_clr] = c.p;
      L.clr_words[L.n_clr] = c.words;
      end += (uint32_t)((c.words / 4 + threads - 1) / threads);
      L.clr_end[L.n_clr] = end;
      ++L.n_clr;
    }
    L.blk_total = end;
  };
  for (int variant = 0; variant < 4; ++variant) {
    const int fmt = variant < 2 ? kF32 : kBF16, tokn = variant % 2 ? 8 : 4;
    CLaunch L{};
    int threads = 0, n_tab = 0, B1 = 0;      // B1: the first call's batch (single-call grid)
    bool tree = false;
    int n_pos = 0;
    float tab_theta[kCompressTables];
    int tab_r[kCompressTables];
    auto flush = [&]() -> hipError_t {
      if (L.n == 0) return hipSuccess;
      add_clears(L, threads);
      const hipError_t e = fmt == kF32 ? (tokn == 4 ? launch_one<kF32, 4>(L, threads, tree, B1, st)
                                                    : launch_one<kF32, 8>(L, threads, tree, B1, st))
                                       : (tokn == 4 ? launch_one<kBF16, 4>(L, threads, tree, B1, st)
                                                    : launch_one<kBF16, 8>(L, threads, tree, B1, st));
      L = CLaunch{};
      threads = 0; n_tab = 0; tree = false; n_pos = 0; B1 = 0;
      return e;
    };
    for (int i = 0; i < n; ++i) {
      const CompressArgs& a = calls[i];
      if (a.in_fmt != fmt || (int64_t)a.B * (a.T / a.m) == 0) continue;
      CompressK k;
      const int thr = plan_call(a, &k);
      if (k.tokn != tokn) continue;
      // the call's rotation table: an equal one already in the pool, or a new one
      int tab = -1;
      if (a.r > 0) {
        for (int q = 0; q < n_tab; ++q)
          if (tab_r[q] == a.r && tab_theta[q] == a.theta) tab = q;
      }
      const uint32_t nblk = (uint32_t)k.gx * (uint32_t)k.gy * (uint32_t)a.B;
      const bool fits = L.n < kCompressGroup && n_pos + a.B <= kCompressPos &&
                        (a.r == 0 || tab >= 0 || n_tab < kCompressTables) &&
                        (L.n == 0 || (uint64_t)L.blk_end[L.n - 1] + nblk < (1u << 30));
      if (!fits) {
        const hipError_t e = flush();
        if (e != hipSuccess) return e;
        tab = -1;
      }
      if (a.r > 0 && tab < 0) {
        tab = n_tab++;
        tab_r[tab] = a.r;
        tab_theta[tab] = a.theta;
        RopeTable rt;
        make_rope_table(&rt, a.r, a.theta);
        for (int p = 0; p < kMaxRopePairs; ++p) L.freq[tab * kMaxRopePairs + p] = rt.inv_freq[p];
      }
      k.freq_off = tab < 0 ? 0 : tab * kMaxRopePairs;
      k.pos_off = n_pos;
      for (int b = 0; b < a.B; ++b) L.pos[n_pos + b] = a.pos0.v[b];
      n_pos += a.B;
      if (L.n == 0) B1 = a.B;
      L.c[L.n] = k;
      L.blk_end[L.n] = (L.n ? L.blk_end[L.n - 1] : 0u) + nblk;
      ++L.n;
      threads = std::max(threads, thr);
      tree = tree || k.s > 1;
    }
    const hipError_t e = flush();
    if (e != hipSuccess) return e;
  }
  // clearing jobs left over: launches of 256-thread clearing workgroups
  while (clr_next < n_clears) {
    CLaunch L{};
    add_clears(L, 256);
    if (L.n_clr == 0) break;
    const hipError_t e = launch_one<kBF16, 4>(L, 256, false, 0, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_compress(CompressArgs a, hipStream_t st) { return launch_compress_group(&a, 1, st); }

}  // namespace lac
