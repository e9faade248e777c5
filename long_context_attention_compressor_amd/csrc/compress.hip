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

// Block (GB, S, epb): thread (x, y, z) owns channel group slice * GB + x of
// entry blockIdx.x * epb + z and token share y of its block; the grid is
// (entry groups, channel slices, sequences), so no index needs a division.
template <int IN, int OUT>
__global__ void __launch_bounds__(512) compress_kernel(CompressArgs a) {
  extern __shared__ float part[];                  // [blockDim][25] when S > 1
  __shared__ double freq[kMaxRopePairs];
  const int GB = a.gb, S = a.s;
  const int s = threadIdx.y;
  const int g = blockIdx.y * GB + threadIdx.x;
  const int b = blockIdx.z;
  const int j = blockIdx.x * a.epb + threadIdx.z;
  const bool live = j < a.N;
  const int t = (threadIdx.z * S + s) * GB + threadIdx.x;
  const int nthreads = GB * S * a.epb;

  float mx[8], den[8], acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) { mx[c] = -INFINITY; den[c] = 0.f; acc[c] = 0.f; }
  // the gains of this thread's 8 channels, requested first
  float4 gain0 = make_float4(1.f, 1.f, 1.f, 1.f), gain1 = gain0;
  if (a.norm_gain) {
    gain0 = *reinterpret_cast<const float4*>(a.norm_gain + g * 8);
    gain1 = *reinterpret_cast<const float4*>(a.norm_gain + g * 8 + 4);
  }

  if (live) {
    const int per = a.per;
    const int64_t row0 = (int64_t)j * a.m + (int64_t)s * per;
    const int64_t xb = (b * a.kv_bstride + row0) * a.D + g * 8;
    const int64_t zb = (b * a.z_bstride + row0) * a.D + g * 8;
    // TOK tokens' loads in flight before any of them is used, kept packed
    // until used (rows past the thread's share re-read its last row and are
    // not used).
    constexpr int TOK = IN == kF32 ? 4 : 8;
    for (int i = 0; i < per; i += TOK) {
      Raw8<IN> xr[TOK], zr[TOK];
#pragma unroll
      for (int u = 0; u < TOK; ++u) {
        const int64_t row = min(i + u, per - 1);
        xr[u] = load_raw8<IN>(a.kv, xb + row * a.D);
        zr[u] = load_raw8<IN>(a.logits, zb + row * a.D);
      }
      if (i == 0) {
        rope_freq_table(freq, a.rope, a.r, t, nthreads);
      }
#pragma unroll
      for (int u = 0; u < TOK; ++u) {
        if (i + u < per) {
          float xv[8], zv[8];
          unpack8<IN>(xr[u], xv);
          unpack8<IN>(zr[u], zv);
          softmax_step<IN>(xv, zv, mx, den, acc);
        }
      }
    }
  } else {
    rope_freq_table(freq, a.rope, a.r, t, nthreads);
  }
  __syncthreads();                   // rotation table complete

  if (S > 1) {
    // Tree merge: at level o, thread s < o absorbs thread s + o.
    float* mine = part + t * 25;
    for (int o = S >> 1; o >= 1; o >>= 1) {
      if (s < 2 * o) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          mine[c] = mx[c];
          mine[8 + c] = den[c];
          mine[16 + c] = acc[c];
        }
      }
      __syncthreads();
      if (s < o) {
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
    const double pos = (double)a.pos0.v[b] + (double)j * a.m;
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
  if constexpr (OUT == kF32) {
    float4* p = reinterpret_cast<float4*>(out + (orow * a.D + c0) * 4);
    p[0] = make_float4(o[0], o[1], o[2], o[3]);
    p[1] = make_float4(o[4], o[5], o[6], o[7]);
  } else if constexpr (OUT == kBF16) {
    uint4* p = reinterpret_cast<uint4*>(out + (orow * a.D + c0) * 2);
    *p = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                    pack_bf16x2(o[6], o[7]));
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

template <int IN, int OUT>
hipError_t launch(const CompressArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t st) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&compress_kernel<IN, OUT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 512 * 25 * (int)sizeof(float));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((compress_kernel<IN, OUT>), grid, block, lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress(CompressArgs a, hipStream_t st) {
  const int G = a.D / 8;
  // Split a block's tokens over S threads until each thread has at most 8
  // (a bf16 thread's loads are then all in flight at once), then give a
  // block at most 256 threads: GB channel groups of one entry, or whole
  // entries when an entry needs fewer threads.
  // With RMSNorm the block keeps all G channel groups of an entry (G is a
  // power of two, at most 64 with the norm), and the token split shrinks to
  // fit: a long block (m' = 128) is then streamed by one compute unit.
  int S = 1;
  while (a.m / S > 8 && S < 256 && a.m % (2 * S) == 0) S *= 2;
  int GB = G;
  if (a.norm_gain == nullptr)
    while (GB * S > 256 && GB % 2 == 0) GB /= 2;
  if (GB * S > 512) {           // few channel groups and a long block: fewer splits
    while (GB * S > 512) S /= 2;
  }
  a.per = a.m / S;
  a.gb = GB;
  a.s = S;
  const int threads = GB * S <= 256 ? (GB == G ? 256 : GB * S) : GB * S;
  const int epb = threads / (GB * S);
  a.epb = epb;
  make_rope_table(&a.rope, a.r, a.theta);
  const size_t lds = S > 1 ? (size_t)threads * 25 * sizeof(float) : 0;
  const int N = a.T / a.m;
  a.N = N;
  if ((int64_t)a.B * N == 0) return hipSuccess;
  const dim3 grid((unsigned)((N + epb - 1) / epb), (unsigned)(G / GB), (unsigned)a.B);
  const dim3 block((unsigned)GB, (unsigned)S, (unsigned)epb);
  TimedLaunch tl(kKernelCompress, st);
  if (a.in_fmt == kF32) {
    if (a.out_fmt == kF32) return launch<kF32, kF32>(a, grid, block, lds, st);
    if (a.out_fmt == kBF16) return launch<kF32, kBF16>(a, grid, block, lds, st);
    return launch<kF32, kMixed>(a, grid, block, lds, st);
  }
  if (a.out_fmt == kF32) return launch<kBF16, kF32>(a, grid, block, lds, st);
  if (a.out_fmt == kBF16) return launch<kBF16, kBF16>(a, grid, block, lds, st);
  return launch<kBF16, kMixed>(a, grid, block, lds, st);
}

}  // namespace lac
