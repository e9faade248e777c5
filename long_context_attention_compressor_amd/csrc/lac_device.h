// lac_device.h -- device helpers shared by the gfx950 kernels of the library:
// number formats, rotary angles, MFMA operand types and small reductions.
#pragma once
#include <cmath>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lac {

constexpr int kWave = 64;
constexpr int kMaxBatch = 128;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// gfx950's block-scaled FP8/FP4 matrix product, 32 x 32 outputs over 64
// products per step: acc[32 x 32] += (A x 2^(sa - 127)) (B x 2^(sb - 127)).
// Operand layout (pinned on the device against exact products): lane l holds
// row (A) or column (B) l % 32; with h = l / 32,
//   FP8 (format 0, E4M3): byte p of the 32 is step index
//       32 (p / 16) + 16 h + p % 16,
//   FP4 (format 4, E2M1; only the first 16 bytes are read): nibble q (value
//       2i in the low nibble of byte i) is step index 32 h + q,
// and the scale of row/column l % 32 over step indices [32c, 32c + 32) comes
// from lane l % 32 + 32 c (byte 0 of its scale word).  The result is laid out
// as for v_mfma_f32_32x32x16_bf16.
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_scaled_32x32x64(const i32x8& a, const i32x8& b, const f32x16& acc,
                                                       int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, FA, FB, 0, sa, 0, sb);
}
// Four 8-byte fragments (consecutive step indices of one lane) as one operand.
__device__ __forceinline__ i32x8 cat4(long a, long b, long c, long d) {
  i32x8 r;
  r[0] = (int)a; r[1] = (int)(a >> 32); r[2] = (int)b; r[3] = (int)(b >> 32);
  r[4] = (int)c; r[5] = (int)(c >> 32); r[6] = (int)d; r[7] = (int)(d >> 32);
  return r;
}

// Streaming loads (read-once data): non-temporal hint, 16 or 8 bytes.
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(static_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

// kMX4E4: MXFP4 indexer keys scored against E4M3 queries on the scaled FP4 MFMA.
enum Fmt { kF32 = 0, kBF16 = 1, kMixed = 2, kE4M3 = 3, kMXFP4 = 4, kMX4E4 = 5 };

// Per-batch positions passed by value (the library keeps nothing on the device).
struct Positions {
  int32_t v[kMaxBatch];
};

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Two floats to two bf16 (lo in the low half), rounded to nearest even by the
// hardware converter (v_cvt_pk_bf16_f32); NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t b = __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &b, 4);
  return u;
}

// Eight E2M1 codes (nibbles of `codes`, element j in bits 4j..4j+3) times
// the E8M0 scale 2^(sc - 127) -> eight bf16, exact (E2M1: bias 1, exponent 0
// subnormal; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  Scale bytes 1..254 go
// through gfx950's scaled FP4 conversion (two codes of one byte per
// instruction, the low nibble first; exact for these scales), the two
// edge bytes (2^-127, NaN) through float arithmetic.
__device__ __noinline__ uint4 e2m1x8_to_bf16x8_edge(uint32_t codes, uint32_t sc) {
  const float scale = sc == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(0x7fc00000u);
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t c = (codes >> (4 * j)) & 7u;
    const float mag = c == 0u ? 0.f : c == 1u ? 0.5f : __uint_as_float(((126u + (c >> 1)) << 23) | ((c & 1u) << 22));
    v[j] = ((codes >> (4 * j + 3)) & 1u ? -mag : mag) * scale;
  }
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}

__device__ __forceinline__ uint4 e2m1x8_to_bf16x8(uint32_t codes, uint32_t sc) {
  if (sc == 0u || sc == 255u) return e2m1x8_to_bf16x8_edge(codes, sc);
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const float scale = __uint_as_float(sc << 23);
  const bf16x2_t r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  const bf16x2_t r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  const bf16x2_t r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  const bf16x2_t r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  uint4 out;
  __builtin_memcpy(&out.x, &r0, 4);
  __builtin_memcpy(&out.y, &r1, 4);
  __builtin_memcpy(&out.z, &r2, 4);
  __builtin_memcpy(&out.w, &r3, 4);
  return out;
}

// x rounded to the nearest bf16 value (ties to even), as a float.
__device__ __forceinline__ float round_bf16(float x) { return bf16_to_f32(pack_bf16x2(x, 0.f) & 0xffffu); }

// Two floats as bf16 high parts plus bf16 low parts: hi = bf16(x), lo =
// bf16(x - hi) (the difference is exact in fp32), so hi + lo carries about 16
// significant bits of x.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t* hi, uint32_t* lo) {
  const uint32_t h = pack_bf16x2(x0, x1);
  *hi = h;
  *lo = pack_bf16x2(x0 - bf16_to_f32(h & 0xffffu), x1 - bf16_to_f32(h >> 16));
}

// ---------------------------------------------------------------- FP8 E4M3 ("fn")
// Exponent bias 7, largest finite 448, subnormal step 2^-9, 0x7f/0xff NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t em = b & 0x7fu;
  float v = em >= 8u ? __uint_as_float((em << 20) + (120u << 23))   // normal: rebias 7 -> 127
                     : (float)em * 0.001953125f;                    // subnormal: em * 2^-9
  if (em == 0x7fu) v = __uint_as_float(0x7fc00000u);
  return (b & 0x80u) ? -v : v;
}

// Eight E4M3 codes (bytes of lo, then hi) -> eight bf16 (exact), with the
// gfx950 packed conversion (scale 1).
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

// Round to nearest even, saturate to +-448, NaN -> 0x7f.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  const float af = __uint_as_float(a);
  if (af >= 448.0f) return s | 0x7eu;
  if (af < 0.015625f) {                              // below 2^-6: multiples of 2^-9
    return s | (uint32_t)__builtin_rintf(af * 512.0f);  // 8 encodes 2^-6 exactly
  }
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) & 0xfff00000u;  // keep 3 mantissa bits
  return s | ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
}

// ---------------------------------------------------------------- rotary angles
// Rotation of pair i (of r/2) at integer position p by angle p * theta^(-2i/r).
// The inverse frequencies are computed on the host in double (one pow per
// pair) and passed by value with the launch; a kernel copies them to LDS.
// The product with the position and its reduction to a quarter turn are
// taken in double, so the angle stays exact to float precision at positions
// in the millions.
constexpr int kMaxRopePairs = 64;   // rope_dims <= 128

struct RopeTable {
  double inv_freq[kMaxRopePairs];
};

inline void make_rope_table(RopeTable* t, int r, float theta) {
  for (int i = 0; i < kMaxRopePairs; ++i)
    t->inv_freq[i] = i < r / 2 ? std::pow((double)theta, -2.0 * (double)i / (double)r) : 0.0;
}

// tab[i] = inv_freq[i], i < r/2, by threads tid of nthreads; the caller
// synchronises.
__device__ __forceinline__ void rope_freq_table(double* tab, const RopeTable& t, int r, int tid,
                                                int nthreads) {
  for (int i = tid; i < r / 2; i += nthreads) tab[i] = t.inv_freq[i];
}

// cos and sin of pos * inv_freq.  The angle is reduced in double to
// x in [-pi/4, pi/4] plus a quarter-turn count q; sin x and cos x are their
// Taylor series through x^9 and x^10 in float (truncation below 2e-9 on
// that interval), and q picks the signs and the swap.
__device__ __forceinline__ void rope_cos_sin(double pos, double inv_freq, float* c, float* s) {
  const double a = pos * inv_freq;
  const double k = rint(a * 0.63661977236758134);          // a / (pi/2)
  double red = fma(-k, 1.5707963267948966, a);             // pi/2, high part
  red = fma(-k, 6.123233995736766e-17, red);               // pi/2, low part
  const float x = (float)red, x2 = x * x;
  const float sx = x * fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, 1.f / 362880.f, -1.f / 5040.f), 1.f / 120.f),
                                     -1.f / 6.f), 1.f);
  const float cx = fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, -1.f / 3628800.f, 1.f / 40320.f),
                                                   -1.f / 720.f), 1.f / 24.f), -0.5f), 1.f);
  const int q = (int)((int64_t)k & 3);
  const float sv = (q & 1) ? cx : sx, cv = (q & 1) ? sx : cx;
  *s = (q & 2) ? -sv : sv;
  *c = ((q + 1) & 2) ? -cv : cv;
}

// ---------------------------------------------------------------- lanes, LDS histograms
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// LDS histogram add for the wave's active lanes: one atomic when every
// active lane holds the same digit (common in the high radix digits), else
// one atomic per lane (cheaper than serialising over many distinct digits).
__device__ __forceinline__ void hist_add(uint32_t* hist, bool on, uint32_t d) {
  const uint64_t active = __ballot(on);
  if (!active) return;
  const int leader = __ffsll((unsigned long long)active) - 1;
  const uint32_t dl = __builtin_amdgcn_readlane(d, leader);
  const uint64_t same = __ballot(on && d == dl);
  if (same == active) {
    if (lane_id() == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(same));
  } else if (on) {
    atomicAdd(&hist[d], 1u);
  }
}

// ---------------------------------------------------------------- ReLU
// max(x, 0) as one integer max: a float with the sign bit set is a negative
// int32 and maps to +0 (so does -0); a non-negative float is unchanged.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// ---------------------------------------------------------------- selection keys
// Order-preserving map of a float score to uint32 (larger score -> larger key).
// -0 is folded onto +0 so that equal scores compare equal.
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---------------------------------------------------------------- positions
__device__ __forceinline__ int64_t n_visible(int64_t t, int64_t N, int m) {
  const int64_t n = t >= 0 ? t / m : 0;
  return n < N ? n : N;
}

}  // namespace lac
