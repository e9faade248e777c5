// attend.hip -- core attention of CSA (sparse, over the selected compressed
// entries) and HCA (dense, over every visible compressed entry), each with
// the raw sliding window and the optional attention sink.
//
// QbitAI rewrite (futuo-fx-trading.com): Multi-Query Attention over the
// selected compressed blocks; the KV entries act as key and value, so RoPE on
// the last 64 dims is matched by a rotation at position -i on the output;
// strict causality.  "深度解析 DeepSeek-V4" (learnblockchain.cn): HCA runs
// dense attention over all compressed entries; "Sliding Window Branch" adds
// the most recent raw entries; "Attention Sink" adds learnable logits to the
// softmax denominator.  For query t, head h:
//   o = sum_e exp(l_e) e / (exp(sink_h) + sum_e exp(l_e)),  l_e = scale q~ . e,
//   y = R(-t) o,  q~ = R(t) q,  window entries e = R(s) raw[s].
//
// Kernels:
//  * rope_window: rotates the raw rows a call needs (positions
//    [max(0, t_first - W + 1), t_last]) once into workspace, in the KV storage
//    format, so every query reads ready window entries exactly like cache rows.
//  * attend_mfma<D, KV>: one workgroup (4 waves) owns a 64-row tile (64 heads
//    of one query, or G = 64/H queries x H heads) and a contiguous share of
//    that tile's entry list (split-K).  Per 32-entry tile: the entries are
//    gathered (FP8 rows decoded to bf16 on the fly) into LDS once and used for
//    both products (K = V).  QK: each wave contracts its quarter of D
//    (v_mfma_f32_32x32x16_bf16, query rows as A operand held in VGPRs), the
//    four partial logit tiles are summed in LDS; the online softmax runs one
//    thread per (row, 8 entries); PV: each wave owns a quarter of the output
//    columns, P (bf16) is the A operand and the entry tile, read column-wise
//    from LDS, the B operand.  fp32 accumulation throughout.
//  * combine: merges split partials (max, sum, unnormalised output) with the
//    sink, divides, applies the output rotation and stores.
//  * attend_f32: a plain VALU kernel for float32 inputs (small shapes).
#include "lac_internal.h"

namespace lac {

namespace {

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline int64_t kv_row_bytes(int fmt, int D, int r) {
  return fmt == kF32 ? 4LL * D : fmt == kBF16 ? 2LL * D : (int64_t)D + r;
}

// ---------------------------------------------------------------- plan
struct AttnPlan {
  int G, Hs, n_htiles, n_qgroups, n_work, nsplit, chunk, max_entries;
  int64_t win_rows, row_bytes;
  size_t off_win, off_po, off_pml, total;
};

AttnPlan make_plan(int B, int Tq, int H, int D, int r, int kv_fmt, int n_entries, int W,
                   bool f32_path) {
  AttnPlan p{};
  p.row_bytes = kv_row_bytes(kv_fmt, D, r);
  p.win_rows = W > 0 ? (int64_t)Tq + W - 1 : 0;
  size_t off = 0;
  p.off_win = off;
  off += round_up((int64_t)B * p.win_rows * p.row_bytes, 256);
  if (f32_path) {
    p.G = 1; p.Hs = H; p.n_htiles = 1; p.n_qgroups = Tq; p.n_work = B * Tq; p.nsplit = 1;
    p.total = off;
    return p;
  }
  p.Hs = H >= 64 ? 64 : H;
  p.G = 64 / p.Hs;
  p.n_htiles = H >= 64 ? H / 64 : 1;
  p.n_qgroups = (Tq + p.G - 1) / p.G;
  p.n_work = B * p.n_qgroups * p.n_htiles;
  p.max_entries = p.G * n_entries + (W > 0 ? W + p.G - 1 : 0);
  if (p.max_entries < 1) p.max_entries = 1;
  const int max_split = (int)((p.max_entries + 127) / 128);
  int ns = p.n_work >= 512 ? 1 : (512 + p.n_work - 1) / p.n_work;
  if (ns > max_split) ns = max_split;
  if (ns < 1) ns = 1;
  p.chunk = (int)round_up((p.max_entries + ns - 1) / ns, 32);
  p.nsplit = (p.max_entries + p.chunk - 1) / p.chunk;
  if (p.nsplit > 1) {
    p.off_po = off;
    off += round_up((int64_t)p.n_work * p.nsplit * 64 * D * 4, 256);
    p.off_pml = off;
    off += round_up((int64_t)p.n_work * p.nsplit * 64 * 2 * 4, 256);
  }
  p.total = off;
  return p;
}

// ---------------------------------------------------------------- window rotation
struct WinArgs {
  const uint8_t* raw;
  uint8_t* win;
  int fmt, B, D, r, Tq, W;
  int64_t T_raw, win_rows, row_bytes;
  float theta;
  Positions qpos, rawpos;
};

__global__ void __launch_bounds__(256) rope_window_kernel(WinArgs a) {
  __shared__ double freq[kMaxRopePairs];
  rope_freq_table(freq, a.r, a.theta);
  __syncthreads();
  const int G8 = a.D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_b = a.win_rows * G8;
  if (gid >= (int64_t)a.B * per_b) return;
  const int b = (int)(gid / per_b);
  const int64_t rem = gid - b * per_b;
  const int64_t row = rem / G8;
  const int g = (int)(rem - row * G8);
  const int64_t lo = max((int64_t)0, (int64_t)a.qpos.v[b] - a.W + 1);
  const int64_t s = lo + row;
  if (s > (int64_t)a.qpos.v[b] + a.Tq - 1) return;
  const uint8_t* src = a.raw + ((int64_t)b * a.T_raw + (s - a.rawpos.v[b])) * a.row_bytes;
  uint8_t* dst = a.win + ((int64_t)b * a.win_rows + row) * a.row_bytes;
  const int c0 = g * 8, nope = a.D - a.r;
  if (c0 < nope) {   // not rotated: copy
    if (a.fmt == kF32) {
      reinterpret_cast<float4*>(dst + c0 * 4)[0] = reinterpret_cast<const float4*>(src + c0 * 4)[0];
      reinterpret_cast<float4*>(dst + c0 * 4)[1] = reinterpret_cast<const float4*>(src + c0 * 4)[1];
    } else if (a.fmt == kBF16) {
      *reinterpret_cast<uint4*>(dst + c0 * 2) = *reinterpret_cast<const uint4*>(src + c0 * 2);
    } else {
      *reinterpret_cast<uint2*>(dst + c0) = *reinterpret_cast<const uint2*>(src + c0);
    }
    return;
  }
  float v[8];
  const int64_t off = a.fmt == kF32 ? c0 * 4 : a.fmt == kBF16 ? c0 * 2 : nope + 2 * (c0 - nope);
  if (a.fmt == kF32) {
    const float4 x = reinterpret_cast<const float4*>(src + off)[0];
    const float4 y = reinterpret_cast<const float4*>(src + off)[1];
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else {
    const uint2 x = reinterpret_cast<const uint2*>(src + off)[0];
    const uint2 y = reinterpret_cast<const uint2*>(src + off)[1];
    const uint32_t w4[4] = {x.x, x.y, y.x, y.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_to_f32(w4[i] & 0xffffu); v[2 * i + 1] = bf16_to_f32(w4[i] >> 16); }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float cs, sn;
    rope_cos_sin((double)s, freq[(c0 - nope) / 2 + q], &cs, &sn);
    const float x0 = v[2 * q], x1 = v[2 * q + 1];
    v[2 * q] = x0 * cs - x1 * sn;
    v[2 * q + 1] = x0 * sn + x1 * cs;
  }
  if (a.fmt == kF32) {
    reinterpret_cast<float4*>(dst + off)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(dst + off)[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    reinterpret_cast<uint2*>(dst + off)[0] = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    reinterpret_cast<uint2*>(dst + off)[1] = make_uint2(pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
}

// ---------------------------------------------------------------- entry lists
struct KArgs {
  const void* q;
  const uint8_t* kv;
  const int32_t* idx;
  const uint8_t* win;
  const float* sink;
  void* out;
  float* part_o;
  float* part_ml;
  int mode, N, k, m, W, B, Tq, H, D, r;
  float theta, scale_log2;
  int G, Hs, n_htiles, n_qgroups, nsplit, chunk;
  int64_t win_rows, row_bytes;
  Positions qpos;
};

// Work item decomposition: blockIdx.x = split (fastest), blockIdx.y = work.
struct Work {
  int b, i0, h0, n_q;       // queries i0 .. i0+n_q-1, heads h0 ..
  int64_t t_first, t_last;
  int64_t n_comp, lo_w, n_tot;
};

__device__ __forceinline__ Work make_work(const KArgs& a, int work) {
  Work w;
  const int ht = work % a.n_htiles;
  const int rest = work / a.n_htiles;
  const int qg = rest % a.n_qgroups;
  w.b = rest / a.n_qgroups;
  w.i0 = qg * a.G;
  w.h0 = ht * 64;
  w.n_q = min(a.G, a.Tq - w.i0);
  w.t_first = (int64_t)a.qpos.v[w.b] + w.i0;
  w.t_last = w.t_first + w.n_q - 1;
  w.n_comp = a.mode == 0 ? (int64_t)w.n_q * a.k : n_visible(w.t_last, a.N, a.m);
  w.lo_w = max((int64_t)0, w.t_first - a.W + 1);
  const int64_t n_win = a.W > 0 ? w.t_last - w.lo_w + 1 : 0;
  w.n_tot = w.n_comp + n_win;
  return w;
}

// Entry e of the work list -> source row pointer (null if it names nothing)
// and its tag: CSA compressed: query g (0..G-1); HCA compressed: -1 - j;
// window: 1 << 30 | (s - lo_w).
__device__ __forceinline__ const uint8_t* entry_src(const KArgs& a, const Work& w, int64_t e,
                                                    int* tag) {
  if (e >= w.n_tot) { *tag = -0x7fffffff; return nullptr; }
  if (e < w.n_comp) {
    int64_t j;
    if (a.mode == 0) {
      const int g = (int)(e / a.k);
      j = a.idx[((int64_t)w.b * a.Tq + w.i0 + g) * a.k + (e - (int64_t)g * a.k)];
      if (j < 0 || j >= a.N) { *tag = -0x7fffffff; return nullptr; }
      *tag = g;
    } else {
      j = e;
      *tag = -1 - (int)j;
    }
    return a.kv + ((int64_t)w.b * a.N + j) * a.row_bytes;
  }
  const int64_t off = e - w.n_comp;
  *tag = (1 << 30) | (int)off;
  return a.win + ((int64_t)w.b * a.win_rows + (w.lo_w - max((int64_t)0, (int64_t)a.qpos.v[w.b] - a.W + 1)) + off) * a.row_bytes;
}

// Whether entry with `tag` is visible to query g of the work item.
__device__ __forceinline__ bool entry_visible(const KArgs& a, const Work& w, int tag, int g) {
  if (tag == -0x7fffffff || g >= w.n_q) return false;
  const int64_t t = w.t_first + g;
  if (tag >= (1 << 30)) {
    const int64_t s = w.lo_w + (tag - (1 << 30));
    return s <= t && s >= t - a.W + 1;
  }
  if (a.mode == 0) return tag == g;
  return (int64_t)(-1 - tag) < n_visible(t, a.N, a.m);
}

// ---------------------------------------------------------------- MFMA attention
template <int D>
struct Geo {
  static constexpr int DW = D / 4;          // columns per wave
  static constexpr int KQ = DW / 16;        // QK k-steps per wave
  static constexpr int DT = DW / 32;        // PV column tiles per wave
  static constexpr int GPT = D / 64;        // 8-dim groups staged per thread
  static constexpr int EROW = 2 * D + 16;   // LDS bytes per staged entry
  static constexpr int SROW = 68;           // floats per (wave, rt, v) logit row
  static constexpr int PROW = 40;           // bf16 per row of P
};

template <int D, int KV>
struct Stage {
  uint4 raw[Geo<D>::GPT];
};

template <int D, int KV>
__device__ __forceinline__ void stage_load(const uint8_t* src, int part, int nope, Stage<D, KV>& st) {
  constexpr int GPT = Geo<D>::GPT;
#pragma unroll
  for (int q = 0; q < GPT; ++q) {
    const int c0 = (part * GPT + q) * 8;
    if (src == nullptr) { st.raw[q] = make_uint4(0, 0, 0, 0); continue; }
    if constexpr (KV == kBF16) {
      st.raw[q] = ld_stream16(src + 2 * c0);
    } else {
      if (c0 < nope) {
        const uint2 x = ld_stream8(src + c0);
        st.raw[q] = make_uint4(x.x, x.y, 0, 0);
      } else {
        const uint8_t* p = src + nope + 2 * (c0 - nope);
        const uint2 x = ld_stream8(p), y = ld_stream8(p + 8);
        st.raw[q] = make_uint4(x.x, x.y, y.x, y.y);
      }
    }
  }
}

template <int D, int KV>
__device__ __forceinline__ void stage_store(uint8_t* lds_row, int part, int nope, const Stage<D, KV>& st) {
  constexpr int GPT = Geo<D>::GPT;
#pragma unroll
  for (int q = 0; q < GPT; ++q) {
    const int c0 = (part * GPT + q) * 8;
    uint4 v = st.raw[q];
    if constexpr (KV == kMixed) {
      if (c0 < nope) {
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[i] = e4m3_to_f32((v.x >> (8 * i)) & 0xffu);
          f[4 + i] = e4m3_to_f32((v.y >> (8 * i)) & 0xffu);
        }
        // E4M3 values are exact in bf16.
        v = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                       pack_bf16x2(f[6], f[7]));
      }
    }
    *reinterpret_cast<uint4*>(lds_row + 2 * c0) = v;
  }
}

template <int D, int KV>
__global__ void __launch_bounds__(256) attend_mfma_kernel(KArgs a) {
  using Gm = Geo<D>;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* Et = smem;                                                   // [32][EROW]
  float* Sp = reinterpret_cast<float*>(Et + 32 * Gm::EROW);             // [4][2][16][SROW]
  uint16_t* Pl = reinterpret_cast<uint16_t*>(Sp + 4 * 2 * 16 * Gm::SROW);  // [64][PROW]
  float* alpha = reinterpret_cast<float*>(Pl + 64 * Gm::PROW);         // [64]
  float* rowm = alpha + 64;                                             // [64]
  float* rowl = rowm + 64;                                              // [64]
  int* tags = reinterpret_cast<int*>(rowl + 64);                        // [32]

  __shared__ double freq[kMaxRopePairs];
  __shared__ float2 qcs[4][kMaxRopePairs];     // (cos, sin) of t_g * freq_p, g < G

  const int tid = threadIdx.x;
  const int wave = tid >> 6, l = tid & 63, hf = l >> 5, ln = l & 31;
  const Work w = make_work(a, blockIdx.y);
  const int split = blockIdx.x;
  const int64_t e_lo = (int64_t)split * a.chunk;
  const int64_t e_hi = min(w.n_tot, e_lo + a.chunk);
  const int nope = a.D - a.r;
  const int npair = a.r / 2;

  rope_freq_table(freq, a.r, a.theta);
  __syncthreads();
  for (int e = tid; e < a.G * npair; e += blockDim.x) {
    const int g = e / npair, p = e - g * npair;
    float cs, sn;
    rope_cos_sin((double)(w.t_first + g), freq[p], &cs, &sn);
    qcs[g][p] = make_float2(cs, sn);
  }
  __syncthreads();

  // ---- query fragments (rotated at t), rows rt*32 + ln, dims wave*DW + s*16 + hf*8
  bf16x8 qf[2][Gm::KQ];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = rt * 32 + ln;
    const int g = row / a.Hs, h = w.h0 + row % a.Hs;
    const bool live = g < w.n_q;
    const __bf16* qp = static_cast<const __bf16*>(a.q) +
                       (((int64_t)w.b * a.Tq + w.i0 + (live ? g : 0)) * a.H + h) * D;
#pragma unroll
    for (int s = 0; s < Gm::KQ; ++s) {
      const int c0 = wave * Gm::DW + s * 16 + hf * 8;
      uint4 raw = live ? *reinterpret_cast<const uint4*>(qp + c0) : make_uint4(0, 0, 0, 0);
      if (c0 >= nope && live) {
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float2 cv = qcs[g][(c0 - nope) / 2 + p];
          const float cs = cv.x, sn = cv.y;
          const float x0 = bf16_to_f32(wd[p] & 0xffffu), x1 = bf16_to_f32(wd[p] >> 16);
          o[p] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
        }
        raw = make_uint4(o[0], o[1], o[2], o[3]);
      }
      qf[rt][s] = *reinterpret_cast<bf16x8*>(&raw);
    }
  }

  // ---- running softmax state: thread (row = tid/4, part = tid%4)
  const int srow = tid >> 2, spart = tid & 3;
  const int sg = srow / a.Hs;
  float m_run = -INFINITY, l_run = 0.f;

  f32x16 oacc[2][Gm::DT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < Gm::DT; ++dt) oacc[rt][dt] = f32x16{};

  const int st_e = tid >> 3, st_part = tid & 7;
  Stage<D, KV> stage;
  int st_tag = 0;
  {
    const uint8_t* src = e_lo + st_e < e_hi ? entry_src(a, w, e_lo + st_e, &st_tag) : nullptr;
    if (e_lo + st_e >= e_hi) st_tag = -0x7fffffff;
    stage_load<D, KV>(src, st_part, nope, stage);
  }

  for (int64_t base = e_lo; base < e_hi; base += 32) {
    __syncthreads();   // previous tile fully consumed
    stage_store<D, KV>(Et + st_e * Gm::EROW, st_part, nope, stage);
    if (st_part == 0) tags[st_e] = st_tag;
    __syncthreads();
    // prefetch the next tile while this one is used
    if (base + 32 < e_hi) {
      const int64_t e = base + 32 + st_e;
      const uint8_t* src = e < e_hi ? entry_src(a, w, e, &st_tag) : nullptr;
      if (e >= e_hi) st_tag = -0x7fffffff;
      stage_load<D, KV>(src, st_part, nope, stage);
    }

    // ---- QK on this wave's quarter of D
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x16 sacc = {};
#pragma unroll
      for (int s = 0; s < Gm::KQ; ++s) {
        const bf16x8 ef = *reinterpret_cast<const bf16x8*>(
            Et + ln * Gm::EROW + 2 * (wave * Gm::DW + s * 16 + hf * 8));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[rt][s], ef, sacc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) Sp[((wave * 2 + rt) * 16 + v) * Gm::SROW + l] = sacc[v];
    }
    __syncthreads();

    // ---- online softmax: thread owns row srow, entries spart*8 .. +8
    {
      const int rt = srow >> 5, rem = srow & 31;
      const int v = 4 * (rem >> 3) + (rem & 3), shf = (rem >> 2) & 1;
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = 0.f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        const float* src = Sp + ((wv * 2 + rt) * 16 + v) * Gm::SROW + shf * 32 + spart * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] += src[e];
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool vis = entry_visible(a, w, tags[spart * 8 + e], sg);
        sv[e] = vis ? sv[e] * a.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[e]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 1));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 2));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float al = exp2f(m_run - m_use);
      float psum = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = exp2f(sv[e] - m_use), p1 = exp2f(sv[e + 1] - m_use);
        psum += p0 + p1;
        pk[e / 2] = pack_bf16x2(p0, p1);
      }
      psum += __shfl_xor(psum, 1);
      psum += __shfl_xor(psum, 2);
      l_run = l_run * al + psum;
      m_run = m_new;
      *reinterpret_cast<uint4*>(Pl + srow * Gm::PROW + spart * 8) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      if (spart == 0) alpha[srow] = al;
    }
    __syncthreads();

    // ---- rescale and PV on this wave's quarter of the output columns
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float al[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) al[v] = alpha[rt * 32 + 8 * (v >> 2) + 4 * hf + (v & 3)];
#pragma unroll
      for (int dt = 0; dt < Gm::DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[rt][dt][v] *= al[v];
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 pf[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        pf[rt] = *reinterpret_cast<const bf16x8*>(Pl + (rt * 32 + ln) * Gm::PROW + s * 16 + hf * 8);
#pragma unroll
      for (int dt = 0; dt < Gm::DT; ++dt) {
        const int col = wave * Gm::DW + dt * 32 + ln;
        const uint8_t* ep = Et + (s * 16 + hf * 8) * Gm::EROW + 2 * col;
        uint32_t u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = *reinterpret_cast<const uint16_t*>(ep + (2 * i) * Gm::EROW);
          const uint32_t hi = *reinterpret_cast<const uint16_t*>(ep + (2 * i + 1) * Gm::EROW);
          u[i] = lo | (hi << 16);
        }
        uint4 uv = make_uint4(u[0], u[1], u[2], u[3]);
        const bf16x8 ef = *reinterpret_cast<bf16x8*>(&uv);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          oacc[rt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[rt], ef, oacc[rt][dt], 0, 0, 0);
      }
    }
  }

  // ---- row statistics to LDS for the epilogue
  __syncthreads();
  if (spart == 0) { rowm[srow] = m_run; rowl[srow] = l_run; }
  __syncthreads();

  if (a.nsplit > 1) {
    const int64_t slot = (int64_t)blockIdx.y * a.nsplit + split;
    float* po = a.part_o + slot * 64 * D;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int dt = 0; dt < Gm::DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = rt * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
          po[row * D + wave * Gm::DW + dt * 32 + ln] = oacc[rt][dt][v];
        }
    if (tid < 64) {
      a.part_ml[(slot * 64 + tid) * 2] = rowm[tid];
      a.part_ml[(slot * 64 + tid) * 2 + 1] = rowl[tid];
    }
    return;
  }

  // ---- single split: normalise, rotate back at -t, store bf16
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = rt * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
      const int g = row / a.Hs, h = w.h0 + row % a.Hs;
      const bool live = g < w.n_q;
      const float mr = rowm[row];
      float den = rowl[row];
      if (a.sink) den += exp2f(a.sink[h] * 1.4426950408889634f - (mr == -INFINITY ? 0.f : mr));
      const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
      for (int dt = 0; dt < Gm::DT; ++dt) {
        const int col = wave * Gm::DW + dt * 32 + ln;
        float o = oacc[rt][dt][v] * inv;
        const float partner = __shfl_xor(o, 1);
        if (col >= nope) {            // rotation at -t: (cos, -sin) of the query's angle
          const float2 cv = qcs[g < 4 ? g : 0][(col - nope) >> 1];
          const float cs = cv.x, sn = -cv.y;
          o = (col & 1) ? partner * sn + o * cs : o * cs - partner * sn;
        }
        if (live) {
          uint16_t* op = static_cast<uint16_t*>(a.out) + (((int64_t)w.b * a.Tq + w.i0 + g) * a.H + h) * D + col;
          *op = (uint16_t)f32_to_bf16(o);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- combine
__global__ void __launch_bounds__(256) combine_kernel(KArgs a) {
  __shared__ float wgt[1024];
  __shared__ float red[2];
  __shared__ double freq[kMaxRopePairs];
  rope_freq_table(freq, a.r, a.theta);
  __syncthreads();
  const int work = blockIdx.x / 64, row = blockIdx.x % 64;
  const Work w = make_work(a, work);
  const int g = row / a.Hs, h = w.h0 + row % a.Hs;
  if (g >= w.n_q) return;
  const int64_t slot0 = (int64_t)work * a.nsplit;
  if (threadIdx.x < 64) {
    float M = -INFINITY;
    for (int s = threadIdx.x; s < a.nsplit; s += 64) M = fmaxf(M, a.part_ml[((slot0 + s) * 64 + row) * 2]);
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float sink2 = a.sink ? a.sink[h] * 1.4426950408889634f : -INFINITY;
    M = fmaxf(M, sink2);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    for (int s = threadIdx.x; s < a.nsplit; s += 64) {
      const float ms = a.part_ml[((slot0 + s) * 64 + row) * 2];
      const float ls = a.part_ml[((slot0 + s) * 64 + row) * 2 + 1];
      const float f = exp2f(ms - Mu);
      wgt[s] = f;
      L += ls * f;
    }
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    if (threadIdx.x == 0) {
      if (a.sink) L += exp2f(sink2 - Mu);
      red[0] = L > 0.f ? 1.f / L : 0.f;
    }
  }
  __syncthreads();
  const float inv = red[0];
  const int64_t t = w.t_first + g;
  const int nope = a.D - a.r;
  uint16_t* op = static_cast<uint16_t*>(a.out) + (((int64_t)w.b * a.Tq + w.i0 + g) * a.H + h) * a.D;
  for (int c = 2 * threadIdx.x; c < a.D; c += 2 * blockDim.x) {
    float o0 = 0.f, o1 = 0.f;
    for (int s = 0; s < a.nsplit; ++s) {
      const float f = wgt[s];
      if (f == 0.f) continue;
      const float2 x = *reinterpret_cast<const float2*>(a.part_o + ((slot0 + s) * 64 + row) * a.D + c);
      o0 += f * x.x;
      o1 += f * x.y;
    }
    o0 *= inv;
    o1 *= inv;
    if (c >= nope) {
      float cs, sn;
      rope_cos_sin(-(double)t, freq[(c - nope) >> 1], &cs, &sn);
      const float r0 = o0 * cs - o1 * sn, r1 = o0 * sn + o1 * cs;
      o0 = r0;
      o1 = r1;
    }
    *reinterpret_cast<uint32_t*>(op + c) = pack_bf16x2(o0, o1);
  }
}

// ---------------------------------------------------------------- float32 VALU path
// One workgroup per query; H*D <= 8192, D <= 256.
__global__ void __launch_bounds__(256) attend_f32_kernel(KArgs a) {
  extern __shared__ float fsm[];
  __shared__ double freq[kMaxRopePairs];
  rope_freq_table(freq, a.r, a.theta);
  const int H = a.H, D = a.D;
  float* qs = fsm;                    // [H][D]
  float* es = qs + H * D;             // [32][D]
  float* lg = es + 32 * D;            // [H][32]
  float* mrow = lg + H * 32;          // [H]
  float* lrow = mrow + H;             // [H]
  float* al = lrow + H;               // [H]
  int* tags = reinterpret_cast<int*>(al + H);   // [32]
  const int tid = threadIdx.x;
  const Work w = make_work(a, blockIdx.x);      // G = 1, one query
  const int64_t t = w.t_first;
  const int nope = D - a.r;
  const float* q = static_cast<const float*>(a.q) + ((int64_t)w.b * a.Tq + w.i0) * H * D;
  for (int e = tid; e < H * D; e += blockDim.x) qs[e] = q[e];
  for (int h = tid; h < H; h += blockDim.x) { mrow[h] = -INFINITY; lrow[h] = 0.f; }
  __syncthreads();
  for (int e = tid; e < H * (a.r / 2); e += blockDim.x) {
    const int h = e / (a.r / 2), p = e % (a.r / 2);
    float cs, sn;
    rope_cos_sin((double)t, freq[p], &cs, &sn);
    float* v = qs + h * D + nope + 2 * p;
    const float x0 = v[0], x1 = v[1];
    v[0] = x0 * cs - x1 * sn;
    v[1] = x0 * sn + x1 * cs;
  }
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  for (int64_t base = 0; base < w.n_tot; base += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * D; e += blockDim.x) {
      const int ei = e / D, c = e % D;
      int tag;
      const uint8_t* src = entry_src(a, w, base + ei, &tag);
      es[e] = src ? reinterpret_cast<const float*>(src)[c] : 0.f;
      if (c == 0) tags[ei] = tag;
    }
    __syncthreads();
    for (int e = tid; e < H * 32; e += blockDim.x) {
      const int h = e / 32, ei = e % 32;
      float dot = 0.f;
      for (int c = 0; c < D; ++c) dot = fmaf(qs[h * D + c], es[ei * D + c], dot);
      lg[e] = entry_visible(a, w, tags[ei], 0) ? dot * a.scale_log2 : -INFINITY;
    }
    __syncthreads();
    for (int h = tid; h < H; h += blockDim.x) {
      float tmax = -INFINITY;
      for (int ei = 0; ei < 32; ++ei) tmax = fmaxf(tmax, lg[h * 32 + ei]);
      const float m_new = fmaxf(mrow[h], tmax);
      const float mu = m_new == -INFINITY ? 0.f : m_new;
      float s = 0.f;
      for (int ei = 0; ei < 32; ++ei) {
        const float p = exp2f(lg[h * 32 + ei] - mu);
        lg[h * 32 + ei] = p;
        s += p;
      }
      al[h] = exp2f(mrow[h] - mu);
      lrow[h] = lrow[h] * al[h] + s;
      mrow[h] = m_new;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int e = tid + i * 256;
      if (e < H * D) {
        const int h = e / D, c = e % D;
        float v = acc[i] * al[h];
        for (int ei = 0; ei < 32; ++ei) v = fmaf(lg[h * 32 + ei], es[ei * D + c], v);
        acc[i] = v;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int e = tid + i * 256;
    if (e < H * D) {
      const int h = e / D;
      const float mu = mrow[h] == -INFINITY ? 0.f : mrow[h];
      float den = lrow[h];
      if (a.sink) den += exp2f(a.sink[h] * 1.4426950408889634f - mu);
      qs[e] = den > 0.f ? acc[i] / den : 0.f;
    }
  }
  __syncthreads();
  for (int e = tid; e < H * (a.r / 2); e += blockDim.x) {
    const int h = e / (a.r / 2), p = e % (a.r / 2);
    float cs, sn;
    rope_cos_sin(-(double)t, freq[p], &cs, &sn);
    float* v = qs + h * D + nope + 2 * p;
    const float x0 = v[0], x1 = v[1];
    v[0] = x0 * cs - x1 * sn;
    v[1] = x0 * sn + x1 * cs;
  }
  __syncthreads();
  float* out = static_cast<float*>(a.out) + ((int64_t)w.b * a.Tq + w.i0) * H * D;
  for (int e = tid; e < H * D; e += blockDim.x) out[e] = qs[e];
}

template <int D, int KV>
hipError_t launch_mfma(const KArgs& k, const AttnPlan& p, hipStream_t st) {
  using Gm = Geo<D>;
  const size_t lds = 32 * Gm::EROW + 4 * 2 * 16 * Gm::SROW * 4 + 64 * Gm::PROW * 2 + 3 * 64 * 4 + 32 * 4;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&attend_mfma_kernel<D, KV>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  {
    TimedLaunch tl(kKernelAttend, st);
    hipLaunchKernelGGL((attend_mfma_kernel<D, KV>), dim3(p.nsplit, p.n_work), dim3(256), lds, st, k);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  TimedLaunch tl(kKernelCombine, st);
  hipLaunchKernelGGL(combine_kernel, dim3(p.n_work * 64), dim3(256), 0, st, k);
  return hipGetLastError();
}

}  // namespace

size_t attend_workspace_bytes(int B, int Tq, int H, int D, int r, int kv_fmt, int n_entries, int W) {
  return make_plan(B, Tq, H, D, r, kv_fmt, n_entries, W, kv_fmt == kF32).total;
}

hipError_t launch_attend(const AttendArgs& a, void* ws, hipStream_t st) {
  const bool f32 = a.kv_fmt == kF32;
  const AttnPlan p = make_plan(a.B, a.Tq, a.H, a.D, a.r, a.kv_fmt, a.n_entries, a.W, f32);
  if (a.B == 0 || a.Tq == 0) return hipSuccess;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  hipError_t e;
  if (a.W > 0) {
    WinArgs wa{};
    wa.raw = static_cast<const uint8_t*>(a.raw);
    wa.win = w8 + p.off_win;
    wa.fmt = a.kv_fmt; wa.B = a.B; wa.D = a.D; wa.r = a.r; wa.Tq = a.Tq; wa.W = a.W;
    wa.T_raw = a.T_raw; wa.win_rows = p.win_rows; wa.row_bytes = p.row_bytes; wa.theta = a.theta;
    wa.qpos = a.qpos; wa.rawpos = a.rawpos;
    const int64_t n = (int64_t)a.B * p.win_rows * (a.D / 8);
    hipLaunchKernelGGL(rope_window_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, wa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  KArgs k{};
  k.q = a.q; k.kv = static_cast<const uint8_t*>(a.kv); k.idx = a.idx; k.win = w8 + p.off_win;
  k.sink = a.sink; k.out = a.out;
  k.part_o = p.nsplit > 1 ? reinterpret_cast<float*>(w8 + p.off_po) : nullptr;
  k.part_ml = p.nsplit > 1 ? reinterpret_cast<float*>(w8 + p.off_pml) : nullptr;
  k.mode = a.mode; k.N = a.N; k.k = a.k; k.m = a.m; k.W = a.W; k.B = a.B; k.Tq = a.Tq;
  k.H = a.H; k.D = a.D; k.r = a.r; k.theta = a.theta;
  k.scale_log2 = a.scale * 1.4426950408889634f;
  k.G = p.G; k.Hs = p.Hs; k.n_htiles = p.n_htiles; k.n_qgroups = p.n_qgroups;
  k.nsplit = p.nsplit; k.chunk = p.chunk; k.win_rows = p.win_rows; k.row_bytes = p.row_bytes;
  k.qpos = a.qpos;
  if (f32) {
    const size_t lds = ((size_t)a.H * a.D + 32 * a.D + a.H * 32 + 3 * a.H) * 4 + 32 * 4;
    TimedLaunch tl(kKernelAttend, st);
    hipLaunchKernelGGL(attend_f32_kernel, dim3(p.n_work), dim3(256), lds, st, k);
    return hipGetLastError();
  }
  if (a.kv_fmt == kBF16) {
    if (a.D == 128) return launch_mfma<128, kBF16>(k, p, st);
    if (a.D == 256) return launch_mfma<256, kBF16>(k, p, st);
    return launch_mfma<512, kBF16>(k, p, st);
  }
  if (a.D == 128) return launch_mfma<128, kMixed>(k, p, st);
  if (a.D == 256) return launch_mfma<256, kMixed>(k, p, st);
  return launch_mfma<512, kMixed>(k, p, st);
}

}  // namespace lac
