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
#include <algorithm>
#include <type_traits>

#include <vector>

#include "lac_internal.h"

namespace lac {

namespace {

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

constexpr int kIdxLds = 2304;   // CSA indices of a split staged in LDS
constexpr int kTile = 32;       // entries per attention tile
constexpr int kGridTarget = 256;   // blocks per launch the split count aims at

__host__ __device__ inline int64_t kv_row_bytes(int fmt, int D, int r) {
  return fmt == kF32 ? 4LL * D : fmt == kBF16 ? 2LL * D : (int64_t)D + r;
}

// ---------------------------------------------------------------- plan
struct AttnPlan {
  int G, Hs, n_htiles, n_qgroups, n_work, nsplit, chunk, wchunk, max_entries;
  int64_t win_rows, row_bytes, win_row_bytes;
  size_t off_zero, off_win, off_ang, off_po, off_pml, total;
};

// Low parts of rotated window dims.  A window row rotated at its position is
// rounded to bf16 for the matrix cores; its dims from lo_base = D - R32 on
// (R32 = r rounded up to 32) also keep the residual x - bf16(x) as a second
// bf16 value, and the tiles holding window rows add that part's products,
// so the rotation adds no rounding beyond the bf16 storage of the raw row.
__host__ __device__ inline int lo_dims(int r) { return (r + 31) / 32 * 32; }
constexpr int kLoRow = 2 * 128 + 16;          // LDS bytes per staged low row (R32 <= 128)

// shared_entries: the G queries of a work item see one common run of compressed
// entries (HCA's causal prefix) rather than G separate selections (CSA).
AttnPlan make_plan(int B, int Tq, int H, int D, int r, int kv_fmt, int n_entries, int W,
                   bool f32_path, bool shared_entries, int grid_target = kGridTarget) {
  AttnPlan p{};
  p.row_bytes = kv_row_bytes(kv_fmt, D, r);
  p.win_rows = W > 0 ? (int64_t)Tq + W - 1 : 0;
  size_t off = 0;
  p.off_zero = off;
  off += 256;
  // pre-rotated window rows (bf16 and mixed formats) carry their low parts
  // after the row: R32 bf16 values for dims lo_base .. D-1
  p.win_row_bytes = p.row_bytes + (f32_path ? 0 : 2 * lo_dims(r));
  p.off_win = off;
  off += round_up((int64_t)B * p.win_rows * p.win_row_bytes, 256);
  p.off_ang = off;
  off += round_up((int64_t)B * Tq * (r / 2) * 8, 256);
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
  p.max_entries = (shared_entries ? n_entries : p.G * n_entries) + (W > 0 ? W + p.G - 1 : 0);
  if (p.max_entries < 1) p.max_entries = 1;
  // One block fills a compute unit's LDS, so the grid is sized to one wave of
  // blocks over the 256 compute units; a split holds at least 2 tiles.
  const int max_split = (int)((p.max_entries + 63) / 64);
  int ns = p.n_work >= grid_target ? 1 : grid_target / p.n_work;
  if (ns > max_split) ns = max_split;
  if (ns < 1) ns = 1;
  p.chunk = (int)round_up((p.max_entries + ns - 1) / ns, 32);
  if (p.chunk > kIdxLds) p.chunk = kIdxLds;    // a split's CSA indices fit in LDS
  p.nsplit = (p.max_entries + p.chunk - 1) / p.chunk;
  int ns_alloc = p.nsplit;
  if (p.nsplit > 1 && W > 0) {
    // Split-K with a window: the window rows (rotated in the kernel, with
    // low parts) get splits of one tile each after the compressed entries'
    // splits, so that their extra work does not lengthen the longest split
    // -- while the launch stays within one wave of blocks over the chip;
    // beyond that the extra splits would start a second wave, and the
    // window rows stay in the last splits of the entry list.  The partials
    // are sized for the window splits, the most any target plans.
    const int n_comp_max = p.max_entries - (W + p.G - 1);
    const int n_win_max = W + p.G - 1;
    const int ns_w = (n_comp_max + p.chunk - 1) / p.chunk + (n_win_max + kTile - 1) / kTile;
    ns_alloc = std::max(ns_alloc, ns_w);
    if ((int64_t)p.n_work * ns_w <= kGridTarget) {
      p.wchunk = kTile;
      p.nsplit = ns_w;
    }
  }
  if (ns_alloc > 1) {
    p.off_po = off;
    off += round_up((int64_t)p.n_work * ns_alloc * 64 * D * 2, 256);
    p.off_pml = off;
    off += round_up((int64_t)p.n_work * ns_alloc * 64 * 2 * 4, 256);
  }
  p.total = off;
  return p;
}

// ---------------------------------------------------------------- window rotation
struct WinArgs {
  const uint8_t* raw;
  uint8_t* win;              // [B, win_rows, win_row_bytes]
  uint8_t* zero_row;
  float2* ang;               // [B, Tq, r/2] (cos, sin) of each query position's angles
  int64_t n_win_items;       // window work items (D/8 per row); angle items follow
  int fmt, B, D, r, Tq, W;
  int64_t T_raw, win_rows, row_bytes, win_row_bytes;
  RopeTable rope;
  Positions qpos, rawpos;
};

__global__ void __launch_bounds__(256) rope_window_kernel(WinArgs a) {
  __shared__ double freq[kMaxRopePairs];
  rope_freq_table(freq, a.rope, a.r, threadIdx.x, 256);
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x < 4) reinterpret_cast<uint32_t*>(a.zero_row)[threadIdx.x] = 0u;
  const int G8 = a.D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.n_win_items) {            // angle table of the query positions
    const int np = a.r / 2;
    const int64_t j = gid - a.n_win_items;
    if (np == 0 || j >= (int64_t)a.B * a.Tq * np) return;
    const int64_t qrow = j / np;
    const int p = (int)(j - qrow * np);
    const int b = (int)(qrow / a.Tq);
    float cs, sn;
    rope_cos_sin((double)((int64_t)a.qpos.v[b] + (qrow - (int64_t)b * a.Tq)), freq[p], &cs, &sn);
    a.ang[j] = make_float2(cs, sn);
    return;
  }
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
  uint8_t* dst = a.win + ((int64_t)b * a.win_rows + row) * a.win_row_bytes;
  const int c0 = g * 8, nope = a.D - a.r;
  const int lo_base = a.D - lo_dims(a.r);
  uint16_t* lrow = reinterpret_cast<uint16_t*>(dst + a.row_bytes);    // the row's low parts
  if (a.fmt != kF32 && c0 >= lo_base && c0 < nope)     // no low part below the rotated dims
    *reinterpret_cast<uint4*>(lrow + (c0 - lo_base)) = make_uint4(0u, 0u, 0u, 0u);
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
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) split_bf16x2(v[2 * q], v[2 * q + 1], &hw[q], &lw[q]);
    reinterpret_cast<uint2*>(dst + off)[0] = make_uint2(hw[0], hw[1]);
    reinterpret_cast<uint2*>(dst + off)[1] = make_uint2(hw[2], hw[3]);
    *reinterpret_cast<uint4*>(lrow + (c0 - lo_base)) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
}

// ---------------------------------------------------------------- entry lists
struct KArgs {
  const void* q;
  const uint8_t* kv;
  const int32_t* idx;
  const uint8_t* win;        // pre-rotated window rows, win_row_bytes each
  const float* sink;
  void* out;
  uint16_t* part_o;         // [work, split, 64, D] bf16 partial outputs / their row sums
  float* part_ml;
  const uint8_t* zero_row;   // 16 zero bytes in workspace (f32 path)
  const float2* ang;         // [B, Tq, r/2] (cos, sin) of the query angles (f32 path)
  const uint8_t* raw;        // [B, T_raw, row] raw window rows, not rotated
  int64_t T_raw;
  int win_rotated;           // window rows come pre-rotated from `win` (prefill)
  int mode, N, k, m, W, B, Tq, H, D, r;
  float theta, scale_log2;
  int G, Hs, n_htiles, n_qgroups, n_work, nsplit, chunk, wchunk;
  int64_t win_rows, row_bytes, win_row_bytes;
  int pos_q, pos_raw;        // q_pos0 and raw_pos0 in the launch's position pool
  const float* q_norm_gain;  // [D] or null: RMSNorm of each query head before its rotation
  float norm_eps;
};

// One launch: up to kAttendGroup independent calls whose workgroups follow
// one another (a call's are work-major, split fastest), their positions in
// one pool and one rotation table shared by all of them, so that the whole
// launch fits one kernel argument.
constexpr int kAttendGroup = 4;
constexpr int kAttendPos = 384;

struct KLaunch {
  KArgs k[kAttendGroup];
  uint32_t blk_end[kAttendGroup];   // workgroups of calls 0 .. i
  int n;
  int32_t pos[kAttendPos];
  double freq[kMaxRopePairs];
};

// A launch's whole argument is one kernel argument: keep it within 4 KB.
static_assert(sizeof(KLaunch) <= 4096, "kernel argument above 4 KB");

// The call that workgroup wg belongs to, and wg's index within that call.
__device__ __forceinline__ int launch_call(const KLaunch& L, uint32_t wg, uint32_t* local) {
  int ci = 0;
  while (ci + 1 < L.n && wg >= L.blk_end[ci]) ++ci;
  *local = wg - (ci ? L.blk_end[ci - 1] : 0u);
  return ci;
}

__device__ __forceinline__ void launch_freq_table(double* tab, const KLaunch& L, int r, int tid,
                                                  int nthreads) {
  for (int i = tid; i < r / 2; i += nthreads) tab[i] = L.freq[i];
}

// Work item decomposition: blockIdx.x = split (fastest), blockIdx.y = work.
struct Work {
  int b, i0, h0, n_q;       // queries i0 .. i0+n_q-1, heads h0 ..
  int64_t t_first;
  int n_comp, n_tot;        // compressed entries, all entries of the list
  int64_t lo_w;             // first window position of the list
  int64_t win_row0;         // its row in the rotated-window buffer
};

// (A launch of one call has its q_pos0 at the start of the position pool.)
template <bool MULTI = true>
__device__ __forceinline__ Work make_work(const KLaunch& L, const KArgs& a, int work) {
  Work w;
  const int ht = work % a.n_htiles;
  const int rest = work / a.n_htiles;
  const int qg = rest % a.n_qgroups;
  w.b = rest / a.n_qgroups;
  w.i0 = qg * a.G;
  w.h0 = ht * 64;
  w.n_q = min(a.G, a.Tq - w.i0);
  const int64_t qpos = L.pos[(MULTI ? a.pos_q : 0) + w.b];
  w.t_first = qpos + w.i0;
  const int64_t t_last = w.t_first + w.n_q - 1;
  w.n_comp = a.mode == 0 ? w.n_q * a.k : (int)n_visible(t_last, a.N, a.m);
  w.lo_w = max((int64_t)0, w.t_first - a.W + 1);
  w.win_row0 = w.lo_w - max((int64_t)0, qpos - a.W + 1);
  const int n_win = a.W > 0 ? (int)(t_last - w.lo_w + 1) : 0;
  w.n_tot = w.n_comp + n_win;
  return w;
}

// Entry tags: CSA compressed entry selected by query g -> g; HCA compressed
// entry j -> -1 - j; window entry at position lo_w + off -> 1 << 30 | off;
// an empty slot -> kNoEntry.
constexpr int kNoEntry = INT32_MIN;
constexpr int kWinTag = 1 << 30;

// Per-query visibility of the work item, from which every (query, entry)
// test is a pair of int32 compares.
struct Vis {
  int nv;          // HCA: compressed entries visible to the query
  int wlo, whi;    // window offsets (relative to lo_w) visible to the query
};

__device__ __forceinline__ Vis make_vis(const KArgs& a, const Work& w, int g) {
  Vis v;
  if (g >= w.n_q) { v.nv = 0; v.wlo = 1; v.whi = 0; return v; }
  const int64_t t = w.t_first + g;
  v.nv = a.mode == 1 ? (int)n_visible(t, a.N, a.m) : 0;
  v.wlo = (int)max((int64_t)0, t - a.W + 1 - w.lo_w);
  v.whi = (int)(t - w.lo_w);
  if (a.W == 0) { v.wlo = 1; v.whi = 0; }
  return v;
}

__device__ __forceinline__ bool visible(int tag, int g, const Vis& v) {
  const int off = tag - kWinTag;
  const bool win = tag >= kWinTag && off >= v.wlo && off <= v.whi;
  const bool sel = tag >= 0 && tag < kWinTag && tag == g;
  const bool dense = tag < 0 && tag != kNoEntry && -1 - tag < v.nv;
  return win | sel | dense;
}

// Entry e of the work list -> source row (null if it names nothing) and tag.
// With from_lds, the CSA index of entry e is lidx[e - e_lo] (LDS).
__device__ __forceinline__ const uint8_t* entry_src(const KArgs& a, const Work& w, int e,
                                                    bool from_lds, const int32_t* lidx, int e_lo,
                                                    int* tag) {
  if (e >= w.n_tot) { *tag = kNoEntry; return nullptr; }
  if (e < w.n_comp) {
    int j;
    if (a.mode == 0) {
      const int g = a.G == 1 ? 0 : e / a.k;
      if (from_lds)
        j = lidx[e - e_lo];
      else
        j = *(const __attribute__((address_space(1))) int32_t*)(
            a.idx + ((int64_t)w.b * a.Tq + w.i0 + g) * a.k + (e - g * a.k));
      if (j < 0 || j >= a.N) { *tag = kNoEntry; return nullptr; }
      *tag = g;
    } else {
      j = e;
      *tag = -1 - j;
    }
    return a.kv + ((int64_t)w.b * a.N + j) * a.row_bytes;
  }
  const int off = e - w.n_comp;
  *tag = kWinTag | off;
  return a.win + ((int64_t)w.b * a.win_rows + w.win_row0 + off) * a.win_row_bytes;
}

// ---------------------------------------------------------------- MFMA attention

// ---- tile loop
// A block holds 64 query rows (G tokens x Hs heads) and eight waves: wave w
// owns rows 16 (w % 4) .. +15 and half of D (w / 4), so two waves share each
// row group.  The products run transposed, on v_mfma_f32_16x16x32_bf16:
//   S^T[e][r] = sum_d E[e][d] Q[r][d]: A = entry rows read from LDS, B = the
//     wave's rotated query slices (its half of D) kept in VGPRs; the two
//     halves' partial logits are summed through LDS, after which both waves
//     of a row group run the same online softmax;
//   O^T[d][r] += sum_e E^T[d][e] P^T[e][r] over the wave's half of D: B = the
//     S^T accumulators themselves (exp'd, packed to bf16 -- a lane holds row
//     r = lane % 16 and entries {4q..4q+3, 16+4q..16+4q+3}, q = lane / 16,
//     which is a valid K order because the A side uses the same order),
//     A = E^T read with ds_read_b64_tr_b16 (a 16-lane group's transposed
//     4 x 16 block).
// Splitting D halves each wave's query and output registers, so two waves
// run per SIMD and hide each other's LDS and MFMA latency.  A lane keeps one
// row's running max (shared by its four lanes) and a partial row sum.  The
// max used for the exponentials moves only when a logit exceeds it by more
// than 2^8 (log2 domain), so the accumulators are rescaled rarely;
// probabilities up to 2^8 are exact enough in bf16 and the final division
// by the row sum (taken with the same max) is unchanged.  Tiles of 32
// entries are gathered into VGPRs one tile ahead (16 threads per row,
// uniform 16-byte loads), written to one of two LDS buffers as bf16 rows
// (E4M3 widened by the hardware converter; window rows rotated here in
// decode), and a barrier publishes them.

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Max over lanes l, l^16, l^32, l^48 (the four lanes that hold one row), by
// the cross-lane swaps of 16-lane rows and 32-lane halves.
__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ bf16x4 ds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}

template <int D>
struct Geo {
  static constexpr int DS = D >= 256 ? 2 : 1;   // waves sharing a row group (D split)
  static constexpr int NT = 256 * DS;            // threads per block
  static constexpr int DW = D / DS;              // dims per wave
  static constexpr int EROW = 2 * D + 16;        // LDS bytes per staged entry
  static constexpr int KH = DW / 32;             // QK k-steps per wave
  static constexpr int DH = DW / 16;             // PV output tiles per wave
  static constexpr int TPR = 8 * DS;             // staging threads per entry row
  static constexpr int NCH = D / 8 / TPR;        // 16-byte chunks per staging thread, bf16 rows
  static constexpr int NCHM = (D / 16 + 8 + TPR - 1) / TPR;   // mixed rows (<= D/16 + 8 chunks)
  static constexpr int NLO = (16 + TPR - 1) / TPR;            // low-part chunks (<= 16 per row)
};

// MULTI false: a launch of one call, grid (splits, work items).  MULTI true:
// a flat grid of several calls' workgroups (KLaunch).
template <int D, int KV, bool MULTI>
__global__ void __launch_bounds__(512) attend_mfma_kernel(KLaunch L) {
  using Gm = Geo<D>;
  constexpr int DS = Gm::DS, NT = Gm::NT, TPR = Gm::TPR;
  __shared__ __align__(16) uint8_t Et[2][kTile * Gm::EROW];     // entry tiles, bf16 rows
  __shared__ __align__(16) uint8_t Elo[2][kTile * kLoRow];      // low parts, dims lo_base..D-1
  // Per entry: the first query slot of the block that sees it and the span of
  // slots after it that do (an empty slot has first = 64, which no slot
  // reaches), so a (row, entry) visibility test is one unsigned compare.
  __shared__ __align__(16) int vis_lo[2][kTile];
  __shared__ __align__(16) int vis_span[2][kTile];
  __shared__ __align__(16) float Sx[DS][4][64][8];             // partial logits [half][group][lane]
  __shared__ float qss[DS][64];              // query RMSNorm: each D part's sum of squares per row
  __shared__ int32_t lidx[kIdxLds];
  __shared__ double freq[kMaxRopePairs];
  extern __shared__ float2 qang[];            // [G][r/2] (cos, sin) of t_g * freq_p

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 3, dh = DS == 2 ? wave >> 2 : 0;
  const int l = tid & 63, lr = l & 15, lq = l >> 4;
  // Entry rows of each 16-row half of a tile are read in the order
  // rho(v) = 2 (v mod 8) + v / 8: the QK operand lane lr reads row rho(lr)
  // and the transposed PV read of lane (lr, lq) row rho(4 lq + lr / 4).  The
  // 16 rows of a 16-lane 16-byte read still hit 16 different 16-byte bank
  // groups (row stride = 16 mod 256 bytes), and the 8 rows of a 32-lane
  // transposed read (32 bytes each) now lie 32 bytes apart, so neither
  // conflicts.  The softmax lane then holds entries rho(4 lq + i) (+ 16):
  // the staging writes each entry's visibility at position rho^-1(row).
  const int q_row = ((lr & 7) << 1) | (lr >> 3);
  const int pv_v = 4 * lq + (lr >> 2);
  const int pv_row = ((pv_v & 7) << 1) | (pv_v >> 3);
  uint32_t lb = 0;
  const int ci = MULTI ? launch_call(L, blockIdx.x, &lb) : 0;
  const KArgs& a = L.k[ci];
  const int work = MULTI ? (int)(lb / (uint32_t)a.nsplit) : (int)blockIdx.y;
  const int split = MULTI ? (int)(lb % (uint32_t)a.nsplit) : (int)blockIdx.x;
  const Work w = make_work<MULTI>(L, a, work);
  // Split -> entry range: chunk entries per split, or, with wchunk, chunk
  // entries per split over the compressed entries and then wchunk per split
  // over the window rows.
  int e_lo, e_hi;
  {
    const int ns_c = a.wchunk > 0 ? (w.n_comp + a.chunk - 1) / a.chunk : 1 << 30;
    if (split < ns_c) {
      e_lo = split * a.chunk;
      e_hi = min(a.wchunk > 0 ? w.n_comp : w.n_tot, e_lo + a.chunk);
    } else {
      e_lo = w.n_comp + (split - ns_c) * a.wchunk;
      e_hi = min(w.n_tot, e_lo + a.wchunk);
    }
  }
  const int nope = a.D - a.r;
  const int npair = a.r / 2;
  const int row_bytes = (int)a.row_bytes;
  const int mode = a.mode, G = a.G, kk = a.k, NN = a.N;
  const int n_comp = w.n_comp;
  const uint8_t* kvb = a.kv + (int64_t)w.b * NN * row_bytes;
  // window row of position lo_w + off: pre-rotated, or raw and rotated here
  const bool rot_here = !a.win_rotated;
  const uint8_t* winb = rot_here
      ? a.raw + ((int64_t)w.b * a.T_raw + (w.lo_w - L.pos[(MULTI ? a.pos_raw : a.B) + w.b])) * row_bytes
      : a.win + ((int64_t)w.b * a.win_rows + w.win_row0) * a.win_row_bytes;
  // low parts of rotated window dims (dims lo_base .. D-1), added on the
  // tiles that hold window rows
  const int lo_base = D - lo_dims(a.r);
  const int n_lo_ch = (D - lo_base) / 8;        // 16-byte chunks of a row's low parts
  const bool has_lo = a.r > 0 && a.W > 0;
  // 32-dim k-steps of this wave's part of D at or past lo_base (its last
  // ones; lo_base is a multiple of 32 and at least D - 128)
  const int nlo = __builtin_amdgcn_readfirstlane(
      max(0, min(Gm::DW, (dh + 1) * Gm::DW - lo_base)) / 32);
  const uint8_t* any_row = static_cast<const uint8_t*>(a.q);   // valid address for empty slots
  const int n_fp8 = KV == kMixed ? nope / 16 : 0;
  const int n_chunks = KV == kMixed ? n_fp8 + a.r / 8 : D / 8;
  const int st_e = tid / TPR, st_part = tid % TPR;
  const int n_tiles = e_hi > e_lo ? (e_hi - e_lo + kTile - 1) / kTile : 0;

  // this lane's query row
  const int row = rg * 16 + lr;
  const int g = row / a.Hs, h = w.h0 + row % a.Hs;
  const bool live = g < w.n_q;

  // Optional RMSNorm of the query heads (before the rotation): the gains of
  // the lane's dims are requested first -- before the query slices, so that
  // the waits for the slices and the first tile count their loads exactly.
  const bool qnorm = a.q_norm_gain != nullptr;
  float4 qg[Gm::KH][2];
  float q_inv = 1.f;
  if (qnorm) {
#pragma unroll
    for (int s = 0; s < Gm::KH; ++s) {
      const float* gp = a.q_norm_gain + dh * Gm::DW + 32 * s + 8 * lq;
      qg[s][0] = *reinterpret_cast<const float4*>(gp);
      qg[s][1] = *reinterpret_cast<const float4*>(gp + 4);
    }
  }

  // query slices of the wave's part of D into registers first
  bf16x8 qreg[Gm::KH];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) +
                       (((int64_t)w.b * a.Tq + w.i0 + (live ? g : 0)) * a.H + h) * D +
                       dh * Gm::DW + 8 * lq;
#pragma unroll
    for (int s = 0; s < Gm::KH; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
  }

  // CSA indices of this split to LDS (the plan keeps them within kIdxLds).
  const int n_idx = mode == 0 ? max(0, min(e_hi, n_comp) - e_lo) : 0;
  if (n_idx > 0) {
    const int32_t* src = a.idx + ((int64_t)w.b * a.Tq + w.i0) * kk + e_lo;
    for (int e = tid; e < n_idx; e += NT) lidx[e] = src[e];
  }
  launch_freq_table(freq, L, a.r, tid, NT);
  __syncthreads();

  constexpr int NST = KV == kMixed ? Gm::NCHM : Gm::NCH;
  uint4 stage[NST], stage_lo[Gm::NLO];
  // first dim of 16-byte staging chunk ch (mixed rows: 16 E4M3 dims per chunk,
  // then 8 bf16 rope dims per chunk)
  auto chunk_dim = [&](int ch) {
    if constexpr (KV == kMixed) return ch < n_fp8 ? 16 * ch : nope + 8 * (ch - n_fp8);
    return 8 * ch;
  };
  int st_tag = kNoEntry, st_lo = 64, st_span = 0;
  // lo_loads: the tile holds pre-rotated window rows, whose low parts are
  // loaded too (a uniform branch; every lane then issues those loads).
  auto load_tile = [&](int base, bool lo_loads) {
    const int e = base + st_e;
    const uint8_t* rs = nullptr;
    int tag = kNoEntry;
    int64_t lo = 64, hi = -1;    // query slots g (0 .. n_q-1) that see the entry
    if (e < e_hi) {
      if (e < n_comp) {
        if (mode == 0) {
          // CSA: the entry was selected by query e / k only
          const int j = lidx[e - e_lo];
          if (j >= 0 && j < NN) {
            rs = kvb + (int64_t)j * row_bytes;
            tag = G == 1 ? 0 : e / kk;
            lo = hi = tag;
          }
        } else {
          // HCA entry e covers positions up to (e+1) m - 1: seen from t >= (e+1) m
          rs = kvb + (int64_t)e * row_bytes;
          tag = -1 - e;
          lo = (int64_t)(e + 1) * a.m - w.t_first;
          hi = w.n_q - 1;
        }
      } else {
        // window row at position s = lo_w + off: seen from t in [s, s + W - 1]
        rs = winb + (int64_t)(e - n_comp) * (rot_here ? row_bytes : (int)a.win_row_bytes);
        tag = kWinTag | (e - n_comp);
        lo = w.lo_w + (e - n_comp) - w.t_first;
        hi = min((int64_t)w.n_q - 1, lo + a.W - 1);
      }
    }
    lo = max(lo, (int64_t)0);
    st_tag = tag;
    st_lo = lo <= hi ? (int)lo : 64;
    st_span = lo <= hi ? (int)(hi - lo) : 0;
    // Every lane issues all NST loads (no divergent branches around them);
    // chunks past the row and empty slots read a valid address and are not
    // used (an empty slot is staged as zeros).
#pragma unroll
    for (int q = 0; q < NST; ++q) {
      const int ch = st_part + TPR * q;
      const uint8_t* src = (rs != nullptr && ch < n_chunks) ? rs + 16 * ch : any_row;
      stage[q] = ld_stream16(src);
    }
    // pre-rotated window rows carry their low parts after the row
    if (lo_loads) {
#pragma unroll
      for (int q = 0; q < Gm::NLO; ++q) {
        const int j = st_part + TPR * q;
        const bool mine = rs != nullptr && tag >= kWinTag && j < n_lo_ch;
        stage_lo[q] = ld_stream16(mine ? rs + 16 * (n_chunks + j) : any_row);
      }
    }
  };
  // A window row is rotated here at its position s: the 16-byte chunk of
  // bf16 rope dims it holds is 4 pairs starting at pair p0; the rotated
  // values leave as bf16 high parts (returned) and low parts (*lo).
  auto rotate_chunk = [&](uint4 v, int p0, int64_t pos, uint4* lo) {
    uint32_t wd[4] = {v.x, v.y, v.z, v.w}, lw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float cs, sn;
      rope_cos_sin((double)pos, freq[p0 + p], &cs, &sn);
      const float x0 = bf16_to_f32(wd[p] & 0xffffu), x1 = bf16_to_f32(wd[p] >> 16);
      split_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs, &wd[p], &lw[p]);
    }
    *lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    return make_uint4(wd[0], wd[1], wd[2], wd[3]);
  };
  // with_lo: the tile holds window rows, so every row of it writes its low
  // parts (zero but for the rotated dims of window rows).
  auto store_tile = [&](int buf, auto with_lo_c) {
    constexpr bool with_lo = decltype(with_lo_c)::value;
    uint8_t* dst_row = Et[buf] + st_e * Gm::EROW;
    uint8_t* lo_row = Elo[buf] + st_e * kLoRow;
    const bool empty = st_tag == kNoEntry;
    const bool is_win = st_tag >= kWinTag;
    const bool win = rot_here && is_win;
    const int64_t wpos = w.lo_w + (st_tag - kWinTag);
#pragma unroll
    for (int q = 0; q < NST; ++q) {
      const int ch = st_part + TPR * q;
      if (ch >= n_chunks) continue;
      uint4 v = empty ? make_uint4(0u, 0u, 0u, 0u) : stage[q];
      uint4 lo = make_uint4(0u, 0u, 0u, 0u);
      const int dc = chunk_dim(ch);
      if constexpr (KV == kMixed) {
        if (ch < n_fp8) {    // 16 E4M3 codes -> 16 bf16 (exact)
          uint4* dst = reinterpret_cast<uint4*>(dst_row + 32 * ch);
          dst[0] = e4m3x8_to_bf16x8(v.x, v.y);
          dst[1] = e4m3x8_to_bf16x8(v.z, v.w);
        } else {
          if (win) v = rotate_chunk(v, 4 * (ch - n_fp8), wpos, &lo);
          *reinterpret_cast<uint4*>(dst_row + 32 * n_fp8 + 16 * (ch - n_fp8)) = v;
        }
      } else {
        if (win && dc >= nope) v = rotate_chunk(v, (dc - nope) / 2, wpos, &lo);
        *reinterpret_cast<uint4*>(dst_row + 16 * ch) = v;
      }
      if (with_lo && win && dc >= nope) *reinterpret_cast<uint4*>(lo_row + 2 * (dc - lo_base)) = lo;
    }
    if constexpr (with_lo) {
      // low-part slot j: the loaded low parts of a pre-rotated window row,
      // else zeros, except where a window row rotated here wrote its own
#pragma unroll
      for (int q = 0; q < Gm::NLO; ++q) {
        const int j = st_part + TPR * q;
        if (j < n_lo_ch && !(win && lo_base + 8 * j >= nope))
          *reinterpret_cast<uint4*>(lo_row + 16 * j) =
              (!rot_here && is_win) ? stage_lo[q] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (st_part == 0) {
      const int vpos = (((st_e & 1) << 3) | ((st_e & 15) >> 1)) | (st_e & 16);   // rho^-1
      vis_lo[buf][vpos] = st_lo;
      vis_span[buf][vpos] = st_span;
    }
  };

  // Unconditional (past the split's end the slots are empty and read a valid
  // address), so the waits for the query slices below can count the three
  // tile loads issued after them and leave those in flight.
  // tiles from t_win on hold window rows (they sit at the end of the entry
  // list, from n_comp on); pre-rotated ones bring their low parts
  const int t_win = has_lo && e_hi > n_comp ? min(n_tiles, max(0, n_comp - e_lo) / kTile) : n_tiles;
  const bool lo_loads = !rot_here && has_lo;
  load_tile(e_lo, lo_loads && t_win == 0);

  // the block's query angles, then the lane's query slices rotated at t
  for (int e = tid; e < G * npair; e += NT) {
    const int gg = e / npair, p = e - gg * npair;
    float cs, sn;
    rope_cos_sin((double)(w.t_first + gg), freq[p], &cs, &sn);
    qang[e] = make_float2(cs, sn);
  }
  float q_ss = 0.f;
  if (qnorm) {
    // the row's four lanes, then (D split over two waves) the other half
#pragma unroll
    for (int s = 0; s < Gm::KH; ++s) {
      uint32_t wd[4];
      __builtin_memcpy(wd, &qreg[s], 16);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = bf16_to_f32(wd[p] & 0xffffu), x1 = bf16_to_f32(wd[p] >> 16);
        q_ss = fmaf(x0, x0, fmaf(x1, x1, q_ss));
      }
    }
    q_ss += __shfl_xor(q_ss, 16);
    q_ss += __shfl_xor(q_ss, 32);
    if (lq == 0) qss[dh][row] = q_ss;
  }
  __syncthreads();
  if (qnorm) {
    if constexpr (DS == 2) q_ss += qss[1 - dh][row];
    q_inv = 1.0f / sqrtf(q_ss / (float)D + a.norm_eps);
  }
  const float2* ang = qang + (live ? g : 0) * npair;
#pragma unroll
  for (int s = 0; s < Gm::KH; ++s) {
    const int d0 = dh * Gm::DW + 32 * s + 8 * lq;
    if (qnorm || d0 >= nope) {
      uint32_t wd[4];
      __builtin_memcpy(wd, &qreg[s], 16);
      float x[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        x[2 * p] = bf16_to_f32(wd[p] & 0xffffu);
        x[2 * p + 1] = bf16_to_f32(wd[p] >> 16);
      }
      if (qnorm) {
        const float gv[8] = {qg[s][0].x, qg[s][0].y, qg[s][0].z, qg[s][0].w,
                             qg[s][1].x, qg[s][1].y, qg[s][1].z, qg[s][1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] *= q_inv * gv[i];
      }
      if (d0 >= nope) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float2 cv = ang[(d0 - nope) / 2 + p];
          const float x0 = x[2 * p], x1 = x[2 * p + 1];
          x[2 * p] = x0 * cv.x - x1 * cv.y;
          x[2 * p + 1] = x0 * cv.y + x1 * cv.x;
        }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) wd[p] = pack_bf16x2(x[2 * p], x[2 * p + 1]);
      __builtin_memcpy(&qreg[s], wd, 16);
    }
  }

  // Every prologue load (query slices, first tile) completes here, so that
  // inside the tile loop only the prefetch of the next tile is outstanding
  // and no wait for it is placed before the compute of the current tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  const float scale_log2 = a.scale_log2;
  float m_run = -INFINITY, l_part = 0.f;
  f32x4 oacc[Gm::DH];
#pragma unroll
  for (int dt = 0; dt < Gm::DH; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float* sx_mine = &Sx[dh][rg][l][0];
  const float* sx_other = &Sx[DS - 1 - dh][rg][l][0];

  // ---- the tile loop, software-pipelined by one tile: iteration t stages
  // tile t and computes its logits (QK) while it runs the softmax and PV of
  // tile t-1, so that the matrix cores work on one tile while the vector
  // unit and LDS serve the other.  Each piece is inlined where it is used,
  // once per combination of window-tile flags (wt: the tile holds window
  // rows and adds their low parts), so that no runtime branch splits an
  // iteration's instruction stream.
#define LAC_INLINE __attribute__((always_inline))
  // store tile t (waits for this thread's prefetched rows), publish it, and
  // prefetch tile t+1
  auto publish = [&](int t, auto wt_c) LAC_INLINE {
    store_tile(t & 1, wt_c);
    lds_barrier();            // tile t visible; every wave is done with tile t-2
    if (t + 1 < n_tiles) load_tile(e_lo + (t + 1) * kTile, lo_loads && t + 1 >= t_win);
  };
  // partial S^T over this wave's half of D, entries 0-15 (s0) and 16-31 (s1);
  // the entry fragments are read one group of k-steps ahead
  auto qk = [&](int buf, auto wt_c, f32x4& s0, f32x4& s1) LAC_INLINE {
    constexpr bool wt = decltype(wt_c)::value;
    const uint8_t* E = Et[buf];
    s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    s1 = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int QG = Gm::KH >= 4 ? 4 : Gm::KH;
    const uint8_t* eb = E + q_row * Gm::EROW + 16 * lq + 2 * dh * Gm::DW;
    bf16x8 fa[2][QG], fb[2][QG];
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      fa[0][u] = *reinterpret_cast<const bf16x8*>(eb + 64 * u);
      fb[0][u] = *reinterpret_cast<const bf16x8*>(eb + 16 * Gm::EROW + 64 * u);
    }
#pragma unroll
    for (int gi = 0; gi < Gm::KH / QG; ++gi) {
      const int cur = gi & 1;
      if (gi + 1 < Gm::KH / QG) {
#pragma unroll
        for (int u = 0; u < QG; ++u) {
          const int st = (gi + 1) * QG + u;
          fa[cur ^ 1][u] = *reinterpret_cast<const bf16x8*>(eb + 64 * st);
          fb[cur ^ 1][u] = *reinterpret_cast<const bf16x8*>(eb + 16 * Gm::EROW + 64 * st);
        }
      }
#pragma unroll
      for (int u = 0; u < QG; ++u) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[cur][u], qreg[gi * QG + u], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[cur][u], qreg[gi * QG + u], s1, 0, 0, 0);
      }
    }
    if constexpr (wt) {
      // the window rows' low parts over the wave's last nlo k-steps
      auto lo_qk = [&](auto nk_c) LAC_INLINE {
        constexpr int NK = decltype(nk_c)::value;
#pragma unroll
        for (int st = Gm::KH - NK; st < Gm::KH; ++st) {
          const uint8_t* lb = Elo[buf] + q_row * kLoRow + 16 * lq + 2 * (dh * Gm::DW + 32 * st - lo_base);
          const bf16x8 la = *reinterpret_cast<const bf16x8*>(lb);
          const bf16x8 lc = *reinterpret_cast<const bf16x8*>(lb + 16 * kLoRow);
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(la, qreg[st], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lc, qreg[st], s1, 0, 0, 0);
        }
      };
      switch (nlo) {
        case 1: lo_qk(std::integral_constant<int, 1>{}); break;
        case 2: lo_qk(std::integral_constant<int, 2>{}); break;
        case 3: lo_qk(std::integral_constant<int, Gm::KH >= 3 ? 3 : 1>{}); break;
        case 4: lo_qk(std::integral_constant<int, Gm::KH >= 4 ? 4 : 1>{}); break;
        default: break;
      }
    }
  };
  // the two halves' partial logits summed (D split over two waves): x = the
  // lane's 8 raw logits of the tile
  auto exchange = [&](const f32x4& s0, const f32x4& s1, float* x) LAC_INLINE {
    float4 o0 = make_float4(0.f, 0.f, 0.f, 0.f), o1 = o0;
    if constexpr (DS == 2) {
      *reinterpret_cast<float4*>(sx_mine) = make_float4(s0[0], s0[1], s0[2], s0[3]);
      *reinterpret_cast<float4*>(sx_mine + 4) = make_float4(s1[0], s1[1], s1[2], s1[3]);
      lds_barrier();
      o0 = *reinterpret_cast<const float4*>(sx_other);
      o1 = *reinterpret_cast<const float4*>(sx_other + 4);
    }
    x[0] = s0[0] + o0.x; x[1] = s0[1] + o0.y; x[2] = s0[2] + o0.z; x[3] = s0[3] + o0.w;
    x[4] = s1[0] + o1.x; x[5] = s1[1] + o1.y; x[6] = s1[2] + o1.z; x[7] = s1[3] + o1.w;
  };
  // online softmax of row `row` over the lane's 8 entries of the tile in
  // buffer buf (the same in both waves of the row group), then
  // O^T += E^T P^T over the wave's half of D, 16 output dims per MFMA; the
  // transposed entry fragments are read PG output tiles ahead
  auto softmax_pv = [&](int buf, auto wt_c, const float* xin) LAC_INLINE {
    constexpr bool wt = decltype(wt_c)::value;
    const uint8_t* E = Et[buf];
    const int4 vl0 = *reinterpret_cast<const int4*>(&vis_lo[buf][4 * lq]);
    const int4 vl1 = *reinterpret_cast<const int4*>(&vis_lo[buf][16 + 4 * lq]);
    const int4 vs0 = *reinterpret_cast<const int4*>(&vis_span[buf][4 * lq]);
    const int4 vs1 = *reinterpret_cast<const int4*>(&vis_span[buf][16 + 4 * lq]);
    const int vlo[8] = {vl0.x, vl0.y, vl0.z, vl0.w, vl1.x, vl1.y, vl1.z, vl1.w};
    const int vsp[8] = {vs0.x, vs0.y, vs0.z, vs0.w, vs1.x, vs1.y, vs1.z, vs1.w};
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = (uint32_t)(g - vlo[i]) <= (uint32_t)vsp[i] ? xin[i] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = row_max4(tmax);
    const bool moved = tmax > m_run + 8.f;          // also true for the first visible entry
    const bool rescale = moved && m_run != -INFINITY;   // the row's O holds earlier entries
    const float m_new = moved ? tmax : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float al = moved ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(x[i] - m_use), p1 = __builtin_amdgcn_exp2f(x[i + 1] - m_use);
      psum += p0 + p1;
      pk[i / 2] = pack_bf16x2(p0, p1);
    }
    l_part = l_part * al + psum;
    m_run = m_new;
    bf16x8 pb;
    __builtin_memcpy(&pb, pk, 16);
    if (__ballot(rescale)) {
#pragma unroll
      for (int dt = 0; dt < Gm::DH; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= al;
    }
    constexpr int PG = Gm::DH >= 8 ? 8 : Gm::DH;
    const uint8_t* tb = E + pv_row * Gm::EROW + 8 * (lr & 3) + 2 * dh * Gm::DW;
    bf16x4 lo[2][PG], hi[2][PG];
#pragma unroll
    for (int u = 0; u < PG; ++u) {
      lo[0][u] = ds_read_tr(tb + 32 * u);
      hi[0][u] = ds_read_tr(tb + 16 * Gm::EROW + 32 * u);
    }
#pragma unroll
    for (int gi = 0; gi < Gm::DH / PG; ++gi) {
      const int cur = gi & 1;
      if (gi + 1 < Gm::DH / PG) {
#pragma unroll
        for (int u = 0; u < PG; ++u) {
          const int dt = (gi + 1) * PG + u;
          lo[cur ^ 1][u] = ds_read_tr(tb + 32 * dt);
          hi[cur ^ 1][u] = ds_read_tr(tb + 16 * Gm::EROW + 32 * dt);
        }
      }
#pragma unroll
      for (int u = 0; u < PG; ++u) {
        const bf16x8 ab = __builtin_shufflevector(lo[cur][u], hi[cur][u], 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[gi * PG + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, pb, oacc[gi * PG + u], 0, 0, 0);
      }
    }
    if constexpr (wt) {
      // the window rows' low parts of the wave's last 2 nlo output tiles
      auto lo_pv = [&](auto nk_c) LAC_INLINE {
        constexpr int NT2 = 2 * decltype(nk_c)::value;
#pragma unroll
        for (int dt = Gm::DH - NT2; dt < Gm::DH; ++dt) {
          const uint8_t* tl = Elo[buf] + pv_row * kLoRow + 8 * (lr & 3) +
                              2 * (dh * Gm::DW + 16 * dt - lo_base);
          const bf16x8 ab = __builtin_shufflevector(ds_read_tr(tl), ds_read_tr(tl + 16 * kLoRow),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, pb, oacc[dt], 0, 0, 0);
        }
      };
      switch (nlo) {
        case 1: lo_pv(std::integral_constant<int, 1>{}); break;
        case 2: lo_pv(std::integral_constant<int, 2>{}); break;
        case 3: lo_pv(std::integral_constant<int, Gm::KH >= 3 ? 3 : 1>{}); break;
        case 4: lo_pv(std::integral_constant<int, Gm::KH >= 4 ? 4 : 1>{}); break;
        default: break;
      }
    }
  };
  // one iteration: tile t staged and its logits formed, tile t-1 consumed.
  // The buffers of tile t-1 are staged over by tile t+1: the exchange's
  // barrier (or, without a D split, one of its own) keeps that after every
  // wave's PV of tile t-1.
  auto iter = [&](int t, auto wq_c, auto wp_c, float* x) LAC_INLINE {
    publish(t, wq_c);
    f32x4 s0, s1;
    qk(t & 1, wq_c, s0, s1);
    softmax_pv((t - 1) & 1, wp_c, x);
    if constexpr (DS == 1) lds_barrier();
    exchange(s0, s1, x);
  };
  using F = std::integral_constant<bool, false>;
  using T = std::integral_constant<bool, true>;
  if (n_tiles > 0) {
    float x[8];
    {
      f32x4 s0, s1;
      if (t_win == 0) { publish(0, T{}); qk(0, T{}, s0, s1); }
      else { publish(0, F{}); qk(0, F{}, s0, s1); }
      exchange(s0, s1, x);
    }
    int t = 1;
    for (; t < t_win; ++t) iter(t, F{}, F{}, x);            // both tiles before the window
    if (t == t_win && t < n_tiles) { iter(t, T{}, F{}, x); ++t; }   // the first window tile
    for (; t < n_tiles; ++t) iter(t, T{}, T{}, x);          // both tiles hold window rows
    if (n_tiles - 1 >= t_win) softmax_pv((n_tiles - 1) & 1, T{}, x);
    else softmax_pv((n_tiles - 1) & 1, F{}, x);
  }
#undef LAC_INLINE

  // ---- row sum over the row's four lanes
  float l_row = l_part;
  l_row += __shfl_xor(l_row, 16);
  l_row += __shfl_xor(l_row, 32);

  // ---- output.  With several splits: the partial output normalised by its
  // own row sum, in bf16 (the range of the values themselves), plus (max, sum); with one: the
  // output normalised (sink included), rotated back at -t, in bf16.  The
  // block's 64 rows are staged in the tile buffers (free once every wave is
  // done with the last tile) so that the global stores are whole rows.
  const bool split_out = a.nsplit > 1;
  float sc;
  if (split_out) {
    sc = l_row > 0.f ? 1.f / l_row : 0.f;
  } else {
    float den = l_row;
    if (a.sink) den += exp2f(a.sink[h] * 1.4426950408889634f - (m_run == -INFINITY ? 0.f : m_run));
    sc = den > 0.f ? 1.f / den : 0.f;
  }
  uint8_t* ob = &Et[0][0];                     // [64][EROW] bytes
  __syncthreads();
  {
    uint8_t* orow = ob + row * Gm::EROW + 2 * (dh * Gm::DW + 4 * lq);
#pragma unroll
    for (int dt = 0; dt < Gm::DH; ++dt) {
      const int d0 = dh * Gm::DW + 16 * dt + 4 * lq;
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = oacc[dt][i] * sc;
      uint2 v;
      if (split_out) {
        v = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      } else {
        if (d0 >= nope) {             // rotation at -t: (cos, -sin) of the query's angle
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float2 cv = ang[(d0 - nope) / 2 + p];
            const float x0 = o[2 * p], x1 = o[2 * p + 1];
            o[2 * p] = x0 * cv.x + x1 * cv.y;
            o[2 * p + 1] = -x0 * cv.y + x1 * cv.x;
          }
        }
        v = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      }
      *reinterpret_cast<uint2*>(orow + 32 * dt) = v;
    }
  }
  const int64_t slot = (int64_t)work * a.nsplit + split;
  if (split_out && lq == 0 && dh == 0) {
    a.part_ml[(slot * 64 + row) * 2] = m_run;
    a.part_ml[(slot * 64 + row) * 2 + 1] = l_row;
  }
  __syncthreads();
  // Row r of the block lands at row r of a contiguous run: the split's slot of
  // the partials, or the output rows (b, i0 + r / Hs, h0 + r % Hs), which are
  // consecutive because Hs == H whenever a block holds several tokens.
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  const int n_rows = split_out ? 64 : w.n_q * a.Hs;
  uint8_t* dst = split_out
      ? reinterpret_cast<uint8_t*>(a.part_o + slot * 64 * D)
      : static_cast<uint8_t*>(a.out) + (((int64_t)w.b * a.Tq + w.i0) * a.H + w.h0) * D * 2;
  // Streaming stores: the rows are read once, by the next kernel, and leave
  // no dirty L2 lines for the end-of-kernel write-back (which would delay
  // that kernel's start on this XCD).
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int k = 0; k < 64 * CPR / NT; ++k) {
    const int c = tid + k * NT;
    if (c < n_rows * CPR) {
      const uint4 v = *reinterpret_cast<const uint4*>(ob + (c / CPR) * Gm::EROW + 16 * (c % CPR));
      __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(dst + (int64_t)c * 16));
    }
  }
}

// ---------------------------------------------------------------- combine
template <bool MULTI>
__global__ void __launch_bounds__(256) combine_kernel(KLaunch L) {
  // wgt holds the split weights (nsplit <= kMaxSplit), then (reused) the split
  // groups' partial sums: (256 / (D/8) - 1) * D floats <= 1920 for D >= 128.
  __shared__ float wgt[kMaxSplit];
  __shared__ float red[1];
  __shared__ float2 angle[kMaxRopePairs];
  uint32_t lb = blockIdx.x;
  const int ci = MULTI ? launch_call(L, blockIdx.x, &lb) : 0;
  const KArgs& a = L.k[ci];
  const int work = (int)(lb / 64), row = (int)(lb % 64);
  const Work w = make_work<MULTI>(L, a, work);
  const int g = row / a.Hs, h = w.h0 + row % a.Hs;
  if (g >= w.n_q) return;
  const int64_t slot0 = (int64_t)work * a.nsplit;
  // Thread (split group sg, column group cg) sums splits sg, sg + n_sg, ... over
  // 8 columns with 16-byte loads, eight splits' loads in flight at a time; the
  // split groups then meet in LDS.  The first eight loads are issued before
  // the split weights are formed.
  const int n_cg = a.D / 8, n_sg = 256 / n_cg;
  const int cg = threadIdx.x % n_cg, sg = threadIdx.x / n_cg;
  const uint16_t* pp = a.part_o + (slot0 * 64 + row) * a.D + 8 * cg;
  const int64_t stride = 64LL * a.D;
  uint4 x[8];
  auto issue = [&](int s0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u * n_sg;
      x[u] = *reinterpret_cast<const uint4*>(pp + (int64_t)(s < a.nsplit ? s : 0) * stride);
    }
  };
  issue(sg);
  // While the loads are in flight, wave 1 forms the angles of the rotation
  // at -t and the last wave the split weights.
  const int nope = a.D - a.r;
  const int64_t t = w.t_first + g;
  if (threadIdx.x >= 64 && threadIdx.x < 64 + a.r / 2) {
    const int p = threadIdx.x - 64;
    float c, sn;
    rope_cos_sin((double)t, L.freq[p], &c, &sn);
    angle[p] = make_float2(c, sn);
  }
  const int wlast = 3;
  if ((int)(threadIdx.x / 64) == wlast) {
    const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + slot0 * 64 + row;
    const int tid = threadIdx.x - 64 * wlast;
    const float2 v0 = tid < a.nsplit ? ml[(int64_t)tid * 64] : make_float2(-INFINITY, 0.f);
    float M = v0.x;
    for (int s = tid + 64; s < a.nsplit; s += 64) M = fmaxf(M, ml[(int64_t)s * 64].x);
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float sink2 = a.sink ? a.sink[h] * 1.4426950408889634f : -INFINITY;
    M = fmaxf(M, sink2);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    if (tid < a.nsplit) {
      const float f = exp2f(v0.x - Mu) * v0.y;
      wgt[tid] = f;
      L = f;
    }
    for (int s = tid + 64; s < a.nsplit; s += 64) {
      const float2 v = ml[(int64_t)s * 64];
      const float f = exp2f(v.x - Mu) * v.y;
      wgt[s] = f;
      L += f;
    }
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    if (tid == 0) {
      if (a.sink) L += exp2f(sink2 - Mu);
      red[0] = L > 0.f ? 1.f / L : 0.f;
    }
  }
  __syncthreads();
  const float inv = red[0];
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = sg; s0 < a.nsplit; s0 += 8 * n_sg) {
    if (s0 != sg) issue(s0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u * n_sg;
      const float wv = s < a.nsplit ? wgt[s] : 0.f;
      const uint32_t wd[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] = fmaf(wv, bf16_to_f32(wd[c] & 0xffffu), acc[2 * c]);
        acc[2 * c + 1] = fmaf(wv, bf16_to_f32(wd[c] >> 16), acc[2 * c + 1]);
      }
    }
  }
  float* part = reinterpret_cast<float*>(wgt + 0);   // the weights are no longer needed
  __syncthreads();
  if (sg > 0) {
#pragma unroll
    for (int c = 0; c < 8; ++c) part[(sg - 1) * a.D + 8 * cg + c] = acc[c];
  }
  __syncthreads();
  if (sg != 0) return;
  for (int o = 1; o < n_sg; ++o)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += part[(o - 1) * a.D + 8 * cg + c];
  uint16_t* op = static_cast<uint16_t*>(a.out) + (((int64_t)w.b * a.Tq + w.i0 + g) * a.H + h) * a.D + 8 * cg;
  uint32_t pk[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = 8 * cg + 2 * q;
    float o0 = acc[2 * q] * inv, o1 = acc[2 * q + 1] * inv;
    if (c >= nope) {
      const float2 cv = angle[(c - nope) >> 1];
      const float r0 = o0 * cv.x + o1 * cv.y, r1 = -o0 * cv.y + o1 * cv.x;
      o0 = r0;
      o1 = r1;
    }
    pk[q] = pack_bf16x2(o0, o1);
  }
  *reinterpret_cast<uint4*>(op) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
}

// ---------------------------------------------------------------- float32 VALU path
// One workgroup per query; H*D <= 8192, D <= 256.
__global__ void __launch_bounds__(256) attend_f32_kernel(KLaunch L) {
  extern __shared__ float fsm[];
  __shared__ double freq[kMaxRopePairs];
  const KArgs& a = L.k[0];
  launch_freq_table(freq, L, a.r, threadIdx.x, 256);
  const int H = a.H, D = a.D;
  float* qs = fsm;                    // [H][D]
  float* es = qs + H * D;             // [32][D]
  float* lg = es + 32 * D;            // [H][32]
  float* mrow = lg + H * 32;          // [H]
  float* lrow = mrow + H;             // [H]
  float* al = lrow + H;               // [H]
  int* tags = reinterpret_cast<int*>(al + H);   // [32]
  const int tid = threadIdx.x;
  const Work w = make_work(L, a, blockIdx.x);   // G = 1, one query
  const Vis vis0 = make_vis(a, w, 0);
  const int64_t t = w.t_first;
  const int nope = D - a.r;
  const float* q = static_cast<const float*>(a.q) + ((int64_t)w.b * a.Tq + w.i0) * H * D;
  for (int e = tid; e < H * D; e += blockDim.x) qs[e] = q[e];
  for (int h = tid; h < H; h += blockDim.x) { mrow[h] = -INFINITY; lrow[h] = 0.f; }
  __syncthreads();
  if (a.q_norm_gain) {                // RMSNorm of each head, before the rotation
    for (int h = tid; h < H; h += blockDim.x) {
      float ss = 0.f;
      for (int c = 0; c < D; ++c) ss = fmaf(qs[h * D + c], qs[h * D + c], ss);
      const float inv = 1.0f / sqrtf(ss / (float)D + a.norm_eps);
      for (int c = 0; c < D; ++c) qs[h * D + c] *= inv * a.q_norm_gain[c];
    }
    __syncthreads();
  }
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
      const uint8_t* src = entry_src(a, w, (int)(base + ei), false, nullptr, 0, &tag);
      es[e] = src ? reinterpret_cast<const float*>(src)[c] : 0.f;
      if (c == 0) tags[ei] = tag;
    }
    __syncthreads();
    for (int e = tid; e < H * 32; e += blockDim.x) {
      const int h = e / 32, ei = e % 32;
      float dot = 0.f;
      for (int c = 0; c < D; ++c) dot = fmaf(qs[h * D + c], es[ei * D + c], dot);
      lg[e] = visible(tags[ei], 0, vis0) ? dot * a.scale_log2 : -INFINITY;
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
hipError_t launch_mfma(const KLaunch& L, size_t lds, hipStream_t st) {
  {
    TimedLaunch tl(kKernelAttend, st);
    if (L.n == 1)
      hipLaunchKernelGGL((attend_mfma_kernel<D, KV, false>), dim3(L.k[0].nsplit, L.k[0].n_work),
                         dim3(Geo<D>::NT), lds, st, L);
    else
      hipLaunchKernelGGL((attend_mfma_kernel<D, KV, true>), dim3(L.blk_end[L.n - 1]),
                         dim3(Geo<D>::NT), lds, st, L);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the calls with split partials, merged by one combine launch; their
  // positions are packed again from the start of the pool (a launch of one
  // call finds them there)
  KLaunch C = L;
  C.n = 0;
  int n_pos = 0;
  for (int i = 0; i < L.n; ++i) {
    const KArgs& k = L.k[i];
    if (k.nsplit == 1) continue;
    C.k[C.n] = k;
    for (int b = 0; b < k.B; ++b) {
      C.pos[n_pos + b] = L.pos[k.pos_q + b];
      C.pos[n_pos + k.B + b] = L.pos[k.pos_raw + b];
    }
    C.k[C.n].pos_q = n_pos;
    C.k[C.n].pos_raw = n_pos + k.B;
    n_pos += 2 * k.B;
    C.blk_end[C.n] = (C.n ? C.blk_end[C.n - 1] : 0u) + (uint32_t)k.n_work * 64u;
    ++C.n;
  }
  if (C.n == 0) return hipSuccess;
  TimedLaunch tl(kKernelCombine, st);
  if (C.n == 1)
    hipLaunchKernelGGL(combine_kernel<false>, dim3(C.blk_end[0]), dim3(256), 0, st, C);
  else
    hipLaunchKernelGGL(combine_kernel<true>, dim3(C.blk_end[C.n - 1]), dim3(256), 0, st, C);
  return hipGetLastError();
}

// The kernel arguments of one call under plan p; positions go to the pool of L.
KArgs make_kargs(const AttendArgs& a, const AttnPlan& p, void* ws, KLaunch* L, int* n_pos) {
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  KArgs k{};
  k.q = a.q; k.kv = static_cast<const uint8_t*>(a.kv); k.idx = a.idx; k.win = w8 + p.off_win;
  k.win_row_bytes = p.win_row_bytes;
  k.sink = a.sink; k.out = a.out; k.zero_row = w8 + p.off_zero;
  k.ang = reinterpret_cast<const float2*>(w8 + p.off_ang);
  k.part_o = p.nsplit > 1 ? reinterpret_cast<uint16_t*>(w8 + p.off_po) : nullptr;
  k.part_ml = p.nsplit > 1 ? reinterpret_cast<float*>(w8 + p.off_pml) : nullptr;
  k.mode = a.mode; k.N = a.N; k.k = a.k; k.m = a.m; k.W = a.W; k.B = a.B; k.Tq = a.Tq;
  k.H = a.H; k.D = a.D; k.r = a.r; k.theta = a.theta;
  k.scale_log2 = a.scale * 1.4426950408889634f;
  k.q_norm_gain = a.q_norm_gain;
  k.norm_eps = a.norm_eps;
  k.G = p.G; k.Hs = p.Hs; k.n_htiles = p.n_htiles; k.n_qgroups = p.n_qgroups; k.n_work = p.n_work;
  k.nsplit = p.nsplit; k.chunk = p.chunk; k.wchunk = p.wchunk; k.win_rows = p.win_rows; k.row_bytes = p.row_bytes;
  k.raw = static_cast<const uint8_t*>(a.raw); k.T_raw = a.T_raw;
  k.win_rotated = a.kv_fmt == kF32 || a.Tq > 8;
  k.pos_q = *n_pos;
  k.pos_raw = *n_pos + a.B;
  for (int b = 0; b < a.B; ++b) {
    L->pos[*n_pos + b] = a.qpos.v[b];
    L->pos[*n_pos + a.B + b] = a.rawpos.v[b];
  }
  *n_pos += 2 * a.B;
  return k;
}

// With many queries per sequence the window rows are shared by many blocks:
// rotate them once up front (and, on the float32 path, the query angles).
// In decode each block rotates its own.
hipError_t rotate_window(const AttendArgs& a, const AttnPlan& p, void* ws, hipStream_t st) {
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  WinArgs wa{};
  wa.raw = static_cast<const uint8_t*>(a.raw);
  wa.win = w8 + p.off_win;
  wa.win_row_bytes = p.win_row_bytes;
  wa.zero_row = w8 + p.off_zero;
  wa.fmt = a.kv_fmt; wa.B = a.B; wa.D = a.D; wa.r = a.r; wa.Tq = a.Tq; wa.W = a.W;
  wa.T_raw = a.T_raw; wa.win_rows = p.win_rows; wa.row_bytes = p.row_bytes;
  make_rope_table(&wa.rope, a.r, a.theta);
  wa.qpos = a.qpos; wa.rawpos = a.rawpos;
  wa.ang = reinterpret_cast<float2*>(w8 + p.off_ang);
  wa.n_win_items = (int64_t)a.B * p.win_rows * (a.D / 8);
  const int64_t n = wa.n_win_items + (int64_t)a.B * a.Tq * (a.r / 2);
  const unsigned blocks = (unsigned)std::max<int64_t>(1, (n + 255) / 256);
  hipLaunchKernelGGL(rope_window_kernel, dim3(blocks), dim3(256), 0, st, wa);
  return hipGetLastError();
}

AttnPlan launch_plan(const AttendArgs& a, int grid_target = kGridTarget) {
  const bool f32 = a.kv_fmt == kF32;
  const AttnPlan loose = make_plan(a.B, a.Tq, a.H, a.D, a.r, a.kv_fmt, a.n_entries, a.W, f32, false, grid_target);
  if (a.mode != 1 || f32) return loose;
  const AttnPlan tight = make_plan(a.B, a.Tq, a.H, a.D, a.r, a.kv_fmt, a.n_entries, a.W, f32, true, grid_target);
  return tight.nsplit <= loose.nsplit ? tight : loose;
}

// Plans of n calls launched together: the one-wave grid (kGridTarget
// workgroups) is shared in proportion to each call's tiles, and while the
// calls' workgroups exceed it, the call with the most gives up one split per
// work item.  A smaller target never adds splits, so every plan fits the
// workspace its call was sized for.
void plan_group(const AttendArgs* calls, const int* idx, int n, AttnPlan* plans) {
  if (n == 1) { plans[0] = launch_plan(calls[idx[0]]); return; }
  int target[kAttendGroup];
  double cost[kAttendGroup], total = 0.0;
  for (int i = 0; i < n; ++i) {
    const AttnPlan p = launch_plan(calls[idx[i]]);
    cost[i] = (double)p.n_work * (double)((p.max_entries + kTile - 1) / kTile);
    total += cost[i];
  }
  for (int i = 0; i < n; ++i) {
    const AttnPlan p = launch_plan(calls[idx[i]]);
    target[i] = std::max(p.n_work, (int)(kGridTarget * cost[i] / std::max(total, 1.0)));
  }
  for (;;) {
    int64_t blocks = 0, worst_blocks = 0;
    int worst = -1;
    for (int i = 0; i < n; ++i) {
      plans[i] = launch_plan(calls[idx[i]], target[i]);
      const int64_t b = (int64_t)plans[i].nsplit * plans[i].n_work;
      blocks += b;
      if (target[i] > plans[i].n_work && b > worst_blocks) { worst = i; worst_blocks = b; }
    }
    if (blocks <= kGridTarget || worst < 0) return;
    target[worst] = std::max(plans[worst].n_work, target[worst] - plans[worst].n_work);
  }
}

}  // namespace

// The workspace is sized without knowing the mode (G * n_entries entries per
// work item, enough for either); HCA launches with its tighter count unless
// that would ask for more splits than the workspace holds.
size_t attend_workspace_bytes(int B, int Tq, int H, int D, int r, int kv_fmt, int n_entries, int W) {
  return make_plan(B, Tq, H, D, r, kv_fmt, n_entries, W, kv_fmt == kF32, false).total;
}

int attend_split_count(const AttendArgs& a) { return launch_plan(a).nsplit; }

// n independent calls: the float32 ones one by one; the others with plans
// made together, their window rotations (prefill shapes) first, then one
// attention launch per (D, KV format) and up to kAttendGroup calls sharing a
// rotation table, each followed by the combine of its split calls.
hipError_t launch_attend_group(const AttendArgs* calls, void* const* ws, int n, hipStream_t st) {
  hipError_t e;
  std::vector<int> idx;
  for (int i = 0; i < n; ++i) {
    const AttendArgs& a = calls[i];
    if (a.B == 0 || a.Tq == 0) continue;
    if (a.kv_fmt == kF32) {
      const AttnPlan p = launch_plan(a);
      if (a.W > 0 && (e = rotate_window(a, p, ws[i], st)) != hipSuccess) return e;
      KLaunch L{};
      int n_pos = 0;
      L.k[0] = make_kargs(a, p, ws[i], &L, &n_pos);
      L.n = 1;
      RopeTable rt;
      make_rope_table(&rt, a.r, a.theta);
      for (int q = 0; q < kMaxRopePairs; ++q) L.freq[q] = rt.inv_freq[q];
      const size_t lds = ((size_t)a.H * a.D + 32 * a.D + a.H * 32 + 3 * a.H) * 4 + 32 * 4;
      TimedLaunch tl(kKernelAttend, st);
      hipLaunchKernelGGL(attend_f32_kernel, dim3(p.n_work), dim3(256), lds, st, L);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      continue;
    }
    idx.push_back(i);
  }
  const int m = (int)idx.size();
  // plans: together for up to kAttendGroup calls at a time, in call order
  for (int g0 = 0; g0 < m; g0 += kAttendGroup) {
    const int gn = std::min(kAttendGroup, m - g0);
    AttnPlan plans[kAttendGroup];
    plan_group(calls, idx.data() + g0, gn, plans);
    for (int i = 0; i < gn; ++i) {
      const AttendArgs& a = calls[idx[g0 + i]];
      if (plans[i].nsplit > kMaxSplit) return hipErrorInvalidValue;
      if (a.W > 0 && a.Tq > 8 && (e = rotate_window(a, plans[i], ws[idx[g0 + i]], st)) != hipSuccess) return e;
    }
    // launches: calls of one (D, KV format) and one rotation table together
    bool done[kAttendGroup] = {};
    for (int i = 0; i < gn; ++i) {
      if (done[i]) continue;
      const AttendArgs& a0 = calls[idx[g0 + i]];
      KLaunch L{};
      int n_pos = 0;
      size_t lds = 0;
      for (int j = i; j < gn; ++j) {
        const AttendArgs& a = calls[idx[g0 + j]];
        const bool same_table = a.r == a0.r && (a.r == 0 || a.theta == a0.theta);
        if (done[j] || a.D != a0.D || a.kv_fmt != a0.kv_fmt || !same_table ||
            n_pos + 2 * a.B > kAttendPos)
          continue;
        const AttnPlan& p = plans[j];
        L.k[L.n] = make_kargs(a, p, ws[idx[g0 + j]], &L, &n_pos);
        L.blk_end[L.n] = (L.n ? L.blk_end[L.n - 1] : 0u) + (uint32_t)p.nsplit * (uint32_t)p.n_work;
        ++L.n;
        lds = std::max(lds, (size_t)p.G * (a.r / 2) * sizeof(float2));   // the block's query angles
        done[j] = true;
      }
      RopeTable rt;
      make_rope_table(&rt, a0.r, a0.theta);
      for (int q = 0; q < kMaxRopePairs; ++q) L.freq[q] = rt.inv_freq[q];
      if (a0.kv_fmt == kBF16) {
        e = a0.D == 128 ? launch_mfma<128, kBF16>(L, lds, st)
          : a0.D == 256 ? launch_mfma<256, kBF16>(L, lds, st) : launch_mfma<512, kBF16>(L, lds, st);
      } else {
        e = a0.D == 128 ? launch_mfma<128, kMixed>(L, lds, st)
          : a0.D == 256 ? launch_mfma<256, kMixed>(L, lds, st) : launch_mfma<512, kMixed>(L, lds, st);
      }
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_attend(const AttendArgs& a, void* ws, hipStream_t st) {
  return launch_attend_group(&a, &ws, 1, st);
}

}  // namespace lac
