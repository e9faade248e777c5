// abi.cpp -- the C ABI declared in include/lac.h: argument validation (pure
// host code, nothing is enqueued on error), workspace sizing, the thread-local
// error string and launch timer, and dispatch to the kernel launchers.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <exception>
#include <vector>

#include "lac.h"
#include "lac_internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local int g_timer_kernel = -1;
thread_local hipEvent_t g_timer_start = nullptr;
thread_local hipEvent_t g_timer_stop = nullptr;

// The launch group open on this thread (lac_group_begin .. lac_group_end):
// the validated calls recorded for one grouped enqueue.
struct Group {
  bool open = false;
  void* stream = nullptr;
  std::vector<lac::CompressArgs> comp;
  std::vector<lac::ClearJob> clears;
  std::vector<lac::AttendArgs> att;
  std::vector<void*> att_ws;
  std::vector<size_t> att_need;
  void close() {
    open = false;
    stream = nullptr;
    comp.clear();
    clears.clear();
    att.clear();
    att_ws.clear();
    att_need.clear();
  }
};
thread_local Group g_group;

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kPosLimit = (int64_t)1 << 31;

// Copies host positions into the by-value struct, checking range and the
// block alignment `mult` (1 = none).
int32_t take_positions(const char* fn, const char* what, const int64_t* src, int B, int64_t span,
                       int mult, lac::Positions* dst) {
  for (int b = 0; b < B; ++b) {
    const int64_t p = src ? src[b] : 0;
    if (p < 0 || p + span >= kPosLimit)
      return fail(LAC_ERR_INVALID, "%s: %s[%d] = %lld is outside [0, 2^31 - %lld)", fn, what, b,
                  (long long)p, (long long)span);
    if (mult > 1 && p % mult != 0)
      return fail(LAC_ERR_INVALID, "%s: %s[%d] = %lld is not a multiple of m = %d", fn, what, b,
                  (long long)p, mult);
    dst->v[b] = (int32_t)p;
  }
  return LAC_OK;
}

// Entry points that cannot be recorded refuse to run inside a group.
int32_t refuse_in_group(const char* fn) {
  return fail(LAC_ERR_INVALID, "%s: not allowed while a launch group is open on this thread", fn);
}

int32_t group_stream(const char* fn, void* stream) {
  if (stream != g_group.stream)
    return fail(LAC_ERR_INVALID, "%s: stream differs from the open launch group's", fn);
  return LAC_OK;
}

int32_t launch_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(LAC_ERR_DEVICE, "%s: launch failed: %s", fn, hipGetErrorString(e));
  g_err[0] = 0;
  return LAC_OK;
}

// The optional RMSNorm of an entry (norm_gain [D] float32, 16-byte aligned,
// eps >= 0) keeps all D/8 channel groups of an entry in one wave, so it needs
// D/8 to be a power of two of at most 64.
int32_t check_norm(const char* fn, const float* gain, float eps) {
  if (!gain) return fail(LAC_ERR_INVALID, "%s: null norm gain", fn);
  if (!aligned(gain, 16)) return fail(LAC_ERR_INVALID, "%s: norm gain must be 16-byte aligned", fn);
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(LAC_ERR_INVALID, "%s: norm eps must be finite and >= 0", fn);
  return LAC_OK;
}

int32_t compress_impl(const char* fn, const void* raw_kv, const void* logits, int32_t in_dtype,
                      void* out, int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                      int32_t rope_dims, float rope_theta, const int64_t* pos0,
                      int64_t kv_bstride, int64_t z_bstride, int64_t out_bstride, void* stream,
                      const float* norm_gain = nullptr, float norm_eps = 0.f, bool norm = false,
                      int32_t overlap = 0) {
  if (in_dtype != LAC_F32 && in_dtype != LAC_BF16)
    return fail(LAC_ERR_UNSUPPORTED, "%s: in_dtype must be LAC_F32 or LAC_BF16", fn);
  if ((out_dtype < LAC_F32 || out_dtype > LAC_KV_E4M3_ROPE_BF16) && out_dtype != LAC_MXFP4)
    return fail(LAC_ERR_UNSUPPORTED, "%s: unknown out_dtype %d", fn, out_dtype);
  if (out_dtype == LAC_MXFP4 && (rope_dims != 0 || D % 32))
    return fail(LAC_ERR_UNSUPPORTED, "%s: MXFP4 output needs rope_dims = 0 and D a multiple of 32", fn);
  if (B < 0 || B > LAC_MAX_BATCH) return fail(LAC_ERR_INVALID, "%s: B = %d outside [0, %d]", fn, B, LAC_MAX_BATCH);
  if (T < 0) return fail(LAC_ERR_INVALID, "%s: T = %d < 0", fn, T);
  if (m < 1 || m > 256) return fail(LAC_ERR_INVALID, "%s: m = %d outside [1, 256]", fn, m);
  if (D < 8 || D > 2048 || D % 8) return fail(LAC_ERR_INVALID, "%s: D = %d must be a multiple of 8 in [8, 2048]", fn, D);
  if (rope_dims < 0 || rope_dims > D || rope_dims > 128 || rope_dims % 8)
    return fail(LAC_ERR_INVALID, "%s: rope_dims = %d must be a multiple of 8 in [0, min(D, 128)]", fn, rope_dims);
  if (rope_dims > 0 && !(rope_theta > 0.f && isfinite(rope_theta)))
    return fail(LAC_ERR_INVALID, "%s: rope_theta must be positive and finite", fn);
  if (overlap < 0 || overlap > 256 - m)
    return fail(LAC_ERR_INVALID, "%s: overlap = %d outside [0, 256 - m]", fn, overlap);
  const int N = T / m;
  int64_t lead_max = 0;        // rows before the first block (overlapping windows)
  for (int b = 0; b < B && overlap > 0; ++b) {
    const int64_t p = pos0 ? pos0[b] : 0;
    const int64_t lead = p < overlap ? (p > 0 ? p : 0) : overlap;
    if (lead > lead_max) lead_max = lead;
  }
  if (B > 1 && (kv_bstride < T + lead_max || z_bstride < T + lead_max || out_bstride < N))
    return fail(LAC_ERR_INVALID, "%s: batch strides must cover T rows (in; plus the overlap's "
                "leading rows) and T/m rows (out)", fn);
  if ((int64_t)B * N * (D / 8) >= lac::kCompressMaxGroups)
    return fail(LAC_ERR_UNSUPPORTED, "%s: B * floor(T/m) * D/8 = %lld reaches 2^31 (one launch's limit)",
                fn, (long long)B * N * (D / 8));
  if (norm) {
    const int G = D / 8;
    if (G > 64 || (G & (G - 1)))
      return fail(LAC_ERR_UNSUPPORTED, "%s: RMSNorm needs D/8 a power of two of at most 64 (D = %d)", fn, D);
    const int32_t st = check_norm(fn, norm_gain, norm_eps);
    if (st) return st;
  }
  lac::CompressArgs a{};
  a.norm_gain = norm ? norm_gain : nullptr;
  a.norm_eps = norm_eps;
  int32_t st = take_positions(fn, "pos0", pos0, B, T, m, &a.pos0);
  if (st) return st;
  if ((int64_t)B * N == 0) { g_err[0] = 0; return LAC_OK; }
  if (!raw_kv || !logits || !out) return fail(LAC_ERR_INVALID, "%s: null tensor pointer", fn);
  // MXFP4 rows (D/2 + D/32 bytes, written as 4-byte code words and scale
  // bytes) need only 4-byte alignment, so that a single row of a cache can
  // be the output
  if (!aligned(raw_kv, 16) || !aligned(logits, 16) || !aligned(out, out_dtype == LAC_MXFP4 ? 4 : 16))
    return fail(LAC_ERR_INVALID, "%s: tensor pointers must be 16-byte aligned (4 for MXFP4 output)", fn);
  if (out_dtype == LAC_KV_E4M3_ROPE_BF16 && (out_bstride * (int64_t)(D + rope_dims)) % 8)
    return fail(LAC_ERR_INVALID, "%s: mixed-format batch stride must keep rows 8-byte aligned", fn);
  a.kv = raw_kv; a.logits = logits; a.out = out;
  a.in_fmt = in_dtype; a.out_fmt = out_dtype;
  a.B = B; a.T = T; a.D = D; a.m = m; a.r = rope_dims; a.theta = rope_theta; a.overlap = overlap;
  a.kv_bstride = kv_bstride; a.z_bstride = z_bstride; a.out_bstride = out_bstride;
  if (g_group.open) {
    if ((st = group_stream(fn, stream))) return st;
    g_group.comp.push_back(a);
    g_err[0] = 0;
    return LAC_OK;
  }
  return launch_status(fn, lac::launch_compress(a, static_cast<hipStream_t>(stream)));
}

// indexer_topk and indexer_topk_noalloc.  With `fixed`, the workspace is the
// library's per-device scratch array (looked up only after every argument
// has been validated), and workspace_bytes is its size.
int32_t indexer_impl(const char* fn, const void* q_idx, const float* w, const void* k_idx,
                     int32_t dtype, int32_t B, int32_t Tq, int32_t H_I, int32_t d_I, int32_t N,
                     const int64_t* q_pos0, int32_t m, int32_t k, int32_t* topk_idx,
                     float* topk_score, void* workspace, size_t workspace_bytes, bool fixed,
                     void* stream) {
  const int round_bf16 = (dtype & LAC_SCORE_BF16) != 0;
  const int prepared = (dtype & LAC_TOPK_PREPARED) != 0;
  const bool q_e4m3 = (dtype & LAC_Q_E4M3) != 0;
  dtype &= ~(LAC_SCORE_BF16 | LAC_TOPK_PREPARED | LAC_Q_E4M3);
  if (q_e4m3 && dtype != LAC_MXFP4)
    return fail(LAC_ERR_UNSUPPORTED, "%s: LAC_Q_E4M3 applies to LAC_MXFP4 keys only", fn);
  if (prepared && fixed)
    return fail(LAC_ERR_INVALID, "%s: LAC_TOPK_PREPARED needs a caller's workspace", fn);
  if (dtype != LAC_F32 && dtype != LAC_BF16 && dtype != LAC_KV_E4M3_ROPE_BF16 && dtype != LAC_E4M3 &&
      dtype != LAC_MXFP4)
    return fail(LAC_ERR_UNSUPPORTED,
                "%s: dtype must be LAC_F32, LAC_BF16, LAC_KV_E4M3_ROPE_BF16, LAC_E4M3 or LAC_MXFP4", fn);
  if (B < 0 || B > LAC_MAX_BATCH) return fail(LAC_ERR_INVALID, "%s: B = %d outside [0, %d]", fn, B, LAC_MAX_BATCH);
  if (Tq < 0 || N < 0) return fail(LAC_ERR_INVALID, "%s: negative Tq or N", fn);
  if (m < 1) return fail(LAC_ERR_INVALID, "%s: m = %d < 1", fn, m);
  if (k < 1 || k > 8192) return fail(LAC_ERR_INVALID, "%s: k = %d outside [1, 8192]", fn, k);
  if (H_I < 1 || d_I < 1) return fail(LAC_ERR_INVALID, "%s: H_I and d_I must be >= 1", fn);
  if (dtype != LAC_F32) {
    if ((H_I != 32 && H_I != 64 && H_I != 128) || (d_I != 64 && d_I != 128))
      return fail(LAC_ERR_UNSUPPORTED, "%s: MFMA path needs H_I in {32, 64, 128} and d_I in {64, 128}", fn);
  } else if ((int64_t)H_I * d_I > 8192) {
    return fail(LAC_ERR_UNSUPPORTED, "%s: float32 path needs H_I * d_I <= 8192", fn);
  }
  if (q_e4m3 && d_I != 128)
    return fail(LAC_ERR_UNSUPPORTED, "%s: E4M3 queries with MXFP4 keys need d_I = 128", fn);
  lac::IndexerArgs a{};
  int32_t st = take_positions(fn, "q_pos0", q_pos0, B, Tq, 1, &a.qpos);
  if (st) return st;
  if ((int64_t)B * Tq == 0) { g_err[0] = 0; return LAC_OK; }
  if (!q_idx || !w || !topk_idx || (N > 0 && !k_idx)) return fail(LAC_ERR_INVALID, "%s: null tensor pointer", fn);
  if (!aligned(q_idx, 16) || !aligned(w, 4) || (k_idx && !aligned(k_idx, 16)) ||
      !aligned(topk_idx, 4) || (topk_score && !aligned(topk_score, 4)))
    return fail(LAC_ERR_INVALID, "%s: misaligned tensor pointer", fn);
  const size_t need = lac::indexer_workspace_bytes(B, Tq, N, k);
  if (fixed) {
    if (need > workspace_bytes)
      return fail(LAC_ERR_WORKSPACE,
                  "%s: this call needs %zu bytes of scratch, above the fixed %zu (use indexer_topk "
                  "with a workspace)", fn, need, workspace_bytes);
    const hipError_t e = lac::noalloc_scratch(&workspace);
    if (e != hipSuccess)
      return fail(LAC_ERR_DEVICE, "%s: no scratch address on the current device: %s", fn,
                  hipGetErrorString(e));
  } else {
    if (!workspace || !aligned(workspace, 256))
      return fail(LAC_ERR_WORKSPACE, "%s: workspace must be non-null and 256-byte aligned", fn);
    if (workspace_bytes < need)
      return fail(LAC_ERR_WORKSPACE, "%s: workspace of %zu bytes is below the %zu needed", fn, workspace_bytes, need);
  }
  a.q = q_idx; a.w = w; a.K = k_idx; a.fmt = q_e4m3 ? lac::kMX4E4 : dtype;
  a.round_bf16 = round_bf16; a.prepared = prepared;
  a.B = B; a.Tq = Tq; a.HI = H_I; a.dI = d_I; a.N = N; a.m = m; a.k = k;
  a.topk_idx = topk_idx; a.topk_score = topk_score;
  return launch_status(fn, lac::launch_indexer_topk(a, workspace, static_cast<hipStream_t>(stream)));
}

struct AttendCommon {
  const void* q; int32_t q_dtype; const void* kv; int32_t kv_dtype; int32_t N;
  const void* raw; int32_t T_raw; const int64_t* raw_pos0; int32_t W; const float* sink;
  float scale; int32_t B, Tq, H, D, r; float theta; const int64_t* q_pos0; void* out;
  void* ws; size_t ws_bytes; void* stream;
  const float* q_norm_gain = nullptr; float norm_eps = 0.f; bool norm = false;
};

int32_t attend_impl(const char* fn, const AttendCommon& c, int mode, const int32_t* idx, int32_t k,
                    int32_t m) {
  if (c.q_dtype != LAC_F32 && c.q_dtype != LAC_BF16)
    return fail(LAC_ERR_UNSUPPORTED, "%s: q_dtype must be LAC_F32 or LAC_BF16", fn);
  if (c.kv_dtype < LAC_F32 || c.kv_dtype > LAC_KV_E4M3_ROPE_BF16)
    return fail(LAC_ERR_UNSUPPORTED, "%s: unknown kv_dtype %d", fn, c.kv_dtype);
  if ((c.q_dtype == LAC_F32) != (c.kv_dtype == LAC_F32))
    return fail(LAC_ERR_UNSUPPORTED, "%s: float32 queries need a float32 KV and vice versa", fn);
  if (c.B < 0 || c.B > LAC_MAX_BATCH) return fail(LAC_ERR_INVALID, "%s: B = %d outside [0, %d]", fn, c.B, LAC_MAX_BATCH);
  if (c.Tq < 0 || c.N < 0 || c.T_raw < 0 || c.W < 0 || c.H < 1)
    return fail(LAC_ERR_INVALID, "%s: negative size or H < 1", fn);
  if (c.r < 0 || c.r > c.D || c.r > 128 || c.r % 8)
    return fail(LAC_ERR_INVALID, "%s: rope_dims = %d must be a multiple of 8 in [0, min(D, 128)]", fn, c.r);
  if (c.r > 0 && !(c.theta > 0.f && isfinite(c.theta)))
    return fail(LAC_ERR_INVALID, "%s: rope_theta must be positive and finite", fn);
  if (!isfinite(c.scale) || c.scale < 0.f) return fail(LAC_ERR_INVALID, "%s: softmax_scale must be finite and >= 0", fn);
  if (c.q_dtype == LAC_F32) {
    if (c.D < 8 || c.D > 256 || c.D % 8 || c.H * c.D > 8192)
      return fail(LAC_ERR_UNSUPPORTED, "%s: float32 path needs D in [8, 256] (multiple of 8) and H*D <= 8192", fn);
  } else {
    if (c.D != 128 && c.D != 256 && c.D != 512)
      return fail(LAC_ERR_UNSUPPORTED, "%s: bf16 path needs D in {128, 256, 512}", fn);
    if (!((c.H <= 64 && 64 % c.H == 0) || c.H % 64 == 0))
      return fail(LAC_ERR_UNSUPPORTED, "%s: bf16 path needs H dividing 64 or a multiple of 64", fn);
  }
  if (c.kv_dtype == LAC_KV_E4M3_ROPE_BF16 && (c.r % 32 || (c.D - c.r) % 32))
    return fail(LAC_ERR_UNSUPPORTED, "%s: the mixed KV format needs rope_dims and D - rope_dims multiples of 32", fn);
  if (mode == 0 && k < 0) return fail(LAC_ERR_INVALID, "%s: k = %d < 0", fn, k);
  if (mode == 1 && m < 1) return fail(LAC_ERR_INVALID, "%s: m = %d < 1", fn, m);
  if (c.norm) {
    const int32_t st = check_norm(fn, c.q_norm_gain, c.norm_eps);
    if (st) return st;
  }
  lac::AttendArgs a{};
  a.q_norm_gain = c.norm ? c.q_norm_gain : nullptr;
  a.norm_eps = c.norm_eps;
  int32_t st = take_positions(fn, "q_pos0", c.q_pos0, c.B, c.Tq, 1, &a.qpos);
  if (st) return st;
  st = take_positions(fn, "raw_pos0", c.raw_pos0, c.B, c.T_raw, 1, &a.rawpos);
  if (st) return st;
  if (c.W > 0) {
    for (int b = 0; b < c.B; ++b) {
      const int64_t qp = c.q_pos0 ? c.q_pos0[b] : 0, rp = c.raw_pos0 ? c.raw_pos0[b] : 0;
      const int64_t lo = qp - c.W + 1 > 0 ? qp - c.W + 1 : 0, hi = qp + c.Tq - 1;
      if (c.Tq > 0 && (lo < rp || hi >= rp + c.T_raw))
        return fail(LAC_ERR_INVALID,
                    "%s: raw window of batch %d needs positions [%lld, %lld] but raw_kv holds [%lld, %lld)",
                    fn, b, (long long)lo, (long long)hi, (long long)rp, (long long)(rp + c.T_raw));
    }
  }
  const int n_entries = mode == 0 ? k : c.N;
  const size_t need = lac::attend_workspace_bytes(c.B, c.Tq, c.H, c.D, c.r, c.kv_dtype, n_entries, c.W);
  if ((int64_t)c.B * c.Tq == 0) { g_err[0] = 0; return LAC_OK; }
  if (!c.q || !c.out) return fail(LAC_ERR_INVALID, "%s: null q or out", fn);
  if (c.N > 0 && !c.kv) return fail(LAC_ERR_INVALID, "%s: null compressed cache", fn);
  if (c.W > 0 && !c.raw) return fail(LAC_ERR_INVALID, "%s: null raw_kv with window > 0", fn);
  if (mode == 0 && k > 0 && !idx) return fail(LAC_ERR_INVALID, "%s: null topk_idx", fn);
  if (!aligned(c.q, 16) || !aligned(c.out, 16) || (c.kv && !aligned(c.kv, 16)) ||
      (c.raw && !aligned(c.raw, 16)) || (idx && !aligned(idx, 4)) || (c.sink && !aligned(c.sink, 4)))
    return fail(LAC_ERR_INVALID, "%s: misaligned tensor pointer", fn);
  if (need > 0 && (!c.ws || !aligned(c.ws, 256)))
    return fail(LAC_ERR_WORKSPACE, "%s: workspace must be non-null and 256-byte aligned", fn);
  if (c.ws_bytes < need)
    return fail(LAC_ERR_WORKSPACE, "%s: workspace of %zu bytes is below the %zu needed", fn, c.ws_bytes, need);
  a.q = c.q; a.kv = c.kv; a.idx = idx; a.raw = c.raw; a.sink = c.sink; a.out = c.out;
  a.q_fmt = c.q_dtype; a.kv_fmt = c.kv_dtype; a.mode = mode;
  a.N = c.N; a.k = mode == 0 ? k : 0; a.m = mode == 1 ? m : 1; a.T_raw = c.T_raw; a.W = c.W;
  a.B = c.B; a.Tq = c.Tq; a.H = c.H; a.D = c.D; a.r = c.r; a.theta = c.theta;
  a.scale = c.scale == 0.f ? 1.0f / sqrtf((float)c.D) : c.scale;
  a.n_entries = n_entries;
  if (lac::attend_split_count(a) > lac::kMaxSplit)
    return fail(LAC_ERR_UNSUPPORTED, "%s: %s too long for one launch (it would take more than %d key splits)",
                fn, mode == 0 ? "the selection" : "the compressed cache", lac::kMaxSplit);
  if (g_group.open) {
    if ((st = group_stream(fn, c.stream))) return st;
    g_group.att.push_back(a);
    g_group.att_ws.push_back(c.ws);
    g_group.att_need.push_back(need);
    g_err[0] = 0;
    return LAC_OK;
  }
  return launch_status(fn, lac::launch_attend(a, c.ws, static_cast<hipStream_t>(c.stream)));
}

}  // namespace

namespace lac {

void arm_timer(int kernel, hipEvent_t start, hipEvent_t stop) {
  g_timer_kernel = (start && stop) ? kernel : -1;
  g_timer_start = start;
  g_timer_stop = stop;
}

TimedLaunch::TimedLaunch(int kernel, hipStream_t st) {
  if (kernel == g_timer_kernel && g_timer_start) {
    (void)hipEventRecord(g_timer_start, st);
    stop_ = g_timer_stop;
    st_ = st;
    g_timer_kernel = -1;
  }
}

TimedLaunch::~TimedLaunch() {
  if (stop_) (void)hipEventRecord(stop_, st_);
}

}  // namespace lac

extern "C" {

int32_t csa_compress(const void* raw_kv, const void* logits, int32_t in_dtype, void* out,
                     int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                     int32_t rope_dims, float rope_theta, const int64_t* pos0,
                     int64_t kv_batch_stride, int64_t logit_batch_stride,
                     int64_t out_batch_stride, void* stream) {
  try {
    return compress_impl("csa_compress", raw_kv, logits, in_dtype, out, out_dtype, B, T, D, m,
                         rope_dims, rope_theta, pos0, kv_batch_stride, logit_batch_stride,
                         out_batch_stride, stream);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "csa_compress: internal error");
  }
}

int32_t hca_compress(const void* raw_kv, const void* logits, int32_t in_dtype, void* out,
                     int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                     int32_t rope_dims, float rope_theta, const int64_t* pos0,
                     int64_t kv_batch_stride, int64_t logit_batch_stride,
                     int64_t out_batch_stride, void* stream) {
  try {
    return compress_impl("hca_compress", raw_kv, logits, in_dtype, out, out_dtype, B, T, D, m,
                         rope_dims, rope_theta, pos0, kv_batch_stride, logit_batch_stride,
                         out_batch_stride, stream);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "hca_compress: internal error");
  }
}

int32_t csa_compress_overlap(const void* raw_kv, const void* logits, int32_t in_dtype, void* out,
                             int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                             int32_t overlap, int32_t rope_dims, float rope_theta,
                             const int64_t* pos0, int64_t kv_batch_stride,
                             int64_t logit_batch_stride, int64_t out_batch_stride, void* stream) {
  try {
    return compress_impl("csa_compress_overlap", raw_kv, logits, in_dtype, out, out_dtype, B, T, D,
                         m, rope_dims, rope_theta, pos0, kv_batch_stride, logit_batch_stride,
                         out_batch_stride, stream, nullptr, 0.f, false, overlap);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "csa_compress_overlap: internal error");
  }
}

int32_t csa_compress_rmsnorm(const void* raw_kv, const void* logits, int32_t in_dtype, void* out,
                             int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                             int32_t rope_dims, float rope_theta, const int64_t* pos0,
                             int64_t kv_batch_stride, int64_t logit_batch_stride,
                             int64_t out_batch_stride, const float* norm_gain, float norm_eps,
                             void* stream) {
  try {
    return compress_impl("csa_compress_rmsnorm", raw_kv, logits, in_dtype, out, out_dtype, B, T, D,
                         m, rope_dims, rope_theta, pos0, kv_batch_stride, logit_batch_stride,
                         out_batch_stride, stream, norm_gain, norm_eps, true);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "csa_compress_rmsnorm: internal error");
  }
}

int32_t hca_compress_rmsnorm(const void* raw_kv, const void* logits, int32_t in_dtype, void* out,
                             int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                             int32_t rope_dims, float rope_theta, const int64_t* pos0,
                             int64_t kv_batch_stride, int64_t logit_batch_stride,
                             int64_t out_batch_stride, const float* norm_gain, float norm_eps,
                             void* stream) {
  try {
    return compress_impl("hca_compress_rmsnorm", raw_kv, logits, in_dtype, out, out_dtype, B, T, D,
                         m, rope_dims, rope_theta, pos0, kv_batch_stride, logit_batch_stride,
                         out_batch_stride, stream, norm_gain, norm_eps, true);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "hca_compress_rmsnorm: internal error");
  }
}

size_t indexer_topk_workspace_size(int32_t B, int32_t Tq, int32_t N, int32_t k) {
  if (B < 0 || Tq < 0 || N < 0 || k < 1) return 0;
  return lac::indexer_workspace_bytes(B, Tq, N, k);
}

int32_t indexer_topk(const void* q_idx, const float* w, const void* k_idx, int32_t dtype,
                     int32_t B, int32_t Tq, int32_t H_I, int32_t d_I, int32_t N,
                     const int64_t* q_pos0, int32_t m, int32_t k, int32_t* topk_idx,
                     float* topk_score, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (g_group.open) return refuse_in_group("indexer_topk");
    return indexer_impl("indexer_topk", q_idx, w, k_idx, dtype, B, Tq, H_I, d_I, N, q_pos0, m, k,
                        topk_idx, topk_score, workspace, workspace_bytes, false, stream);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "indexer_topk: internal error");
  }
}

int32_t indexer_topk_noalloc(const void* q_idx, const float* w, const void* k_idx, int32_t dtype,
                             int32_t B, int32_t Tq, int32_t H_I, int32_t d_I, int32_t N,
                             const int64_t* q_pos0, int32_t m, int32_t k, int32_t* topk_idx,
                             float* topk_score, void* stream) {
  try {
    if (g_group.open) return refuse_in_group("indexer_topk_noalloc");
    return indexer_impl("indexer_topk_noalloc", q_idx, w, k_idx, dtype, B, Tq, H_I, d_I, N,
                        q_pos0, m, k, topk_idx, topk_score, nullptr, lac::kNoallocScratchBytes,
                        true, stream);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "indexer_topk_noalloc: internal error");
  }
}

int32_t indexer_topk_prepare(int32_t B, int32_t Tq, int32_t N, int32_t k, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const char* fn = "indexer_topk_prepare";
  try {
    if (B < 0 || B > LAC_MAX_BATCH) return fail(LAC_ERR_INVALID, "%s: B = %d outside [0, %d]", fn, B, LAC_MAX_BATCH);
    if (Tq < 0 || N < 0) return fail(LAC_ERR_INVALID, "%s: negative Tq or N", fn);
    if (k < 1 || k > 8192) return fail(LAC_ERR_INVALID, "%s: k = %d outside [1, 8192]", fn, k);
    const size_t need = lac::indexer_workspace_bytes(B, Tq, N, k);
    if (!workspace || !aligned(workspace, 256))
      return fail(LAC_ERR_WORKSPACE, "%s: workspace must be non-null and 256-byte aligned", fn);
    if (workspace_bytes < need)
      return fail(LAC_ERR_WORKSPACE, "%s: workspace of %zu bytes is below the %zu needed", fn, workspace_bytes, need);
    const lac::ClearJob c = lac::indexer_clear_job(B, Tq, N, k, workspace);
    if (g_group.open) {
      int32_t st = group_stream(fn, stream);
      if (st) return st;
      if (c.words) g_group.clears.push_back(c);
      g_err[0] = 0;
      return LAC_OK;
    }
    return launch_status(fn, lac::launch_clear(c, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "%s: internal error", fn);
  }
}

size_t attend_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t D, int32_t rope_dims,
                             int32_t kv_dtype, int32_t n_entries, int32_t window) {
  if (B < 0 || Tq < 0 || H < 1 || D < 8 || rope_dims < 0 || n_entries < 0 || window < 0) return 0;
  if (kv_dtype < LAC_F32 || kv_dtype > LAC_KV_E4M3_ROPE_BF16) return 0;
  return lac::attend_workspace_bytes(B, Tq, H, D, rope_dims, kv_dtype, n_entries, window);
}

int32_t csa_attend(const void* q, int32_t q_dtype, const void* ckv, int32_t kv_dtype, int32_t N,
                   const int32_t* topk_idx, int32_t k, const void* raw_kv, int32_t T_raw,
                   const int64_t* raw_pos0, int32_t window, const float* sink,
                   float softmax_scale, int32_t B, int32_t Tq, int32_t H, int32_t D,
                   int32_t rope_dims, float rope_theta, const int64_t* q_pos0, void* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  try {
    AttendCommon c{q, q_dtype, ckv, kv_dtype, N, raw_kv, T_raw, raw_pos0, window, sink,
                   softmax_scale, B, Tq, H, D, rope_dims, rope_theta, q_pos0, out, workspace,
                   workspace_bytes, stream};
    return attend_impl("csa_attend", c, 0, topk_idx, k, 1);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "csa_attend: internal error");
  }
}

int32_t hca_attend(const void* q, int32_t q_dtype, const void* hkv, int32_t kv_dtype, int32_t N,
                   int32_t m, const void* raw_kv, int32_t T_raw, const int64_t* raw_pos0,
                   int32_t window, const float* sink, float softmax_scale, int32_t B, int32_t Tq,
                   int32_t H, int32_t D, int32_t rope_dims, float rope_theta,
                   const int64_t* q_pos0, void* out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  try {
    AttendCommon c{q, q_dtype, hkv, kv_dtype, N, raw_kv, T_raw, raw_pos0, window, sink,
                   softmax_scale, B, Tq, H, D, rope_dims, rope_theta, q_pos0, out, workspace,
                   workspace_bytes, stream};
    return attend_impl("hca_attend", c, 1, nullptr, 0, m);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "hca_attend: internal error");
  }
}

int32_t csa_attend_rmsnorm(const void* q, int32_t q_dtype, const void* ckv, int32_t kv_dtype,
                           int32_t N, const int32_t* topk_idx, int32_t k, const void* raw_kv,
                           int32_t T_raw, const int64_t* raw_pos0, int32_t window,
                           const float* sink, float softmax_scale, int32_t B, int32_t Tq,
                           int32_t H, int32_t D, int32_t rope_dims, float rope_theta,
                           const int64_t* q_pos0, void* out, void* workspace,
                           size_t workspace_bytes, const float* q_norm_gain, float norm_eps,
                           void* stream) {
  try {
    AttendCommon c{q, q_dtype, ckv, kv_dtype, N, raw_kv, T_raw, raw_pos0, window, sink,
                   softmax_scale, B, Tq, H, D, rope_dims, rope_theta, q_pos0, out, workspace,
                   workspace_bytes, stream, q_norm_gain, norm_eps, true};
    return attend_impl("csa_attend_rmsnorm", c, 0, topk_idx, k, 1);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "csa_attend_rmsnorm: internal error");
  }
}

int32_t hca_attend_rmsnorm(const void* q, int32_t q_dtype, const void* hkv, int32_t kv_dtype,
                           int32_t N, int32_t m, const void* raw_kv, int32_t T_raw,
                           const int64_t* raw_pos0, int32_t window, const float* sink,
                           float softmax_scale, int32_t B, int32_t Tq, int32_t H, int32_t D,
                           int32_t rope_dims, float rope_theta, const int64_t* q_pos0, void* out,
                           void* workspace, size_t workspace_bytes, const float* q_norm_gain,
                           float norm_eps, void* stream) {
  try {
    AttendCommon c{q, q_dtype, hkv, kv_dtype, N, raw_kv, T_raw, raw_pos0, window, sink,
                   softmax_scale, B, Tq, H, D, rope_dims, rope_theta, q_pos0, out, workspace,
                   workspace_bytes, stream, q_norm_gain, norm_eps, true};
    return attend_impl("hca_attend_rmsnorm", c, 1, nullptr, 0, m);
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "hca_attend_rmsnorm: internal error");
  }
}

size_t grouped_projection_workspace_size(int32_t T, int32_t H, int32_t D, int32_t G, int32_t d_g,
                                         int32_t d) {
  if (T < 0 || H < 1 || D < 1 || G < 1 || H % G || d_g < 1 || d < 1) return 0;
  if ((int64_t)H * D > (1 << 22) || (int64_t)G * d_g > (1 << 22) || d > (1 << 22)) return 0;
  return lac::projection_workspace_bytes(T, H, D, G, d_g, d);
}

int32_t grouped_output_projection(const void* attn, const void* w1, const void* w2, int32_t T,
                                  int32_t H, int32_t D, int32_t G, int32_t d_g, int32_t d,
                                  void* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  const char* fn = "grouped_output_projection";
  try {
    if (g_group.open) return refuse_in_group(fn);
    if (T < 0 || H < 1 || D < 1 || G < 1 || d_g < 1 || d < 1)
      return fail(LAC_ERR_INVALID, "%s: negative T or a width < 1", fn);
    if (H % G) return fail(LAC_ERR_INVALID, "%s: G = %d does not divide H = %d", fn, G, H);
    const int64_t K1 = (int64_t)(H / G) * D, Y = (int64_t)G * d_g;
    if ((int64_t)H * D > (1 << 22) || Y > (1 << 22) || d > (1 << 22))
      return fail(LAC_ERR_UNSUPPORTED, "%s: H*D, G*d_g and d must be at most 2^22", fn);
    if (!lac::projection_shape_ok(K1, d_g, Y, d))
      return fail(LAC_ERR_UNSUPPORTED,
                  "%s: needs (H/G)*D and G*d_g multiples of 256, d_g and d multiples of 256", fn);
    if (T == 0) return LAC_OK;
    if (!attn || !w1 || !w2 || !out) return fail(LAC_ERR_INVALID, "%s: null tensor pointer", fn);
    if (!aligned(attn, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(out, 16))
      return fail(LAC_ERR_INVALID, "%s: tensor pointers must be 16-byte aligned", fn);
    const size_t need = grouped_projection_workspace_size(T, H, D, G, d_g, d);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
      return fail(LAC_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned and hold %zu bytes",
                  fn, need);
    lac::ProjectArgs p{attn, w1, w2, workspace, out, T, H, D, G, d_g, d};
    const hipStream_t st = static_cast<hipStream_t>(stream);
    lac::TimedLaunch tl(lac::kKernelProject, st);
    return launch_status(fn, lac::launch_projection(p, st));
  } catch (...) {
    return fail(LAC_ERR_DEVICE, "%s: internal error", fn);
  }
}

const char* lac_last_error(void) { return g_err; }

int32_t lac_group_begin(void* stream) {
  if (g_group.open)
    return fail(LAC_ERR_INVALID, "lac_group_begin: a launch group is already open on this thread");
  g_group.close();
  g_group.open = true;
  g_group.stream = stream;
  g_err[0] = 0;
  return LAC_OK;
}

int32_t lac_group_end(void* stream) {
  const char* fn = "lac_group_end";
  if (!g_group.open) return fail(LAC_ERR_INVALID, "%s: no launch group is open on this thread", fn);
  try {
    int32_t st = group_stream(fn, stream);
    // attention workspaces are written by the library: no two may overlap
    const size_t na = g_group.att.size();
    for (size_t i = 0; i < na && st == LAC_OK; ++i) {
      const uintptr_t lo_i = reinterpret_cast<uintptr_t>(g_group.att_ws[i]);
      for (size_t j = i + 1; j < na && st == LAC_OK; ++j) {
        const uintptr_t lo_j = reinterpret_cast<uintptr_t>(g_group.att_ws[j]);
        if (g_group.att_need[i] && g_group.att_need[j] && lo_i < lo_j + g_group.att_need[j] &&
            lo_j < lo_i + g_group.att_need[i])
          st = fail(LAC_ERR_WORKSPACE, "%s: attention calls %zu and %zu of the group share workspace memory",
                    fn, i, j);
      }
    }
    if (st) { g_group.close(); return st; }
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (!g_group.comp.empty() || !g_group.clears.empty())
      e = lac::launch_compress_group(g_group.comp.data(), (int)g_group.comp.size(), hs,
                                     g_group.clears.data(), (int)g_group.clears.size());
    if (e == hipSuccess && na)
      e = lac::launch_attend_group(g_group.att.data(), g_group.att_ws.data(), (int)na, hs);
    g_group.close();
    return launch_status(fn, e);
  } catch (...) {
    g_group.close();
    return fail(LAC_ERR_DEVICE, "%s: internal error", fn);
  }
}

int32_t lac_group_cancel(void) {
  if (!g_group.open) return fail(LAC_ERR_INVALID, "lac_group_cancel: no launch group is open on this thread");
  g_group.close();
  g_err[0] = 0;
  return LAC_OK;
}

int32_t lac_time_next_launch(int32_t kernel, void* start, void* stop) {
  if (kernel < 0 || kernel >= lac::kKernelCount)
    return fail(LAC_ERR_INVALID, "lac_time_next_launch: unknown kernel %d", kernel);
  lac::arm_timer(kernel, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop));
  return LAC_OK;
}

}  // extern "C"
