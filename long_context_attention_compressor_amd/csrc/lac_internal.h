// lac_internal.h -- launch interfaces between the C ABI (abi.cpp) and the
// kernel files.  Everything here is host-visible and takes plain values.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lac_device.h"

namespace lac {

enum KernelId {
  kKernelCompress = 0,
  kKernelIndexerScore = 1,
  kKernelTopk = 2,
  kKernelAttend = 3,
  kKernelCombine = 4,
  kKernelProject = 5,
  kKernelCount = 6
};

// One-shot, thread-local launch timer (see lac_time_next_launch).  Records the
// armed start event on construction and the stop event on destruction when
// this launch is of the armed kernel.
struct TimedLaunch {
  TimedLaunch(int kernel, hipStream_t st);
  ~TimedLaunch();
  hipEvent_t stop_ = nullptr;
  hipStream_t st_ = nullptr;
};
void arm_timer(int kernel, hipEvent_t start, hipEvent_t stop);

// Device words to zero: the indexer workspace's counters (indexer_clear_job),
// done by a small fill launch (launch_clear) or inside a compress launch.
struct ClearJob {
  uint32_t* p;
  uint64_t words;        // a multiple of 64
};

// ---------------------------------------------------------------- compress
struct CompressArgs {
  const void* kv;
  const void* logits;
  void* out;
  int in_fmt, out_fmt;
  int B, T, D, m, r;
  int overlap;            // CSA window overlap o (tokens before the block), 0 = none
  float theta;
  int64_t kv_bstride, z_bstride, out_bstride;  // rows
  const float* norm_gain;   // [D] or null: RMSNorm of each entry before its rotation
  float norm_eps;
  Positions pos0;
};
hipError_t launch_compress(CompressArgs a, hipStream_t st);
// n independent calls (none reads what another writes), in as few launches
// as their input formats and the launch's argument pools allow.
hipError_t launch_compress_group(const CompressArgs* calls, int n, hipStream_t st,
                                 const ClearJob* clears = nullptr, int n_clears = 0);
// Launch limit: a call's workgroups, at most B * floor(T/m) * D/8, stay below 2^31.
constexpr int64_t kCompressMaxGroups = (int64_t)1 << 31;

// ---------------------------------------------------------------- indexer + top-k
struct IndexerArgs {
  const void* q;         // [B, Tq, HI, dI]
  const float* w;        // [B, Tq, HI]
  const void* K;         // [B, N, dI]
  int fmt;               // kF32 | kBF16 | kMixed (E4M3 keys) | kE4M3 (E4M3 queries and keys) | kMXFP4 (MXFP4 keys)
                         // | kMX4E4 (MXFP4 keys, E4M3 queries)
  int round_bf16;        // scores rounded to bf16 before selection
  int prepared;          // the workspace's counters are already zero (indexer_topk_prepare)
  int B, Tq, HI, dI, N, m, k;
  int32_t* topk_idx;     // [B, Tq, k]
  float* topk_score;     // [B, Tq, k] or null
  Positions qpos;
};
size_t indexer_workspace_bytes(int B, int Tq, int N, int k);
ClearJob indexer_clear_job(int B, int Tq, int N, int k, void* ws);
hipError_t launch_clear(const ClearJob& c, hipStream_t st);
// Lightning-Indexer scores (score.hip) into the top-k workspace: the score
// rows, and on the split path the key histogram and the tile counters, both
// cleared beforehand.  nv_max: largest visible count over the rows.
constexpr int kScoreHistBins = 4096;   // top-12-bit key histogram bins
struct ScoreBuffers {
  float* scores;          // [R, Np]
  int64_t Np;
  uint32_t* hist;         // [R, kScoreHistBins] or null
  uint32_t* tile_ctr;     // [R, 16 * 32] or null
  bool split;
};
hipError_t launch_indexer_scores(const IndexerArgs& a, const ScoreBuffers& sb, int64_t nv_max,
                                 hipStream_t st);
hipError_t launch_indexer_topk(const IndexerArgs& a, void* ws, hipStream_t st);

// ---------------------------------------------------------------- fixed scratch
// Size of the per-device scratch array of the allocation-free entry point, and
// its device address on the current device (looked up once per device).
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

// ---------------------------------------------------------------- attention
struct AttendArgs {
  const void* q;          // [B, Tq, H, D]
  const void* kv;         // [B, N, row]
  const int32_t* idx;     // [B, Tq, k] (CSA) or null (HCA)
  const void* raw;        // [B, T_raw, row]
  const float* sink;      // [H] or null
  void* out;              // [B, Tq, H, D]
  int q_fmt, kv_fmt;
  int mode;               // 0 = CSA, 1 = HCA
  int N, k, m, T_raw, W;
  int B, Tq, H, D, r;
  float theta, scale;
  int n_entries;          // k (CSA) or N (HCA): sizes the split plan
  Positions qpos, rawpos;
  const float* q_norm_gain;   // [D] or null: RMSNorm of each query head before its rotation
  float norm_eps;
};
size_t attend_workspace_bytes(int B, int Tq, int H, int D, int r, int kv_fmt, int n_entries,
                              int W);
// Splits of the key range per work item that a launch would use; a launch
// refuses more than kMaxSplit (the combine step keeps one weight per split in LDS).
constexpr int kMaxSplit = 2048;
int attend_split_count(const AttendArgs& a);
hipError_t launch_attend(const AttendArgs& a, void* ws, hipStream_t st);
// n independent calls (none reads what another writes; workspaces disjoint),
// their splits planned together so that they share one wave of workgroups,
// in one attention launch (and one combine launch) per kernel instance.
hipError_t launch_attend_group(const AttendArgs* calls, void* const* ws, int n, hipStream_t st);

// ---------------------------------------------------------------- grouped output projection
struct ProjectArgs {
  const void* attn;       // [T, H, D] bf16
  const void* w1;         // [G, d_g, (H/G)*D] bf16
  const void* w2;         // [d, G*d_g] bf16
  void* y;                // workspace: y [T, G*d_g] bf16, then split partial sums
  void* out;              // [T, d] bf16
  int T, H, D, G, d_g, d;
};
// Contraction widths K1 = (H/G)*D and G*d_g, output widths d_g and d that the
// product kernel tiles exactly.
bool projection_shape_ok(int64_t K1, int64_t d_g, int64_t Kout, int64_t d);
// Workspace: y [T, G*d_g] bf16, and for T <= 64 the split partial sums after it.
size_t projection_workspace_bytes(int T, int H, int D, int G, int d_g, int d);
hipError_t launch_projection(const ProjectArgs& p, hipStream_t st);

}  // namespace lac
