// project.hip -- grouped output projection.
//
// QbitAI rewrite (futuo-fx-trading.com), grouped output projection step: the
// head dimension is 512, so instead of one projection of all heads straight
// back to the model width d, the n_h heads are split into g groups, each
// group's concatenated output is projected to an intermediate width d_g, and
// the g results, concatenated, are projected back to d.  Both steps are
// dense bf16 products with fp32 accumulation:
//     y[t, g*d_g + j] = sum_c W1[g][j][c] * attn[t, g*(H/G)*D + c]
//     out[t, j]       = sum_c W2[j][c]    * y[t, c]
// Each is C[b] = A[b] * B[b]^T with both operands contiguous in the
// contraction index (activations [M, K], weights [N, K]), so one kernel runs
// both: the first batched over the groups, the second with one batch.
//
// Kernel.  A 256 x 256 output tile per block of eight waves (two per SIMD,
// so one wave's waits and barrier overlap the other's MFMAs), each wave a
// 128 x 64 part held as 4 x 2 v_mfma_f32_32x32x16_bf16 accumulators (128
// fp32 per lane).  Four waves of 128 x 128 each did 10% less work per second.  The contraction runs in
// steps of 32: per step the block stages a 256 x 32 slice of each operand in
// LDS with loads that write LDS directly (no registers), four slots deep, so
// a slice is requested three steps before it is read; the fragments of the
// next slice are read from LDS while the current one's MFMAs run.  Rows are
// 64 bytes; their four 16-byte chunks are XOR-swizzled by (row / 4) % 4.
// A 16-byte LDS read is served 16 lanes at a time over 64 four-byte banks
// (256 bytes): sixteen consecutive rows at one logical chunk then fill all
// 16 slots of the bank window (the rocprofv3 counter SQ_LDS_BANK_CONFLICT
// reads 0; keyed by row pair, which would suit 8 lanes over 32 banks, it
// reads half the LDS busy cycles).  Per
// 16-deep step a wave reads 4 A and 2 B fragments (6 KB from LDS) for 8
// MFMAs.  The MFMA takes the weight fragment as its first operand, so a
// lane's accumulator holds four runs of four consecutive output columns of
// one row and stores them as 8-byte pieces.
//
// Block order.  Blocks are dealt to the eight XCDs round robin; the kernel
// maps block i to tile (i % 8) * (tiles / 8) + i / 8, so each XCD sweeps a
// contiguous range of the tile order.  That order walks bands of 8 row tiles
// column by column, so the 32 blocks an XCD runs at once cover about 8 row
// tiles x 4 column tiles and share 12 operand slices through the XCD's L2
// (a row-major order would give 2 + 28 slices at d = 7168, all 28 weight
// slices streamed by every XCD).
#include "lac_internal.h"

namespace lac {

namespace {

constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kStages = 4;                       // LDS slices in flight
constexpr int kGroupM = 8;                       // row tiles per band of the tile order
constexpr int kRowB = kBK * 2;                   // bytes per staged row
constexpr int kSliceB = 256 * kRowB;             // bytes per staged operand slice

struct GemmArgs {
  const __bf16* A;        // [batch][M, K] rows lda apart, batch sA apart
  const __bf16* B;        // [batch][N, K] rows ldb apart, batch sB apart
  __bf16* C;              // [batch][M, N] rows ldc apart, batch sC apart
  int M, N, K;
  int64_t lda, ldb, ldc, sA, sB, sC;
  int mt, nt, tiles;      // tiles per batch (mt * nt) and in all batches
  int S;                  // contraction slices (grid = tiles * S)
  float* P;               // S > 1: fp32 partials [S][M][ldp], batch b at column b * N
  int64_t ldp;
};

// The staging loads write LDS directly and are tracked by hand: the waits and
// barriers below are written out (asm with a memory clobber, so the compiler
// neither moves LDS accesses across them nor adds waits of its own).
constexpr int kWaves = 8;                        // 2 (rows) x 4 (columns) waves per block
constexpr int kLoadsPerSlice = 2 * (256 / 16) / kWaves;   // staging loads per wave per slice

__device__ __forceinline__ void wait_vm(void) {
  // wait until all but the kStages - 2 newest slices' staging loads have landed
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerSlice * (kStages - 2)) : "memory");
}
__device__ __forceinline__ void wait_lds_reads(void) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
__device__ __forceinline__ void block_barrier(void) {
  asm volatile("s_barrier" ::: "memory");
}

__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_nt_bf16_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t lds[kStages][2][kSliceB];   // [stage][A | B]
  const int l = lane_id(), ln = l & 31, hf = l >> 5;
  const int wave = threadIdx.x >> 6, wm = wave >> 2, wn = wave & 3;

  // XCD-contiguous tile order (see the header); within a batch, bands of
  // kGroupM row tiles walked column by column.
  const int nb = gridDim.x;
  const int per_xcd = nb >> 3;
  int tile = blockIdx.x;
  if ((nb & 7) == 0) tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int split = tile / a.tiles;
  tile -= split * a.tiles;
  const int Ks = a.K / a.S, k_begin = split * Ks;
  const int batch = tile / (a.mt * a.nt);
  const int rem = tile - batch * a.mt * a.nt;
  const int band = rem / (kGroupM * a.nt), in_band = rem - band * kGroupM * a.nt;
  const int rows_in_band = min(a.mt - band * kGroupM, kGroupM);
  const int m0 = (band * kGroupM + in_band % rows_in_band) * kBM;
  const int n0 = (in_band / rows_in_band) * kBN;

  // Both operands are read through buffer resources based at the tile's
  // first row: the contraction offset goes in the scalar offset, and rows
  // past M fall outside the A resource, which returns zeros for them (their
  // results are never stored).
  const __bf16* At = a.A + batch * a.sA + (int64_t)m0 * a.lda + k_begin;
  const __bf16* Bt = a.B + batch * a.sB + (int64_t)n0 * a.ldb + k_begin;
  const int64_t a_bytes = ((int64_t)(a.M - 1 - m0) * a.lda + Ks) * 2;
  const int64_t b_bytes = ((int64_t)(kBN - 1) * a.ldb + Ks) * 2;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(At), 0, (int)min(a_bytes, (int64_t)0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(Bt), 0, (int)min(b_bytes, (int64_t)0x7fffffff), 0x00020000);

  // Staging: a load instruction fills 1 KB of LDS, lane i the 16 bytes at
  // 16 i, i.e. rows of 64 bytes, lane i at row i / 4, slot i % 4.  Slot s of
  // row r holds the row's chunk s ^ ((r / 4) % 4), so each lane fetches that
  // chunk.  Wave w stages rows 32 w .. 32 w + 31 of both operands (2 loads
  // each).
  constexpr int kRowsPerWave = 256 / kWaves;
  int aofs[kRowsPerWave / 16], bofs[kRowsPerWave / 16];
#pragma unroll
  for (int u = 0; u < kRowsPerWave / 16; ++u) {
    const int row = wave * kRowsPerWave + u * 16 + (l >> 2);
    const int chunk = (l & 3) ^ ((row >> 2) & 3);
    aofs[u] = (int)((int64_t)row * a.lda * 2) + chunk * 16;
    bofs[u] = (int)((int64_t)row * a.ldb * 2) + chunk * 16;
  }
  typedef __attribute__((address_space(3))) void lds_void;
  auto stage = [&](int slot, int k0) {
#pragma unroll
    for (int u = 0; u < kRowsPerWave / 16; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_void*)&lds[slot][0][(wave * kRowsPerWave + u * 16) * kRowB], 16, aofs[u],
          k0 * 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (lds_void*)&lds[slot][1][(wave * kRowsPerWave + u * 16) * kRowB], 16, bofs[u],
          k0 * 2, 0, 0);
    }
  };

  constexpr int NJ = 2;                   // 32-column tiles per wave
  f32x16 acc[NJ][4];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x16{};

  // Fragment rows: A row wm*128 + i*32 + ln, B row wn*64 + j*32 + ln; the
  // row's swizzle key is (ln / 4) % 4 (the tile offsets are multiples of 32).
  // F[kk][0..3] are the A fragments of 16-deep step kk, F[kk][4..7] the B ones.
  const int arow = (wm * 128 + ln) * kRowB, brow = (wn * 32 * NJ + ln) * kRowB;
  typedef bf16x8 Frags[kBK / 16][4 + NJ];
  auto read_frags = [&](int slot, Frags& F) {
    const uint8_t* la = lds[slot][0];
    const uint8_t* lb = lds[slot][1];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int cofs = ((kk * 2 + hf) ^ ((ln >> 2) & 3)) << 4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        F[kk][i] = *reinterpret_cast<const bf16x8*>(la + arow + i * 32 * kRowB + cofs);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        F[kk][4 + j] = *reinterpret_cast<const bf16x8*>(lb + brow + j * 32 * kRowB + cofs);
    }
  };
  auto mfmas = [&](const Frags& F) {
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[kk][4 + j], F[kk][i], acc[j][i],
                                                              0, 0, 0);
  };

  // All kStages slots are filled before the loop.  Step kt holds the
  // fragments of slice kt in registers (read during step kt - 1); it waits
  // for slice kt + 1, passes the barrier (every wave's part of slice kt + 1
  // has landed and every wave's reads of slot kt % kStages are complete),
  // refills that slot with slice kt + kStages, reads the fragments of slice
  // kt + 1 and runs the MFMAs of slice kt, so LDS reads overlap a step of
  // MFMAs and a slice is requested kStages - 1 steps before it is read.
  // Slices past the last one reload it (in bounds, never used), so every wave
  // issues the same loads each step and the wait count is constant.
  const int nk = Ks / kBK;               // even
#pragma unroll
  for (int s = 0; s < kStages; ++s) stage(s, min(s, nk - 1) * kBK);
  Frags F0, F1;
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerSlice * (kStages - 1)) : "memory");
  block_barrier();
  read_frags(0, F0);
  auto step = [&](int kt, const Frags& cur, Frags& next) {
    // The scheduling barriers keep each step's MFMAs inside the step (they
    // touch no memory, so nothing else would stop the compiler from pulling
    // the next step's MFMAs up to right after their fragment reads).
    __builtin_amdgcn_sched_barrier(0);
    wait_vm();
    wait_lds_reads();
    block_barrier();
    stage(kt % kStages, min(kt + kStages, nk - 1) * kBK);
    read_frags((kt + 1) % kStages, next);
    mfmas(cur);
    // Order inside the step: the staging loads, then one fragment read per
    // two MFMAs, so the reads for the next step start early and spread out.
    __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerSlice, 0);   // VMEM reads
#pragma unroll
    for (int g = 0; g < 2 * (4 + NJ); ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * 4 * NJ - 2 * (4 + NJ), 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, F0, F1);
    step(kt + 1, F1, F0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no LDS write may outlive the block

  // acc[j][i][v]: column n0 + wn*64 + j*32 + 8*(v/4) + 4*hf + v%4 of row
  // m0 + wm*128 + i*32 + ln.
  if (a.S > 1) {                         // fp32 partials of this slice
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + wm * 128 + i * 32 + ln;
      if (row < a.M) {
        float* pr = a.P + ((int64_t)split * a.M + row) * a.ldp + batch * a.N + n0 + wn * 32 * NJ +
                    4 * hf;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& c = acc[j][i];
            *reinterpret_cast<f32x4*>(pr + j * 32 + 8 * g) =
                f32x4{c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]};
          }
      }
    }
    return;
  }
  __bf16* Cb = a.C + batch * a.sC;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + i * 32 + ln;
    if (row < a.M) {
      __bf16* cr = Cb + (int64_t)row * a.ldc + n0 + wn * 32 * NJ + 4 * hf;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& c = acc[j][i];
          const uint2 v = make_uint2(pack_bf16x2(c[4 * g], c[4 * g + 1]),
                                     pack_bf16x2(c[4 * g + 2], c[4 * g + 3]));
          *reinterpret_cast<uint2*>(cr + j * 32 + 8 * g) = v;
        }
    }
  }
}

// ---------------------------------------------------------------- few tokens
// With a few tokens (decode) the products stream the weights once and do
// little arithmetic, so the tiled kernel above would leave most of the chip
// idle.  Here each wave owns 32 weight rows and one of S slices of the
// contraction, and keeps all tokens (TT tiles of 32) in the MFMA's second
// operand: a 128-deep step is eight MFMAs, each fed by one 16-byte load per
// lane from its own row, two steps in flight (a whole slice, usually).  Each load touches one line
// per row, and the step's eight loads the same 32 lines, so the weights are
// read with the default cache policy: with the streaming hint the lines left
// the cache between the loads and every weight byte crossed HBM about eight
// times.  The S partial sums go to workspace in fp32 and a second kernel
// adds them in a fixed order and rounds to bf16, so results do not depend on
// timing.
constexpr int kSkinnyMaxT = 64;
constexpr int kSkinnyStep = 128;                 // contraction per step
constexpr int kSkinnyMinSteps = 2;               // steps per wave at least

struct SkinnyArgs {
  const __bf16* W;        // [batch][N, K] rows ldw apart, batch sW apart
  const __bf16* X;        // [batch][T, K] rows ldx apart, batch sX apart
  float* P;               // [S][T][ldp] partial sums; batch b at column b * N
  int T, N, K, S, batches;
  int64_t ldw, sW, ldx, sX, ldp;
};

template <int TT>
__global__ void __launch_bounds__(256) gemm_skinny_kernel(SkinnyArgs a) {
  const int l = lane_id(), ln = l & 31, hf = l >> 5;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rtiles = a.N / 32;
  const int per_batch = rtiles * a.S;
  if (wid >= per_batch * a.batches) return;
  const int batch = wid / per_batch;
  const int r = wid - batch * per_batch;
  const int split = r / rtiles, rt = r - split * rtiles;   // neighbouring waves: neighbouring rows
  const int Ks = a.K / a.S;
  const int k0 = split * Ks;
  const __bf16* Wt = a.W + batch * a.sW + (int64_t)rt * 32 * a.ldw + k0;
  const __bf16* Xt = a.X + batch * a.sX + k0;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(Wt), 0, (int)min(((int64_t)31 * a.ldw + Ks) * 2, (int64_t)0x7fffffff),
      0x00020000);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(Xt), 0, (int)min(((int64_t)(a.T - 1) * a.ldx + Ks) * 2, (int64_t)0x7fffffff),
      0x00020000);
  // Load c of a step gives lane (ln, hf) the 16 bytes at 32 c + 16 hf of its
  // row's 256-byte stretch, so one load touches one line per row.  Token
  // lanes past T read row T - 1 again (same lines, results never stored).
  const int wofs = (int)((int64_t)ln * a.ldw * 2) + hf * 16;
  int xofs[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
    xofs[tt] = (int)((int64_t)min(tt * 32 + ln, a.T - 1) * a.ldx * 2) + hf * 16;

  typedef u32x4 Step[1 + TT][8];          // [weights | token tiles][chunk]
  auto load = [&](Step& b, int kk) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      b[0][c] = __builtin_amdgcn_raw_buffer_load_b128(rw, wofs + c * 32, kk * 2, 0);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        b[1 + tt][c] = __builtin_amdgcn_raw_buffer_load_b128(rx, xofs[tt] + c * 32, kk * 2, 0);
  };
  f32x16 acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[tt] = f32x16{};
  auto mfmas = [&](const Step& b) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, b[0][c]), __builtin_bit_cast(bf16x8, b[1 + tt][c]),
            acc[tt], 0, 0, 0);
  };
  // Two steps per round, both in flight at once (the usual slice is one
  // round); the loads are unconditional, so the memory-counter waits are exact.
  const int ns = Ks / kSkinnyStep;        // even
  for (int s = 0; s < ns; s += 2) {
    Step b0, b1;
    load(b0, s * kSkinnyStep);
    load(b1, (s + 1) * kSkinnyStep);
    mfmas(b0);
    mfmas(b1);
  }

  // acc[tt][v]: weight row 32 rt + 8 (v / 4) + 4 hf + v % 4, token 32 tt + ln.
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int t = tt * 32 + ln;
    if (t < a.T) {
      float* pr = a.P + ((int64_t)split * a.T + t) * a.ldp + batch * a.N + rt * 32 + 4 * hf;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(pr + 8 * g) =
            f32x4{acc[tt][4 * g], acc[tt][4 * g + 1], acc[tt][4 * g + 2], acc[tt][4 * g + 3]};
    }
  }
}

// out[t, n] = bf16(sum over s of P[s][t][n]), s in order; four columns per thread.
__global__ void __launch_bounds__(256) split_sum_kernel(const float* P, int S, int T, int64_t ldp,
                                                        int ncols, __bf16* out, int64_t ldo) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= (int64_t)T * ncols) return;
  const int t = (int)(e / ncols), n = (int)(e - (int64_t)t * ncols);
  // loads in groups of up to 16 (S is a power of two, at most 64), each
  // group's loads issued together, then added in order
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 16) {
    f32x4 part[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s0 + s < S)
        part[s] = *reinterpret_cast<const f32x4*>(P + ((int64_t)(s0 + s) * T + t) * ldp + n);
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s0 + s < S) sum += part[s];
  }
  *reinterpret_cast<uint2*>(out + (int64_t)t * ldo + n) =
      make_uint2(pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3]));
}

// Contraction slices for the few-token kernel: enough waves to keep HBM busy
// (about 16 per compute unit, all loads of a wave in flight at once when it
// has two steps), each at least kSkinnyMinSteps steps long, a power of two
// (at most 64) that divides K / kSkinnyStep into an even count.
int skinny_splits(int64_t rows, int64_t K) {
  const int64_t steps = K / kSkinnyStep;
  int S = 1;
  while (S < 64 && rows / 32 * S < 4096 && steps % (2 * S * 2) == 0 &&
         steps / (2 * S) >= kSkinnyMinSteps)
    S *= 2;
  return S;
}

hipError_t launch_skinny(const SkinnyArgs& s0, int S, hipStream_t st) {
  SkinnyArgs s = s0;
  s.S = S;
  const int waves = s.N / 32 * S * s.batches;
  const int blocks = (waves + 3) / 4;
  if (s.T <= 32)
    hipLaunchKernelGGL(gemm_skinny_kernel<1>, dim3(blocks), dim3(256), 0, st, s);
  else
    hipLaunchKernelGGL(gemm_skinny_kernel<2>, dim3(blocks), dim3(256), 0, st, s);
  return hipGetLastError();
}

hipError_t launch_split_sum(const float* P, int S, int T, int64_t ldp, int ncols, __bf16* out,
                            int64_t ldo, hipStream_t st) {
  const int64_t quads = (int64_t)T * ncols / 4;
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st,
                     P, S, T, ldp, ncols, out, ldo);
  return hipGetLastError();
}

// Contraction slices for the tiled kernel: with fewer tiles than compute
// units, split the contraction until the grid covers the chip, keeping at
// least 8 (an even number of) 32-deep steps per slice.
int tiled_splits(int64_t tiles, int64_t K) {
  int S = 1;
  while (tiles * S < 256 && (K / kBK) % (4 * S) == 0 && K / kBK / (2 * S) >= 8) S *= 2;
  return S;
}

// With S > 1 the kernel writes fp32 partials to P and split_sum_kernel adds
// them in order into C (the column offset of batch b is b * N in both).
hipError_t launch_gemm(const GemmArgs& g0, int batches, float* P, hipStream_t st) {
  GemmArgs g = g0;
  g.mt = (g.M + kBM - 1) / kBM;
  g.nt = g.N / kBN;
  g.tiles = g.mt * g.nt * batches;
  if (g.tiles == 0) return hipSuccess;
  g.S = tiled_splits(g.tiles, g.K);
  g.P = P;
  g.ldp = (int64_t)g.N * batches;
  hipLaunchKernelGGL(gemm_nt_bf16_kernel, dim3(g.tiles * g.S), dim3(64 * kWaves), 0, st, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.S == 1) return e;
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)(((int64_t)g.M * g.ldp / 4 + 255) / 256)),
                     dim3(256), 0, st, P, g.S, g.M, g.ldp, (int)g.ldp, g.C, g.ldc);
  return hipGetLastError();
}

}  // namespace

size_t projection_workspace_bytes(int T, int H, int D, int G, int d_g, int d) {
  const int64_t K1 = (int64_t)(H / G) * D, Y = (int64_t)G * d_g;
  size_t bytes = (((size_t)T * Y * 2) + 255) & ~(size_t)255;       // y
  if (T <= kSkinnyMaxT) {
    const size_t p1 = (size_t)skinny_splits(Y, K1) * T * Y * 4;
    const size_t p2 = (size_t)skinny_splits(d, Y) * T * d * 4;
    bytes += p1 > p2 ? p1 : p2;
  } else {
    const int64_t mt = (T + kBM - 1) / kBM;
    const int S1 = tiled_splits(mt * (d_g / kBN) * G, K1), S2 = tiled_splits(mt * (d / kBN), Y);
    const size_t p1 = S1 > 1 ? (size_t)S1 * T * Y * 4 : 0;
    const size_t p2 = S2 > 1 ? (size_t)S2 * T * d * 4 : 0;
    bytes += p1 > p2 ? p1 : p2;
  }
  return bytes;
}

bool projection_shape_ok(int64_t K1, int64_t d_g, int64_t Kout, int64_t d) {
  return K1 % (2 * kSkinnyStep) == 0 && Kout % (2 * kSkinnyStep) == 0 && d_g % kBN == 0 &&
         d % kBN == 0;
}

hipError_t launch_projection(const ProjectArgs& p, hipStream_t st) {
  const int64_t K1 = (int64_t)(p.H / p.G) * p.D, Y = (int64_t)p.G * p.d_g;
  if (p.T <= kSkinnyMaxT) {
    __bf16* y = static_cast<__bf16*>(p.y);
    float* P = reinterpret_cast<float*>(static_cast<uint8_t*>(p.y) +
                                        ((((size_t)p.T * Y * 2) + 255) & ~(size_t)255));
    SkinnyArgs s1{};
    s1.W = static_cast<const __bf16*>(p.w1);
    s1.X = static_cast<const __bf16*>(p.attn);
    s1.P = P;
    s1.T = p.T;
    s1.N = p.d_g;
    s1.K = (int)K1;
    s1.batches = p.G;
    s1.ldw = K1;
    s1.sW = (int64_t)p.d_g * K1;
    s1.ldx = (int64_t)p.H * p.D;
    s1.sX = K1;
    s1.ldp = Y;
    const int S1 = skinny_splits(Y, K1);
    hipError_t e = launch_skinny(s1, S1, st);
    if (e == hipSuccess) e = launch_split_sum(P, S1, p.T, Y, (int)Y, y, Y, st);
    if (e != hipSuccess) return e;
    SkinnyArgs s2{};
    s2.W = static_cast<const __bf16*>(p.w2);
    s2.X = y;
    s2.P = P;
    s2.T = p.T;
    s2.N = p.d;
    s2.K = (int)Y;
    s2.batches = 1;
    s2.ldw = Y;
    s2.ldx = Y;
    s2.ldp = p.d;
    const int S2 = skinny_splits(p.d, Y);
    e = launch_skinny(s2, S2, st);
    if (e == hipSuccess)
      e = launch_split_sum(P, S2, p.T, p.d, p.d, static_cast<__bf16*>(p.out), p.d, st);
    return e;
  }
  GemmArgs g1{};
  g1.A = static_cast<const __bf16*>(p.attn);
  g1.B = static_cast<const __bf16*>(p.w1);
  g1.C = static_cast<__bf16*>(p.y);
  g1.M = p.T;
  g1.N = p.d_g;
  g1.K = (int)K1;
  g1.lda = (int64_t)p.H * p.D;
  g1.ldb = K1;
  g1.ldc = Y;
  g1.sA = K1;
  g1.sB = (int64_t)p.d_g * K1;
  g1.sC = p.d_g;
  float* P = reinterpret_cast<float*>(static_cast<uint8_t*>(p.y) +
                                      ((((size_t)p.T * Y * 2) + 255) & ~(size_t)255));
  hipError_t e = launch_gemm(g1, p.G, P, st);
  if (e != hipSuccess) return e;
  GemmArgs g2{};
  g2.A = static_cast<const __bf16*>(p.y);
  g2.B = static_cast<const __bf16*>(p.w2);
  g2.C = static_cast<__bf16*>(p.out);
  g2.M = p.T;
  g2.N = p.d;
  g2.K = (int)Y;
  g2.lda = Y;
  g2.ldb = Y;
  g2.ldc = p.d;
  return launch_gemm(g2, 1, P, st);
}

}  // namespace lac
