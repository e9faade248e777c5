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
// Kernel.  A 256 x 256 output tile per block of four waves, each wave a
// 128 x 128 quarter held as 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators
// (256 fp32 per lane, in the accumulator registers).  The contraction runs in
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
// 16-deep step a wave reads 4 A and 4 B fragments (8 KB from LDS) for 16
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
  int mt, nt, tiles;      // tiles per batch (mt * nt) and in all
};

// The staging loads write LDS directly and are tracked by hand: the waits and
// barriers below are written out (asm with a memory clobber, so the compiler
// neither moves LDS accesses across them nor adds waits of its own).
__device__ __forceinline__ void wait_vm(void) {
  // every wave has 8 staging loads per slice; wait until all but the
  // kStages - 2 newest slices have landed
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(8 * (kStages - 2)) : "memory");
}
__device__ __forceinline__ void wait_lds_reads(void) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
__device__ __forceinline__ void block_barrier(void) {
  asm volatile("s_barrier" ::: "memory");
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_nt_bf16_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t lds[kStages][2][kSliceB];   // [stage][A | B]
  const int l = lane_id(), ln = l & 31, hf = l >> 5;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;

  // XCD-contiguous tile order (see the header); within a batch, bands of
  // kGroupM row tiles walked column by column.
  const int nb = gridDim.x;
  const int per_xcd = nb >> 3;
  int tile = blockIdx.x;
  if ((nb & 7) == 0) tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
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
  const __bf16* At = a.A + batch * a.sA + (int64_t)m0 * a.lda;
  const __bf16* Bt = a.B + batch * a.sB + (int64_t)n0 * a.ldb;
  const int64_t a_bytes = ((int64_t)(a.M - 1 - m0) * a.lda + a.K) * 2;
  const int64_t b_bytes = ((int64_t)(kBN - 1) * a.ldb + a.K) * 2;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(At), 0, (int)min(a_bytes, (int64_t)0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(Bt), 0, (int)min(b_bytes, (int64_t)0x7fffffff), 0x00020000);

  // Staging: a load instruction fills 1 KB of LDS, lane i the 16 bytes at
  // 16 i, i.e. rows of 64 bytes, lane i at row i / 4, slot i % 4.  Slot s of
  // row r holds the row's chunk s ^ ((r / 4) % 4), so each lane fetches that
  // chunk.  Wave w stages rows 64 w .. 64 w + 63 of both operands (4 loads
  // each).
  int aofs[4], bofs[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = wave * 64 + u * 16 + (l >> 2);
    const int chunk = (l & 3) ^ ((row >> 2) & 3);
    aofs[u] = (int)((int64_t)row * a.lda * 2) + chunk * 16;
    bofs[u] = (int)((int64_t)row * a.ldb * 2) + chunk * 16;
  }
  typedef __attribute__((address_space(3))) void lds_void;
  auto stage = [&](int slot, int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_void*)&lds[slot][0][(wave * 64 + u * 16) * kRowB], 16, aofs[u], k0 * 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (lds_void*)&lds[slot][1][(wave * 64 + u * 16) * kRowB], 16, bofs[u], k0 * 2, 0, 0);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x16{};

  // Fragment rows: A row wm*128 + i*32 + ln, B row wn*128 + j*32 + ln; the
  // row's swizzle key is (ln / 4) % 4 (the tile offsets are multiples of 32).
  // F[kk][0..3] are the A fragments of 16-deep step kk, F[kk][4..7] the B ones.
  const int arow = (wm * 128 + ln) * kRowB, brow = (wn * 128 + ln) * kRowB;
  typedef bf16x8 Frags[kBK / 16][8];
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
      for (int j = 0; j < 4; ++j)
        F[kk][4 + j] = *reinterpret_cast<const bf16x8*>(lb + brow + j * 32 * kRowB + cofs);
    }
  };
  auto mfmas = [&](const Frags& F) {
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j)
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
  const int nk = a.K / kBK;              // even
#pragma unroll
  for (int s = 0; s < kStages; ++s) stage(s, min(s, nk - 1) * kBK);
  Frags F0, F1;
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(8 * (kStages - 1)) : "memory");
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
    __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);        // VMEM reads
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // MFMA
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, F0, F1);
    step(kt + 1, F1, F0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no LDS write may outlive the block

  // acc[j][i][v]: column n0 + wn*128 + j*32 + 8*(v/4) + 4*hf + v%4 of row
  // m0 + wm*128 + i*32 + ln.
  __bf16* Cb = a.C + batch * a.sC;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + i * 32 + ln;
    if (row < a.M) {
      __bf16* cr = Cb + (int64_t)row * a.ldc + n0 + wn * 128 + 4 * hf;
#pragma unroll
      for (int j = 0; j < 4; ++j)
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

hipError_t launch_gemm(const GemmArgs& g0, int batches, hipStream_t st) {
  GemmArgs g = g0;
  g.mt = (g.M + kBM - 1) / kBM;
  g.nt = g.N / kBN;
  g.tiles = g.mt * g.nt * batches;
  if (g.tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_nt_bf16_kernel, dim3(g.tiles), dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace

bool projection_shape_ok(int64_t K1, int64_t d_g, int64_t Kout, int64_t d) {
  return K1 % (2 * kBK) == 0 && Kout % (2 * kBK) == 0 && d_g % kBN == 0 && d % kBN == 0;
}

hipError_t launch_projection(const ProjectArgs& p, hipStream_t st) {
  const int64_t K1 = (int64_t)(p.H / p.G) * p.D, Y = (int64_t)p.G * p.d_g;
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
  hipError_t e = launch_gemm(g1, p.G, st);
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
  return launch_gemm(g2, 1, st);
}

}  // namespace lac
