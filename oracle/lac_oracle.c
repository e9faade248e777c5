/*
 * lac_oracle.c -- plain CPU oracle for hybrid compressed attention (CSA + HCA).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU library is checked against.  It shares no code,
 * header, table or constant with the GPU library, and the GPU library never
 * calls it.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load it.
 *
 * Every quantity is computed in double precision straight from the stored
 * input bytes (decoded here by this file's own decoders), in the order the
 * pages describe the method.  Sources, by page title and section:
 *
 *   [P2] "深度解析 DeepSeek-V4：百万级长文本的低成本突破" (learnblockchain.cn),
 *        section "CSA：Compressed Sparse Attention" (Step 1 Compress,
 *        Step 2 Select, and its ASCII diagram), section "HCA：Heavily
 *        Compressed Attention", section "Sliding Window Branch", section
 *        "Attention Sink".
 *   [P3] "DeepSeek-V4" rewrite of the QbitAI article (futuo-fx-trading.com):
 *        the passages on partial RoPE over the last 64 dims with the
 *        position -i rotation on the output, strict causality of the
 *        compressed blocks, the lightning indexer + top-k step, and MQA over
 *        the selected blocks.
 *   [P4] "DeepSeek V4 技术架构深度解析" (aicoding.csdn.net), section
 *        "KV Cache优化细节" (FP8 storage with BF16 RoPE dims) and the FP4/FP8/
 *        BF16 bit-layout table in section "三、FP4量化".
 *   [P1] "DeepSeek V4的4个技巧" (hubwiz.com), section "技巧1：混合注意力"
 *        (top 2048 of the summary blocks).
 *   [P3] also: the grouped output projection step (heads in g groups, each
 *        projected to d_g, the concatenation projected back to d), which
 *        follows core attention.
 *
 * Where the pages leave a step open, the plainest reading is taken; each is
 * named where it is used (and listed in the design notes of the repository).
 *
 * Storage codes (argument `dtype`):
 *   0  float32 rows of D values
 *   1  bfloat16 rows of D values
 *   2  mixed rows: D-r bytes of FP8 E4M3 (the non-rotated dims) followed by
 *      r bfloat16 values (the rotated dims), (D-r) + 2r bytes per row
 *   3  float64 rows of D values (used only by the self-tests)
 *   4  MXFP4 rows (indexer keys): D/2 bytes of E2M1 codes, element 2i in the
 *      low nibble of byte i and 2i+1 in the high nibble, then D/32 E8M0
 *      scale bytes, one per block of 32 consecutive elements
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define LO_F32 0
#define LO_BF16 1
#define LO_MIXED 2
#define LO_F64 3
#define LO_MXFP4 4

/* ------------------------------------------------------------------------ */
/* Number formats ([P4] bit-layout table: BF16 = 8 exponent + 7 mantissa     */
/* bits, E4M3 = 4 exponent + 3 mantissa bits).                               */
/* ------------------------------------------------------------------------ */

double lo_bf16_decode(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 (ties to even), directly from the
 * exact value (no intermediate float rounding).  Overflow goes to infinity. */
uint16_t lo_bf16_encode(double v) {
    if (isnan(v)) return 0x7FC0;
    double a = fabs(v);
    double q;
    if (a == 0.0) {
        q = 0.0;
    } else {
        int e;
        (void)frexp(a, &e);          /* a = f * 2^e, 0.5 <= f < 1 */
        int unbiased = e - 1;        /* a = 1.xxx * 2^unbiased */
        if (unbiased < -126) unbiased = -126; /* subnormal spacing 2^-133 */
        double step = ldexp(1.0, unbiased - 7);
        q = nearbyint(a / step) * step; /* default rounding mode: ties to even */
        if (q > 3.3895313892515355e38) q = INFINITY; /* beyond the largest bf16 */
    }
    float f = (float)(signbit(v) ? -q : q); /* exact: q is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* E4M3 "fn" variant: bias 7, no infinities, only S.1111.111 is NaN,
 * largest finite 448, subnormal step 2^-9. */
double lo_e4m3_decode(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round to nearest E4M3 (ties to even), saturating to +-448; NaN -> 0x7F.
 * Reading: the pages give the format only, not a scale, so the store is
 * unscaled and saturating. */
uint8_t lo_e4m3_encode(double v) {
    if (isnan(v)) return 0x7F;
    uint8_t s = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0) return s | 0x7E;
    if (a < ldexp(1.0, -6)) {                  /* subnormal range */
        double q = nearbyint(a * 512.0);       /* multiples of 2^-9 */
        if (q >= 8.0) return s | 0x08;         /* rounds up to 2^-6 */
        return s | (uint8_t)q;
    }
    int e;
    double f = frexp(a, &e);                   /* a = f * 2^e, 0.5 <= f < 1 */
    int E = e - 1;                             /* a = (2f) * 2^E */
    double q = nearbyint(2.0 * f * 8.0);       /* 8..16 eighths */
    if (q >= 16.0) { q = 8.0; E += 1; }
    return s | (uint8_t)(((E + 7) << 3) | ((int)q - 8));
}

/* E2M1 ([P4] bit-layout table: FP4 = 2 exponent bits + 1 mantissa bit).
 * Reading: exponent bias 1, E = 0 subnormal (m * 0.5), no infinities or NaN,
 * so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4 and 6. */
double lo_e2m1_decode(uint8_t nibble) {
    int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* E8M0 block scale ([P2] "FP4 Quantization-Aware Training": FP4 block
 * scales fold into FP8 on dequantisation).  Reading: a power of two
 * 2^(b - 127), b = 255 NaN. */
double lo_e8m0_decode(uint8_t b) {
    if (b == 255) return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* Nearest E2M1 magnitude code of |x| (ties to the even code, i.e. mantissa
 * bit 0), saturating at 6: the grid is 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static uint8_t e2m1_code(double a) {
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    int c;
    if (a >= 6.0) return 7;
    for (c = 0; c < 7; ++c) {
        double mid = 0.5 * (grid[c] + grid[c + 1]);
        if (a < mid) return (uint8_t)c;
        if (a == mid) return (uint8_t)((c & 1) ? c + 1 : c);   /* even code */
    }
    return 7;
}

/* One MXFP4 row from D values (D a multiple of 32).  Reading of the
 * quantisation (the pages give the format, not the rule): each block of 32
 * takes the shared exponent e = floor(log2(max |v|)) - 2 (2 is E2M1's largest
 * exponent, so the block's largest value lands in [4, 8)), clamped to
 * [-127, 127], stored as the E8M0 byte e + 127 (127 for an all-zero block);
 * every value v becomes the nearest E2M1 code of v / 2^e (ties to even,
 * saturating at 6), with the sign bit set for v < 0. */
static void mxfp4_encode_row(const double* v, int D, uint8_t* p) {
    int blk, c;
    memset(p, 0, (size_t)D / 2);
    for (blk = 0; blk < D / 32; ++blk) {
        double amax = 0.0;
        for (c = 0; c < 32; ++c) amax = fmax(amax, fabs(v[32 * blk + c]));
        int e = 0;
        if (amax > 0.0) {
            int ex;
            frexp(amax, &ex);                  /* amax = f * 2^ex, 0.5 <= f < 1 */
            e = ex - 1 - 2;
            if (e < -127) e = -127;
            if (e > 127) e = 127;
        }
        p[D / 2 + blk] = (uint8_t)(e + 127);
        for (c = 0; c < 32; ++c) {
            double x = ldexp(v[32 * blk + c], -e);
            uint8_t code = (uint8_t)(e2m1_code(fabs(x)) | (x < 0.0 ? 8 : 0));
            int i = 32 * blk + c;
            p[i / 2] |= (uint8_t)(code << (4 * (i & 1)));
        }
    }
}

static int64_t row_bytes(int dtype, int D, int r) {
    switch (dtype) {
    case LO_F32: return 4LL * D;
    case LO_BF16: return 2LL * D;
    case LO_MIXED: return (int64_t)(D - r) + 2LL * r;
    case LO_F64: return 8LL * D;
    case LO_MXFP4: return (int64_t)D / 2 + D / 32;
    }
    return -1;
}

/* Decode one stored row into D doubles. */
static void decode_row(const uint8_t* p, int dtype, int D, int r, double* out) {
    int c;
    switch (dtype) {
    case LO_F32:
        for (c = 0; c < D; ++c) { float f; memcpy(&f, p + 4 * c, 4); out[c] = f; }
        break;
    case LO_BF16:
        for (c = 0; c < D; ++c) { uint16_t h; memcpy(&h, p + 2 * c, 2); out[c] = lo_bf16_decode(h); }
        break;
    case LO_MIXED:
        for (c = 0; c < D - r; ++c) out[c] = lo_e4m3_decode(p[c]);
        for (c = 0; c < r; ++c) {
            uint16_t h;
            memcpy(&h, p + (D - r) + 2 * c, 2);
            out[D - r + c] = lo_bf16_decode(h);
        }
        break;
    case LO_F64:
        memcpy(out, p, 8 * (size_t)D);
        break;
    case LO_MXFP4:
        for (c = 0; c < D; ++c) {
            uint8_t code = (uint8_t)((p[c / 2] >> (4 * (c & 1))) & 15);
            out[c] = lo_e2m1_decode(code) * lo_e8m0_decode(p[D / 2 + c / 32]);
        }
        break;
    }
}

/* Encode one row of D doubles into the storage format. */
static void encode_row(const double* v, int dtype, int D, int r, uint8_t* p) {
    int c;
    switch (dtype) {
    case LO_F32:
        for (c = 0; c < D; ++c) { float f = (float)v[c]; memcpy(p + 4 * c, &f, 4); }
        break;
    case LO_BF16:
        for (c = 0; c < D; ++c) { uint16_t h = lo_bf16_encode(v[c]); memcpy(p + 2 * c, &h, 2); }
        break;
    case LO_MIXED:
        for (c = 0; c < D - r; ++c) p[c] = lo_e4m3_encode(v[c]);
        for (c = 0; c < r; ++c) {
            uint16_t h = lo_bf16_encode(v[D - r + c]);
            memcpy(p + (D - r) + 2 * c, &h, 2);
        }
        break;
    case LO_F64:
        memcpy(p, v, 8 * (size_t)D);
        break;
    case LO_MXFP4:
        mxfp4_encode_row(v, D, p);
        break;
    }
}

int64_t lo_row_bytes(int dtype, int D, int r) { return row_bytes(dtype, D, r); }

void lo_decode_rows(const void* src, int dtype, int64_t n_rows, int D, int r, double* out) {
    int64_t rb = row_bytes(dtype, D, r), i;
    for (i = 0; i < n_rows; ++i) decode_row((const uint8_t*)src + i * rb, dtype, D, r, out + i * D);
}

void lo_encode_rows(const double* v, int dtype, int64_t n_rows, int D, int r, void* dst) {
    int64_t rb = row_bytes(dtype, D, r), i;
    for (i = 0; i < n_rows; ++i) encode_row(v + i * D, dtype, D, r, (uint8_t*)dst + i * rb);
}

/* ------------------------------------------------------------------------ */
/* Partial RoPE ([P3]: rotary position encoding on the last 64 dims of the   */
/* query and the KV entries only; the output is rotated at position -i).     */
/* Reading: pairs (D-r+2i, D-r+2i+1), frequency theta^(-2i/r), all in double. */
/* ------------------------------------------------------------------------ */
void lo_rope(double* v, int D, int r, double theta, double pos) {
    int i;
    for (i = 0; i < r / 2; ++i) {
        double freq = pow(theta, -2.0 * i / (double)r);
        double ang = pos * freq;
        double c = cos(ang), s = sin(ang);
        double a = v[D - r + 2 * i], b = v[D - r + 2 * i + 1];
        v[D - r + 2 * i] = a * c - b * s;
        v[D - r + 2 * i + 1] = a * s + b * c;
    }
}

/* ------------------------------------------------------------------------ */
/* RMSNorm ([P2] section "Attention Sink": V4 applies RMSNorm to the queries */
/* and the compressed KV entries before core attention; [P3] the same for    */
/* CSA and HCA, against exploding logits).  Reading: over all D dims of one  */
/* vector, v <- v / sqrt(mean(v^2) + eps) * gain (gain per dim, fp32), taken */
/* before the rotation.                                                     */
/* ------------------------------------------------------------------------ */
void lo_rmsnorm(double* v, int D, const float* gain, double eps) {
    double ms = 0.0;
    int c;
    for (c = 0; c < D; ++c) ms += v[c] * v[c];
    ms /= (double)D;
    double inv = 1.0 / sqrt(ms + eps);
    for (c = 0; c < D; ++c) v[c] = v[c] * inv * (double)gain[c];
}

/* ------------------------------------------------------------------------ */
/* Compression ([P2] CSA Step 1; HCA uses the same pooling with m' tokens).   */
/* Every m consecutive KV entries merge into one with learned softmax        */
/* weights; reading: one softmax over the m tokens per channel, fed by a      */
/* logit tensor of the same shape as the KV; no entry for a partial block.   */
/* The entry is then rotated at the position of its first token.             */
/* ------------------------------------------------------------------------ */

/* alpha (optional, [B, T/m, m, D]) receives the per-channel weights.       */
/* norm_gain (optional, [D]): the entry is RMSNorm'd (eps norm_eps) before   */
/* its rotation.                                                             */
int lo_compress2(const void* x, const void* z, int in_dtype, int B, int T, int D, int m,
                 int r, double theta, const int64_t* pos0, int64_t x_bstride,
                 int64_t z_bstride, const float* norm_gain, double norm_eps, double* out,
                 double* alpha) {
    if (m < 1 || D < 1 || r < 0 || r > D || (r & 1)) return 1;
    int N = T / m;
    int64_t rb = row_bytes(in_dtype, D, 0);
    int64_t bj;
#pragma omp parallel for schedule(static)
    for (bj = 0; bj < (int64_t)B * N; ++bj) {
        int b = (int)(bj / N), j = (int)(bj % N);
        double* xs = malloc(sizeof(double) * (size_t)m * D);
        double* zs = malloc(sizeof(double) * (size_t)m * D);
        int i, c;
        for (i = 0; i < m; ++i) {
            int64_t row = (int64_t)j * m + i;
            decode_row((const uint8_t*)x + (b * x_bstride + row) * rb, in_dtype, D, 0, xs + i * D);
            decode_row((const uint8_t*)z + (b * z_bstride + row) * rb, in_dtype, D, 0, zs + i * D);
        }
        double* o = out + bj * D;
        for (c = 0; c < D; ++c) {
            double mu = -INFINITY, den = 0.0, acc = 0.0;
            for (i = 0; i < m; ++i) mu = fmax(mu, zs[i * D + c]);
            for (i = 0; i < m; ++i) den += exp(zs[i * D + c] - mu);
            for (i = 0; i < m; ++i) {
                double a = exp(zs[i * D + c] - mu) / den;
                if (alpha) alpha[(bj * m + i) * D + c] = a;
                acc += a * xs[i * D + c];
            }
            o[c] = acc;
        }
        if (norm_gain) lo_rmsnorm(o, D, norm_gain, norm_eps);
        lo_rope(o, D, r, theta, (double)(pos0 ? pos0[b] : 0) + (double)j * m);
        free(xs);
        free(zs);
    }
    return 0;
}

int lo_compress(const void* x, const void* z, int in_dtype, int B, int T, int D, int m,
                int r, double theta, const int64_t* pos0, int64_t x_bstride,
                int64_t z_bstride, double* out, double* alpha) {
    return lo_compress2(x, z, in_dtype, B, T, D, m, r, theta, pos0, x_bstride, z_bstride, NULL,
                        0.0, out, alpha);
}

/* ------------------------------------------------------------------------ */
/* Overlapping compression windows for CSA.  [P3] says, of HCA, that its     */
/* compression has none of the overlap CSA's has and pools each m' tokens as  */
/* one group; the pages give no extent.  Reading: CSA entry j (block start    */
/* p_j = pos0 + j*m) pools the m tokens of its own block and the o tokens     */
/* before it, positions [max(0, p_j - o), p_j + m), with one softmax over      */
/* those tokens per channel; o = 0 is the plain compression above.  The       */
/* newest token of entry j is still p_j + m - 1, so the causality rule of the */
/* indexer and the attention (query t sees entry j iff j < floor(t/m)) is     */
/* unchanged: the overlap reaches only further back.  The entry is rotated at */
/* p_j.  Input rows: row 0 of sequence b is at position pos0[b] - lead_b with */
/* lead_b = min(o, pos0[b]), and T rows follow the lead (entries: T/m).      */
/* alpha (optional, [B, T/m, m + o, D]): slot i holds the weight of position  */
/* p_j - o + i (0 for positions before the sequence start).                   */
/* ------------------------------------------------------------------------ */
int lo_compress_overlap(const void* x, const void* z, int in_dtype, int B, int T, int D, int m,
                        int o, int r, double theta, const int64_t* pos0, int64_t x_bstride,
                        int64_t z_bstride, double* out, double* alpha) {
    if (m < 1 || o < 0 || D < 1 || r < 0 || r > D || (r & 1)) return 1;
    int N = T / m, L = m + o;
    int64_t rb = row_bytes(in_dtype, D, 0);
    int64_t bj;
#pragma omp parallel for schedule(static)
    for (bj = 0; bj < (int64_t)B * N; ++bj) {
        int b = (int)(bj / N), j = (int)(bj % N);
        int64_t p0 = pos0 ? pos0[b] : 0;
        int64_t lead = o < p0 ? o : p0;
        int64_t pj = p0 + (int64_t)j * m;
        double* xs = malloc(sizeof(double) * (size_t)L * D);
        double* zs = malloc(sizeof(double) * (size_t)L * D);
        int* have = malloc(sizeof(int) * (size_t)L);
        int i, c;
        for (i = 0; i < L; ++i) {
            int64_t pos = pj - o + i;
            have[i] = pos >= 0;
            if (!have[i]) continue;
            int64_t row = pos - (p0 - lead);
            decode_row((const uint8_t*)x + (b * x_bstride + row) * rb, in_dtype, D, 0, xs + (int64_t)i * D);
            decode_row((const uint8_t*)z + (b * z_bstride + row) * rb, in_dtype, D, 0, zs + (int64_t)i * D);
        }
        double* ov = out + bj * D;
        for (c = 0; c < D; ++c) {
            double mu = -INFINITY, den = 0.0, acc = 0.0;
            for (i = 0; i < L; ++i)
                if (have[i]) mu = fmax(mu, zs[(int64_t)i * D + c]);
            for (i = 0; i < L; ++i)
                if (have[i]) den += exp(zs[(int64_t)i * D + c] - mu);
            for (i = 0; i < L; ++i) {
                double a = have[i] ? exp(zs[(int64_t)i * D + c] - mu) / den : 0.0;
                if (alpha) alpha[(bj * L + i) * D + c] = a;
                if (have[i]) acc += a * xs[(int64_t)i * D + c];
            }
            ov[c] = acc;
        }
        lo_rope(ov, D, r, theta, (double)pj);
        free(xs);
        free(zs);
        free(have);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Lightning indexer ([P3] "对每名query token，用一名轻量之indexer计算它与每  */
/* 名压缩KV块之相关性分数"; the score s = sum_h w_h * ReLU(q_h . k) is the      */
/* indexer of DeepSeek-V3.2 that the pages say V4 keeps).  Strict causality   */
/* ([P3]): query t sees compressed entry j only when j < floor(t/m).         */
/* ------------------------------------------------------------------------ */

static int64_t n_visible(int64_t t, int N, int m) {
    int64_t n = t >= 0 ? t / m : 0;
    return n < N ? n : N;
}

/* rows: n_rows pairs (b, i).  scores: [n_rows, N]; entries not visible are
 * set to -inf.  nvis (optional): [n_rows].  q is stored in dtype, K in
 * k_dtype (the same formats; LO_MIXED with no rotated dims is E4M3 codes,
 * for queries as well as keys; keys may also be LO_MXFP4). */
int lo_index_scores2(const void* q, int dtype, const float* w, const void* K, int k_dtype,
                     int B, int Tq, int HI, int dI, int N, const int64_t* qpos0, int m,
                     const int32_t* rows, int n_rows, double* scores, int32_t* nvis) {
    (void)B;
    if (dtype != LO_F32 && dtype != LO_BF16 && dtype != LO_F64 && dtype != LO_MIXED) return 2;
    if (k_dtype != LO_F32 && k_dtype != LO_BF16 && k_dtype != LO_F64 && k_dtype != LO_MIXED &&
        k_dtype != LO_MXFP4)
        return 2;
    if (k_dtype == LO_MXFP4 && dI % 32) return 3;
    if (dI < 1 || dI > 1024) return 3;
    int64_t rb = row_bytes(dtype, dI, 0), krb = row_bytes(k_dtype, dI, 0);
    double* qd = malloc(sizeof(double) * (size_t)n_rows * HI * dI);
    int rr, h;
    for (rr = 0; rr < n_rows; ++rr) {
        int b = rows[2 * rr], i = rows[2 * rr + 1];
        for (h = 0; h < HI; ++h)
            decode_row((const uint8_t*)q + (((int64_t)b * Tq + i) * HI + h) * rb, dtype, dI, 0,
                       qd + ((int64_t)rr * HI + h) * dI);
        if (nvis) nvis[rr] = (int32_t)n_visible(qpos0[b] + i, N, m);
    }
    int64_t task;
#pragma omp parallel for schedule(static)
    for (task = 0; task < (int64_t)n_rows * N; ++task) {
        int r2 = (int)(task / N);
        int64_t j = task % N;
        int b = rows[2 * r2], i = rows[2 * r2 + 1];
        if (j >= n_visible(qpos0[b] + i, N, m)) { scores[task] = -INFINITY; continue; }
        double kd[1024];
        int c, hh;
        decode_row((const uint8_t*)K + ((int64_t)b * N + j) * krb, k_dtype, dI, 0, kd);
        double s = 0.0;
        for (hh = 0; hh < HI; ++hh) {
            const double* qh = qd + ((int64_t)r2 * HI + hh) * dI;
            double dot = 0.0;
            for (c = 0; c < dI; ++c) dot += qh[c] * kd[c];
            s += (double)w[((int64_t)b * Tq + i) * HI + hh] * (dot > 0.0 ? dot : 0.0);
        }
        scores[task] = s;
    }
    free(qd);
    return 0;
}

/* Index scores kept in BF16 ("DeepSeek V4 技术架构深度解析", section "三、FP4量化",
 * its table of the quantisation scheme: the index scores go from FP32 to
 * BF16).  Rounds every finite score in place to the nearest bf16 value, ties
 * to even; -inf (an entry not visible) stays. */
int lo_round_scores_bf16(double* s, int64_t n) {
    int64_t i;
    for (i = 0; i < n; ++i)
        if (isfinite(s[i])) s[i] = lo_bf16_decode(lo_bf16_encode(s[i]));
    return 0;
}

int lo_index_scores(const void* q, const float* w, const void* K, int dtype, int B, int Tq,
                    int HI, int dI, int N, const int64_t* qpos0, int m,
                    const int32_t* rows, int n_rows, double* scores, int32_t* nvis) {
    return lo_index_scores2(q, dtype, w, K, dtype, B, Tq, HI, dI, N, qpos0, m, rows, n_rows,
                            scores, nvis);
}

/* ------------------------------------------------------------------------ */
/* Top-k ([P2] Step 2 Select and its diagram; [P1] top 2048).  Order:        */
/* higher score first, lower index first among equal scores (reading); the   */
/* first min(k, n_vis) are kept and the rest of the k slots hold -1.          */
/* ------------------------------------------------------------------------ */
typedef struct { double s; int32_t j; } lo_pair;

static int pair_cmp(const void* a, const void* b) {
    const lo_pair* x = (const lo_pair*)a;
    const lo_pair* y = (const lo_pair*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

int lo_topk(const double* scores, int n_rows, int N, const int32_t* nvis, int k, int32_t* idx) {
    int rr;
#pragma omp parallel for schedule(dynamic, 1)
    for (rr = 0; rr < n_rows; ++rr) {
        int nv = nvis[rr], j;
        lo_pair* p = malloc(sizeof(lo_pair) * (size_t)(nv > 0 ? nv : 1));
        for (j = 0; j < nv; ++j) { p[j].s = scores[(int64_t)rr * N + j]; p[j].j = j; }
        qsort(p, (size_t)nv, sizeof(lo_pair), pair_cmp);
        for (j = 0; j < k; ++j) idx[(int64_t)rr * k + j] = j < nv ? p[j].j : -1;
        free(p);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Core attention ([P3] MQA over the selected compressed blocks; [P2] HCA    */
/* dense over all compressed entries; [P2] sliding window of recent raw      */
/* entries; [P2] attention sink in the denominator; [P3] KV entry = key =    */
/* value, q rotated at t, raw entries at their position s, output at -t).     */
/* Readings: one softmax over compressed entries, window entries and the    */
/* optional sink; the window is raw positions [max(0, t-W+1), t]; entries   */
/* are not de-duplicated between the two sets.                               */
/* mode 0 = CSA (entries from idx, -1 skipped), mode 1 = HCA (entries        */
/* j < min(N, floor(t/m))).                                                  */
/* out: [n_rows, H, D].                                                      */
/* ------------------------------------------------------------------------ */
/* q_norm_gain (optional, [D]): each query head vector is RMSNorm'd (eps    */
/* norm_eps) before its rotation.                                           */
int lo_attend2(const void* q, int q_dtype, const void* kv, int kv_dtype, int N, int mode,
               const int32_t* idx, int k, int m, const void* raw, int T_raw,
               const int64_t* raw_pos0, int W, const double* sink, double scale, int B, int Tq,
               int H, int D, int r, double theta, const int64_t* qpos0, const int32_t* rows,
               int n_rows, const float* q_norm_gain, double norm_eps, double* out) {
    (void)B;
    int64_t qrb = row_bytes(q_dtype, D, 0);
    int64_t krb = row_bytes(kv_dtype, D, r);
    int64_t task;
    int rr0;
    if (scale == 0.0) scale = 1.0 / sqrt((double)D);
    /* The raw buffer must hold every window position; anything else is
     * rejected, never read.  A CSA index outside [0, N) names no entry: it is
     * skipped like the -1 padding of a short selection. */
    for (rr0 = 0; rr0 < n_rows; ++rr0) {
        int b = rows[2 * rr0], i = rows[2 * rr0 + 1];
        int64_t t = qpos0[b] + i;
        int64_t s_lo = t - W + 1 < 0 ? 0 : t - W + 1;
        if (W > 0 && (s_lo < raw_pos0[b] || t >= raw_pos0[b] + T_raw)) return 4;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (task = 0; task < (int64_t)n_rows * H; ++task) {
        int rr = (int)(task / H), h = (int)(task % H);
        int b = rows[2 * rr], i = rows[2 * rr + 1];
        int64_t t = qpos0[b] + i;
        double* qv = malloc(sizeof(double) * (size_t)D);
        double* ev = malloc(sizeof(double) * (size_t)D);
        double* acc = calloc((size_t)D, sizeof(double));
        double* y = out + ((int64_t)rr * H + h) * D;
        int c;
        decode_row((const uint8_t*)q + (((int64_t)b * Tq + i) * H + h) * qrb, q_dtype, D, 0, qv);
        if (q_norm_gain) lo_rmsnorm(qv, D, q_norm_gain, norm_eps);
        lo_rope(qv, D, r, theta, (double)t);

        /* Collect the logits first (to take their maximum), then weights. */
        int64_t n_comp = 0, n_win = 0, e;
        int64_t s_lo = t - W + 1 < 0 ? 0 : t - W + 1;
        if (W > 0 && t >= 0) n_win = t - s_lo + 1;
        int64_t hca_n = mode == 1 ? n_visible(t, N, m) : 0;
        n_comp = mode == 0 ? k : hca_n;
        double* logit = malloc(sizeof(double) * (size_t)(n_comp + n_win + 1));
        int* valid = malloc(sizeof(int) * (size_t)(n_comp + n_win + 1));
        double mx = sink ? sink[h] : -INFINITY;
        for (e = 0; e < n_comp + n_win; ++e) {
            valid[e] = 0;
            if (e < n_comp) {
                int64_t j = mode == 0 ? idx[(int64_t)rr * k + e] : e;
                if (j < 0 || j >= N) continue;
                decode_row((const uint8_t*)kv + ((int64_t)b * N + j) * krb, kv_dtype, D, r, ev);
            } else {
                int64_t s = s_lo + (e - n_comp);
                decode_row((const uint8_t*)raw + ((int64_t)b * T_raw + (s - raw_pos0[b])) * krb,
                           kv_dtype, D, r, ev);
                lo_rope(ev, D, r, theta, (double)s);
            }
            double dot = 0.0;
            for (c = 0; c < D; ++c) dot += qv[c] * ev[c];
            logit[e] = scale * dot;
            valid[e] = 1;
            if (logit[e] > mx) mx = logit[e];
        }
        double den = sink ? exp(sink[h] - mx) : 0.0;
        for (e = 0; e < n_comp + n_win; ++e) {
            if (!valid[e]) continue;
            double p = exp(logit[e] - mx);
            den += p;
            if (e < n_comp) {
                int64_t j = mode == 0 ? idx[(int64_t)rr * k + e] : e;
                decode_row((const uint8_t*)kv + ((int64_t)b * N + j) * krb, kv_dtype, D, r, ev);
            } else {
                int64_t s = s_lo + (e - n_comp);
                decode_row((const uint8_t*)raw + ((int64_t)b * T_raw + (s - raw_pos0[b])) * krb,
                           kv_dtype, D, r, ev);
                lo_rope(ev, D, r, theta, (double)s);
            }
            for (c = 0; c < D; ++c) acc[c] += p * ev[c];
        }
        for (c = 0; c < D; ++c) y[c] = den > 0.0 ? acc[c] / den : 0.0;
        lo_rope(y, D, r, theta, -(double)t);
        free(qv);
        free(ev);
        free(acc);
        free(logit);
        free(valid);
    }
    return 0;
}

int lo_attend(const void* q, int q_dtype, const void* kv, int kv_dtype, int N, int mode,
              const int32_t* idx, int k, int m, const void* raw, int T_raw,
              const int64_t* raw_pos0, int W, const double* sink, double scale, int B, int Tq,
              int H, int D, int r, double theta, const int64_t* qpos0, const int32_t* rows,
              int n_rows, double* out) {
    return lo_attend2(q, q_dtype, kv, kv_dtype, N, mode, idx, k, m, raw, T_raw, raw_pos0, W,
                      sink, scale, B, Tq, H, D, r, theta, qpos0, rows, n_rows, NULL, 0.0, out);
}

/* ------------------------------------------------------------------------ */
/* Grouped output projection ([P3]: with head dimension c = 512, projecting  */
/* every head's output straight back to d would be costly, so the n_h heads  */
/* are split into g groups, each group is projected to an intermediate      */
/* width d_g, and the concatenation is projected back to d).  Reading: group */
/* gi holds heads gi*H/G .. (gi+1)*H/G - 1, concatenated in head order;      */
/*   y[gi] = W1[gi] x[gi]  (W1 [G, d_g, (H/G)*D]),                          */
/*   out   = W2 [y[0]; ...; y[G-1]]  (W2 [d, G*d_g]).                        */
/* attn [T, H, D] and the weights are stored in `dtype` (F32 | BF16);       */
/* out [T, d] in double.  y_dtype is the format y is held in between the    */
/* two products: F64 keeps it exact, BF16 rounds it to nearest even first   */
/* (what a caller that stores y in bfloat16 computes).                       */
/* ------------------------------------------------------------------------ */
int lo_grouped_projection(const void* attn, const void* w1, const void* w2, int dtype, int T,
                          int H, int D, int G, int d_g, int d, int y_dtype, double* out) {
    if (G < 1 || H % G || T < 0 || D < 1 || d_g < 1 || d < 1) return 1;
    if (y_dtype != 3 && y_dtype != 1) return 1;
    int64_t K1 = (int64_t)(H / G) * D, Y = (int64_t)G * d_g;
    int64_t t;
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < T; ++t) {
        double* x = malloc(sizeof(double) * (size_t)H * D);
        double* y = malloc(sizeof(double) * (size_t)Y);
        double* row = malloc(sizeof(double) * (size_t)(K1 > Y ? K1 : Y));
        int64_t gi, j, c;
        decode_row((const uint8_t*)attn + t * row_bytes(dtype, H * D, 0), dtype, H * D, 0, x);
        for (gi = 0; gi < G; ++gi)
            for (j = 0; j < d_g; ++j) {
                decode_row((const uint8_t*)w1 + (gi * d_g + j) * row_bytes(dtype, (int)K1, 0),
                           dtype, (int)K1, 0, row);
                double acc = 0.0;
                for (c = 0; c < K1; ++c) acc += row[c] * x[gi * K1 + c];
                y[gi * d_g + j] = acc;
            }
        if (y_dtype == 1)
            for (c = 0; c < Y; ++c) y[c] = lo_bf16_decode(lo_bf16_encode(y[c]));
        for (j = 0; j < d; ++j) {
            decode_row((const uint8_t*)w2 + j * row_bytes(dtype, (int)Y, 0), dtype, (int)Y, 0, row);
            double acc = 0.0;
            for (c = 0; c < Y; ++c) acc += row[c] * y[c];
            out[t * d + j] = acc;
        }
        free(x);
        free(y);
        free(row);
    }
    return 0;
}

int lo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
