/*
 * lac.h -- C ABI of the MI355X (gfx950) hybrid compressed attention library.
 *
 * Five operations, one per step of the method as the pages state it:
 *   csa_compress / hca_compress   pool m (CSA) or m' (HCA) raw KV entries
 *   indexer_topk                  Lightning-Indexer scores + top-k selection
 *   csa_attend                    MQA over the selected compressed entries
 *   hca_attend                    MQA over all visible compressed entries
 * Both attend calls also take the raw sliding window, the optional sink, the
 * partial RoPE and its inverse on the output.  After core attention,
 *   grouped_output_projection     heads in g groups -> d_g each -> d
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory.  Every tensor pointer is a DEVICE pointer owned by the caller.
 *   The library never allocates, frees or copies between host and device,
 *   and never synchronises.  Scratch memory is passed in as `workspace`
 *   (device, 256-byte aligned), sized by the *_workspace_size() queries,
 *   which are pure host arithmetic.  Tensors are dense row-major; base
 *   pointers must be 16-byte aligned.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Work is
 *   enqueued asynchronously; the calls are thread-safe (no global state
 *   except the thread-local error string, the thread-local launch timer, the
 *   thread-local launch group and the fixed device scratch of
 *   indexer_topk_noalloc, whose overlapping calls on one GPU race).
 * Positions.  Host arrays of B int64 (NULL = all zero).  Query i of sequence
 *   b sits at absolute position q_pos0[b] + i; raw row i at raw_pos0[b] + i.
 *   Compressed entry j covers positions [j*m, j*m + m - 1] and is rotated at
 *   position j*m.  Positions must be below 2^31.
 * Storage formats (lac_dtype):
 *   LAC_F32   float32 values
 *   LAC_BF16  bfloat16 values
 *   LAC_KV_E4M3_ROPE_BF16  KV rows of (D - r) FP8 E4M3 bytes ("fn" variant:
 *             bias 7, max 448, no infinities) for the non-rotated dims,
 *             followed by r bfloat16 values for the rotated dims; a row is
 *             (D - r) + 2r bytes (576 B at D = 512, r = 64).  Stores round to
 *             nearest even and saturate to +-448, unscaled.
 *   LAC_E4M3  FP8 E4M3 codes ("fn" variant as above), one byte per value,
 *             unscaled (indexer queries and keys only).
 *   LAC_MXFP4 indexer keys as FP4 E2M1 codes with block scales: a row of d
 *             values is d/2 bytes of codes (value 2i in the low nibble of
 *             byte i, 2i+1 in the high nibble; sign, 2 exponent bits with
 *             bias 1, 1 mantissa bit, exponent 0 subnormal: magnitudes 0,
 *             0.5, 1, 1.5, 2, 3, 4, 6) followed by d/32 E8M0 scale bytes,
 *             byte b scaling its block of 32 values by 2^(b - 127) (255 is
 *             NaN).  d/2 + d/32 bytes per row (68 at d = 128).
 *   The mixed format follows the KV-cache storage of "DeepSeek V4 技术架构深度
 *   解析" (aicoding.csdn.net), section "KV Cache优化细节", and its bit-layout
 *   table in section "三、FP4量化".
 * Errors.  Every argument is validated before anything is enqueued.  On an
 *   invalid argument a call returns a non-zero lac_status, enqueues nothing,
 *   leaves outputs untouched and sets lac_last_error().  A failed kernel
 *   launch returns LAC_ERR_DEVICE.  Device-side faults surface at the
 *   caller's next synchronisation.  No C++ exception crosses the ABI.
 *
 * Page references are by title and section:
 *   [P1] "DeepSeek V4的4个技巧" (hubwiz.com), section "技巧1：混合注意力".
 *   [P2] "深度解析 DeepSeek-V4：百万级长文本的低成本突破" (learnblockchain.cn),
 *        sections "CSA：Compressed Sparse Attention", "HCA：Heavily Compressed
 *        Attention", "Sliding Window Branch", "Attention Sink".
 *   [P3] the QbitAI article as rewritten on futuo-fx-trading.com: partial RoPE
 *        passage, strict-causality passage, the lightning indexer + top-k step,
 *        core attention (MQA) step, grouped output projection step.
 */
#ifndef LAC_H
#define LAC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LAC_OK = 0,
    LAC_ERR_INVALID = 1,     /* a pointer, size, position or combination is invalid */
    LAC_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype/dim combination)   */
    LAC_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small          */
    LAC_ERR_DEVICE = 4       /* the HIP runtime refused a launch                    */
} lac_status;

typedef enum {
    LAC_F32 = 0,
    LAC_BF16 = 1,
    LAC_KV_E4M3_ROPE_BF16 = 2,
    LAC_E4M3 = 3,
    LAC_MXFP4 = 4
} lac_dtype;

/* Flag for the dtype of indexer_topk: round every score to bf16 before the
 * selection (see indexer_topk). */
#define LAC_SCORE_BF16 0x100
/* Flag for the dtype of indexer_topk: the workspace was prepared by
 * indexer_topk_prepare (see there). */
#define LAC_TOPK_PREPARED 0x200
/* Flag for the dtype of indexer_topk, with LAC_MXFP4 keys only: q_idx holds
 * E4M3 codes (see indexer_topk). */
#define LAC_Q_E4M3 0x400

/* Largest batch the position arrays may describe. */
#define LAC_MAX_BATCH 128

/*
 * csa_compress -- [P2] CSA Step 1 "Compress": every m consecutive KV entries
 * are merged into one entry with learned softmax weights.  Reading of the
 * weights: for entry j and channel c, alpha_i = softmax over the block's m
 * tokens of logits[j*m + i, c]; out[j, c] = sum_i alpha_i * raw_kv[j*m + i, c].
 * The entry is then rotated on its last `rope_dims` dims at position
 * pos0[b] + j*m ([P3] partial RoPE; interleaved pairs (D-r+2i, D-r+2i+1),
 * frequency rope_theta^(-2i/r)).  Indexer keys use the same call with
 * rope_dims = 0.  Only complete blocks are emitted: floor(T/m) entries.
 *
 *   raw_kv   [B, kv_batch_stride rows, D] in in_dtype (LAC_F32 | LAC_BF16);
 *            rows 0..T-1 of each batch are read
 *   logits   [B, logit_batch_stride rows, D] in in_dtype
 *   out      [B, out_batch_stride rows, row] in out_dtype (LAC_F32,
 *            LAC_BF16, LAC_KV_E4M3_ROPE_BF16 or, for indexer keys,
 *            LAC_MXFP4); rows 0..T/m-1 of each batch are written.
 *            LAC_MXFP4 (rope_dims = 0, D a multiple of 32): each block of 32
 *            channels of an entry takes the shared exponent
 *            e = floor(log2 max|v|) - 2 (clamped to [-127, 127]; 0 for an
 *            all-zero block), stored as the scale byte e + 127, and each
 *            value the nearest E2M1 code of v / 2^e, ties to even,
 *            saturating at 6, sign bit for v < 0.  Reading: the pages give
 *            the FP4 format and its block scales, not the rounding rule.
 *            An MXFP4 out pointer needs only 4-byte alignment.
 *   m        block size, 1..256 (4 for CSA)
 *   pos0     host [B], position of raw row 0; a multiple of m
 * D must be a multiple of 8, rope_dims a multiple of 8 with rope_dims <= min(D, 128).
 * Streams raw KV and logits once from HBM; fp32 arithmetic.
 */
int32_t csa_compress(const void* raw_kv, const void* logits, int32_t in_dtype, void* out,
                     int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                     int32_t rope_dims, float rope_theta, const int64_t* pos0,
                     int64_t kv_batch_stride, int64_t logit_batch_stride,
                     int64_t out_batch_stride, void* stream);

/*
 * hca_compress -- [P2] HCA: the same pooling with the much larger block m'
 * (128 in the pages), without overlap between blocks.  Arguments and
 * behaviour are those of csa_compress.
 */
int32_t hca_compress(const void* raw_kv, const void* logits, int32_t in_dtype, void* out,
                     int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                     int32_t rope_dims, float rope_theta, const int64_t* pos0,
                     int64_t kv_batch_stride, int64_t logit_batch_stride,
                     int64_t out_batch_stride, void* stream);

/*
 * csa_compress_overlap -- csa_compress with overlapping windows.  The QbitAI
 * rewrite says that HCA's compression has none of the overlap that CSA's
 * has (each m' tokens pooled as one group); it gives no extent.  Reading:
 * entry j, whose block starts at p_j = pos0[b] + j*m, pools the positions
 * [max(0, p_j - overlap), p_j + m): its own m tokens and the `overlap`
 * tokens before them, with one softmax per channel over all of them, and
 * is rotated at p_j.  Its newest token is still p_j + m - 1, so a query at
 * t sees it iff j < floor(t/m), as without overlap.  overlap = 0 is
 * csa_compress.
 *   raw_kv, logits  row 0 of sequence b holds position
 *            pos0[b] - min(overlap, pos0[b]); T rows (floor(T/m) entries)
 *            follow those leading rows, so a batch stride must cover
 *            T + min(overlap, pos0[b]) rows
 *   overlap  0 .. 256 - m tokens
 * Other arguments, formats and errors as csa_compress.
 */
int32_t csa_compress_overlap(const void* raw_kv, const void* logits, int32_t in_dtype, void* out,
                             int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                             int32_t overlap, int32_t rope_dims, float rope_theta,
                             const int64_t* pos0, int64_t kv_batch_stride,
                             int64_t logit_batch_stride, int64_t out_batch_stride, void* stream);

/*
 * csa_compress_rmsnorm, hca_compress_rmsnorm -- csa_compress / hca_compress
 * with the RMSNorm of each compressed entry fused into the epilogue.  [P2]
 * (section "Attention Sink") and [P3] apply RMSNorm to the compressed KV
 * entries before core attention.  Reading: after pooling and before the
 * rotation, over all D dims of the entry,
 *     e <- e / sqrt(mean_c(e[c]^2) + norm_eps) * norm_gain[c]
 * in fp32; the rotation then follows as in csa_compress.
 *   norm_gain  [D] float32 device array, 16-byte aligned (caller-owned)
 *   norm_eps   >= 0 and finite
 * Needs D/8 a power of two of at most 64 (D in {8, ..., 512}); else
 * LAC_ERR_UNSUPPORTED.  Other arguments and errors as csa_compress.
 */
int32_t csa_compress_rmsnorm(const void* raw_kv, const void* logits, int32_t in_dtype, void* out,
                             int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                             int32_t rope_dims, float rope_theta, const int64_t* pos0,
                             int64_t kv_batch_stride, int64_t logit_batch_stride,
                             int64_t out_batch_stride, const float* norm_gain, float norm_eps,
                             void* stream);
int32_t hca_compress_rmsnorm(const void* raw_kv, const void* logits, int32_t in_dtype, void* out,
                             int32_t out_dtype, int32_t B, int32_t T, int32_t D, int32_t m,
                             int32_t rope_dims, float rope_theta, const int64_t* pos0,
                             int64_t kv_batch_stride, int64_t logit_batch_stride,
                             int64_t out_batch_stride, const float* norm_gain, float norm_eps,
                             void* stream);

/*
 * indexer_topk -- [P3] lightning indexer + top-k; [P2] CSA Step 2 "Select";
 * [P1] top 2048.  For query t = q_pos0[b] + i, the visible entries are
 * j < n_vis(t) = min(N, floor(t/m)) ([P3] strict causality: a query never
 * sees its own compressed block).  Score (reading of the indexer):
 *     s[j] = sum_h w[b,i,h] * max(0, q_idx[b,i,h,:] . k_idx[b,j,:])
 * with no scale and no rotation, accumulated in fp32.  The selection keeps
 * the first min(k, n_vis) entries in the order (score descending, index
 * ascending); the chosen indices are written in ascending index order and
 * the remaining slots hold -1.
 *
 *   q_idx       [B, Tq, H_I, d_I] in dtype (LAC_F32 | LAC_BF16 | LAC_E4M3),
 *               or bf16 when dtype is LAC_KV_E4M3_ROPE_BF16
 *   w           [B, Tq, H_I] float32
 *   k_idx       [B, N, d_I] in dtype; with LAC_KV_E4M3_ROPE_BF16, E4M3 keys of
 *               d_I bytes (the mixed row format with no rotated dims, as
 *               csa_compress writes it with rope_dims = 0).  A low-precision
 *               indexer key cache: [P2] runs the indexer's QK path in FP4
 *               (CSA Step 2 Select; section "FP4 Quantization-Aware
 *               Training", whose FP4 block scales dequantize losslessly into
 *               FP8).  Here the keys are stored as unscaled E4M3, widened
 *               exactly to bf16, and scored as above.  With LAC_E4M3 both
 *               q_idx and k_idx are E4M3 codes of d_I bytes per row and the
 *               products run on the FP8 matrix cores (each product exact,
 *               sums in fp32).  With LAC_MXFP4, q_idx is bf16 and k_idx
 *               holds MXFP4 rows (d_I/2 + d_I/32 bytes each): the FP4 QK
 *               path of [P2] (CSA Step 2 Select; "FP4 Quantization-Aware
 *               Training": FP4 block scales fold losslessly into FP8).
 *               Each key value E2M1 x 2^(b - 127) is formed exactly in bf16
 *               (which holds every such FP8 value) and scored as above.
 *               With LAC_MXFP4 | LAC_Q_E4M3 (d_I = 128 only), q_idx holds
 *               E4M3 codes of d_I bytes per head and each product of an
 *               E4M3 query value with a key's E2M1 code and block scale runs
 *               on the block-scaled FP4 matrix cores as stored (no widening:
 *               every product exact, sums in fp32).
 *   topk_idx    [B, Tq, k] int32, output
 *   topk_score  [B, Tq, k] float32, output (score of each chosen index,
 *               -inf in padded slots); may be NULL
 *   workspace   >= indexer_topk_workspace_size(B, Tq, N, k) bytes
 * dtype | LAC_TOPK_PREPARED: the workspace went through indexer_topk_prepare
 * with the same B, Tq, N and k and nothing wrote it since; the call skips
 * zeroing its counters.
 * dtype | LAC_SCORE_BF16: every score is rounded to the nearest bf16 value
 * (ties to even) once it is summed, and the selection runs on the rounded
 * scores with the same order (score descending, index ascending), so equal
 * rounded scores go to the lower index; topk_score returns the rounded
 * scores.  "DeepSeek V4 技术架构深度解析" (section "三、FP4量化", its
 * table of the quantisation scheme) keeps the index scores in BF16.
 * LAC_BF16, LAC_KV_E4M3_ROPE_BF16, LAC_E4M3 and LAC_MXFP4 need H_I in {32, 64, 128} and
 * d_I in {64, 128} (MFMA tiles); LAC_F32 needs H_I * d_I <= 8192.
 * 1 <= k <= 8192.
 */
size_t indexer_topk_workspace_size(int32_t B, int32_t Tq, int32_t N, int32_t k);
int32_t indexer_topk(const void* q_idx, const float* w, const void* k_idx, int32_t dtype,
                     int32_t B, int32_t Tq, int32_t H_I, int32_t d_I, int32_t N,
                     const int64_t* q_pos0, int32_t m, int32_t k, int32_t* topk_idx,
                     float* topk_score, void* workspace, size_t workspace_bytes, void* stream);

/*
 * indexer_topk_prepare -- the part of indexer_topk that reads none of its
 * inputs: zeroing the histograms and counters that its workspace must hold
 * zero on entry (shapes with at most 64 query rows and more than 16384
 * entries; for other shapes there is nothing to zero and the call enqueues
 * nothing).  indexer_topk with dtype | LAC_TOPK_PREPARED on the same
 * workspace and the same B, Tq, N and k then skips that zeroing.  A prepared
 * workspace serves one indexer_topk call: the caller guarantees that nothing
 * else writes the workspace in between.
 * Inside a launch group (lac_group_begin) the zeroing joins the group's
 * compress launch as extra workgroups: it reads nothing the other calls write,
 * so it may share a group with the compress calls whose output the indexer
 * call then reads.  Outside a group it is one small kernel launch.
 *   workspace  >= indexer_topk_workspace_size(B, Tq, N, k) bytes, 256-byte aligned
 * Errors as indexer_topk; LAC_TOPK_PREPARED on indexer_topk_noalloc is
 * LAC_ERR_INVALID.
 */
int32_t indexer_topk_prepare(int32_t B, int32_t Tq, int32_t N, int32_t k, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * indexer_topk_noalloc -- indexer_topk for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * indexer_topk, without the workspace: the call uses a fixed scratch array
 * that the library holds in device memory, 32 MiB on each GPU it runs on,
 * from the first call on that GPU until the process ends.  The call itself
 * allocates and frees nothing.  A call whose indexer_topk_workspace_size(B,
 * Tq, N, k) exceeds 32 MiB returns LAC_ERR_WORKSPACE and enqueues nothing
 * (32 MiB covers, e.g., B = 4 rows at N = 262144 and B = 32 at N = 32768).
 * Every call on one GPU shares that GPU's array and the array keeps the last
 * call's contents (each call clears what it needs cleared): calls that may
 * overlap on one GPU (different streams, or host threads without ordering)
 * race, and must be serialised by the caller.
 */
int32_t indexer_topk_noalloc(const void* q_idx, const float* w, const void* k_idx, int32_t dtype,
                             int32_t B, int32_t Tq, int32_t H_I, int32_t d_I, int32_t N,
                             const int64_t* q_pos0, int32_t m, int32_t k, int32_t* topk_idx,
                             float* topk_score, void* stream);

/*
 * attend_workspace_size -- scratch for csa_attend / hca_attend: the rotated
 * copy of the raw window and split-K partial results.  n_entries is the
 * number of compressed entries one query may attend: k for csa_attend, N for
 * hca_attend; the same values must be passed to the attend call.
 */
size_t attend_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t D, int32_t rope_dims,
                             int32_t kv_dtype, int32_t n_entries, int32_t window);

/*
 * csa_attend -- [P3] core attention: Multi-Query Attention over the selected
 * compressed entries; [P2] plus the sliding window of the most recent raw
 * entries and the attention sink.  For query t and head h:
 *     q~   = R(t) q[b,i,h]                       (rotation of the last r dims)
 *     E    = { ckv[b,j] : j in topk_idx[b,i,:], j >= 0 }
 *            U { R(s) raw_kv[b, s - raw_pos0[b]] : max(0, t-W+1) <= s <= t }
 *     l_e  = scale * (q~ . e)                    (each entry is key and value)
 *     o    = sum_e exp(l_e) e / (exp(sink[h]) + sum_e exp(l_e))
 *     out  = R(-t) o                             ([P3] output rotation at -i)
 * Readings: one softmax over both sets and the sink; no de-duplication; an
 * empty set with no sink gives 0.
 *
 *   q         [B, Tq, H, D] in q_dtype (LAC_F32 | LAC_BF16), not rotated
 *   ckv       [B, N, row] in kv_dtype, rotated at the block start
 *   topk_idx  [B, Tq, k] int32; -1 entries are skipped; values >= N are
 *             skipped as well (they name no entry)
 *   raw_kv    [B, T_raw, row] in kv_dtype, not rotated; must hold every
 *             window position of every query (else LAC_ERR_INVALID); may be
 *             NULL when window == 0
 *   sink      [H] float32 logits, or NULL for none
 *   softmax_scale  0 selects 1/sqrt(D)
 *   out       [B, Tq, H, D] in q_dtype
 *   workspace >= attend_workspace_size(B, Tq, H, D, rope_dims, kv_dtype, k, window)
 * q_dtype LAC_F32 needs kv_dtype LAC_F32, D <= 256 and H*D <= 8192;
 * q_dtype LAC_BF16 needs kv_dtype LAC_BF16 or LAC_KV_E4M3_ROPE_BF16,
 * D in {128, 256, 512} and H dividing 64 or a multiple of 64.
 * rope_dims: a multiple of 8, <= min(D, 128).
 */
int32_t csa_attend(const void* q, int32_t q_dtype, const void* ckv, int32_t kv_dtype, int32_t N,
                   const int32_t* topk_idx, int32_t k, const void* raw_kv, int32_t T_raw,
                   const int64_t* raw_pos0, int32_t window, const float* sink,
                   float softmax_scale, int32_t B, int32_t Tq, int32_t H, int32_t D,
                   int32_t rope_dims, float rope_theta, const int64_t* q_pos0, void* out,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * hca_attend -- [P2] HCA: dense attention over all compressed entries,
 * here all j < n_vis(t) = min(N, floor(t/m)) ([P3] strict causality), plus
 * the raw window and sink exactly as csa_attend.  m is the HCA block m'.
 *   hkv       [B, N, row] in kv_dtype
 *   workspace >= attend_workspace_size(B, Tq, H, D, rope_dims, kv_dtype, N, window)
 * Other arguments as csa_attend.
 */
int32_t hca_attend(const void* q, int32_t q_dtype, const void* hkv, int32_t kv_dtype, int32_t N,
                   int32_t m, const void* raw_kv, int32_t T_raw, const int64_t* raw_pos0,
                   int32_t window, const float* sink, float softmax_scale, int32_t B, int32_t Tq,
                   int32_t H, int32_t D, int32_t rope_dims, float rope_theta,
                   const int64_t* q_pos0, void* out, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * csa_attend_rmsnorm, hca_attend_rmsnorm -- csa_attend / hca_attend with the
 * RMSNorm of each query head fused into the prologue ([P2] section
 * "Attention Sink", [P3]: RMSNorm of the queries before core attention).
 * Reading: before the rotation at t, over all D dims of q[b,i,h],
 *     q <- q / sqrt(mean_c(q[c]^2) + norm_eps) * q_norm_gain[c]
 * in fp32 (then rounded to bf16 once, with the rotation, on the bf16 path).
 * The compressed entries are expected RMSNorm'd already (the *_compress_rmsnorm
 * calls); raw window rows are used as given.
 *   q_norm_gain  [D] float32 device array, 16-byte aligned (caller-owned)
 *   norm_eps     >= 0 and finite
 * Other arguments, limits and errors as csa_attend / hca_attend.
 */
int32_t csa_attend_rmsnorm(const void* q, int32_t q_dtype, const void* ckv, int32_t kv_dtype,
                           int32_t N, const int32_t* topk_idx, int32_t k, const void* raw_kv,
                           int32_t T_raw, const int64_t* raw_pos0, int32_t window,
                           const float* sink, float softmax_scale, int32_t B, int32_t Tq,
                           int32_t H, int32_t D, int32_t rope_dims, float rope_theta,
                           const int64_t* q_pos0, void* out, void* workspace,
                           size_t workspace_bytes, const float* q_norm_gain, float norm_eps,
                           void* stream);
int32_t hca_attend_rmsnorm(const void* q, int32_t q_dtype, const void* hkv, int32_t kv_dtype,
                           int32_t N, int32_t m, const void* raw_kv, int32_t T_raw,
                           const int64_t* raw_pos0, int32_t window, const float* sink,
                           float softmax_scale, int32_t B, int32_t Tq, int32_t H, int32_t D,
                           int32_t rope_dims, float rope_theta, const int64_t* q_pos0, void* out,
                           void* workspace, size_t workspace_bytes, const float* q_norm_gain,
                           float norm_eps, void* stream);

/*
 * grouped_output_projection -- the projection after core attention, in two
 * dense products ([P3], grouped output projection step: with a head
 * dimension of 512 the n_h heads are split into g groups, each group's output
 * is projected to an intermediate width d_g, and the concatenated results
 * are projected back to the model width d):
 *     y[t, g*d_g + j] = sum_c w1[g, j, c] * attn[t, g*(H/G)*D + c]
 *     out[t, j]       = sum_c w2[j, c]    * y[t, c]
 *   Group g holds heads g*H/G .. (g+1)*H/G - 1, concatenated in head order.
 *   attn  [T, H, D] bfloat16 (the attend output with T = B * Tq)
 *   w1    [G, d_g, (H/G)*D] bfloat16
 *   w2    [d, G*d_g] bfloat16
 *   out   [T, d] bfloat16 (fp32 accumulation, rounded to nearest even)
 *   workspace >= grouped_projection_workspace_size(T, H, D, G, d_g, d)
 *         bytes: holds y [T, G*d_g] in bfloat16 between the products
 *         (rounded to nearest even, as a caller storing y in bfloat16
 *         would), and where the products' contraction is split (T <= 64,
 *         or too few output tiles to cover the chip) the fp32 partial sums
 *         of the slices, which are added in a fixed order.
 *   Supported: (H/G)*D and G*d_g multiples of 256, d_g and d multiples of 256,
 *   H*D, G*d_g and d at most 2^22; others return LAC_ERR_UNSUPPORTED.  T = 0
 *   is a no-op.  G must divide H (else LAC_ERR_INVALID).
 */
size_t grouped_projection_workspace_size(int32_t T, int32_t H, int32_t D, int32_t G, int32_t d_g,
                                         int32_t d);
int32_t grouped_output_projection(const void* attn, const void* w1, const void* w2, int32_t T,
                                  int32_t H, int32_t D, int32_t G, int32_t d_g, int32_t d,
                                  void* out, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Launch groups.  lac_group_begin(stream) opens a group on the calling host
 * thread.  Until lac_group_end(stream), the compress calls (csa_compress,
 * csa_compress_overlap, hca_compress and their _rmsnorm forms) and the
 * attention calls (csa_attend, hca_attend and their _rmsnorm forms) made on
 * this thread validate their arguments exactly as outside a group, return
 * LAC_OK and enqueue nothing: they are recorded, with copies of their scalar
 * and host-array arguments (not of the device memory their pointers name).
 * lac_group_end enqueues every recorded call on `stream`:
 *   - the compress calls as one kernel launch (per input dtype, at most four
 *     calls and 384 batch positions per launch);
 *   - the attention calls as one attention launch followed by one combine
 *     launch (per D and KV dtype, at most four calls sharing one rope_theta
 *     and rope_dims per launch; float32 calls run one by one; prefill shapes
 *     add each call's window-rotation launch first), with the calls' key
 *     splits planned together so that they share one wave of workgroups.
 * Compress results are those of the same calls made outside the group; an
 * attention call's key range may be split differently, so its output may
 * differ from the ungrouped call's in the rounding of the split sums.  For a
 * decode step this replaces up to seven launches by three: each launch has
 * a fixed cost of several microseconds.
 *
 * The caller guarantees that the calls of one group are independent: no call
 * reads device memory that another call of the group writes, and no two
 * calls write the same memory (outputs, or workspaces: overlapping attention
 * workspaces are detected and refused).  Memory named by a recorded call must
 * stay valid until the enqueued work completes, as for any call.
 *
 * indexer_topk_prepare may be recorded too: its zeroing joins the compress
 * launch (see there).
 * Inside a group, every call must pass the group's stream (else
 * LAC_ERR_INVALID, nothing recorded), and indexer_topk, indexer_topk_noalloc
 * and grouped_output_projection return LAC_ERR_INVALID.  lac_group_begin on a
 * thread whose group is open returns LAC_ERR_INVALID; lac_group_end without
 * an open group returns LAC_ERR_INVALID.  lac_group_end always closes the
 * group: on an error (another stream, overlapping workspaces:
 * LAC_ERR_WORKSPACE, a refused launch: LAC_ERR_DEVICE) it enqueues nothing
 * further and drops what remains.  A group with no calls is a no-op.  The
 * launch timer brackets a grouped launch like any other launch of its
 * kernel.  lac_group_cancel closes the open group and drops its recorded
 * calls without enqueuing any (LAC_ERR_INVALID when none is open).
 */
int32_t lac_group_begin(void* stream);
int32_t lac_group_end(void* stream);
int32_t lac_group_cancel(void);

/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next call on this thread. */
const char* lac_last_error(void);

/*
 * Launch timer, for measurement.  Arms a one-shot request on this thread:
 * the next launch of kernel `kernel` (LAC_KERNEL_*) enqueued by this thread
 * records hipEvent_t `start` just before it and `stop` just after it, on the
 * stream of the launch.  Passing NULL events disarms.  LAC_KERNEL_PROJECT
 * brackets all launches of one grouped_output_projection call (from 65
 * tokens up, its two products run the same kernel).
 */
enum {
    LAC_KERNEL_COMPRESS = 0,
    LAC_KERNEL_INDEXER_SCORE = 1,
    LAC_KERNEL_TOPK = 2,
    LAC_KERNEL_ATTEND = 3,
    LAC_KERNEL_COMBINE = 4,
    LAC_KERNEL_PROJECT = 5
};
int32_t lac_time_next_launch(int32_t kernel, void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* LAC_H */
