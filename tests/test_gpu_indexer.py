"""GPU parity of indexer_topk against the oracle's Lightning-Indexer scores
and top-k (QbitAI rewrite: indexer + top-k step; 深度解析 DeepSeek-V4, CSA
Step 2 Select), under the near-tie rule, for both selection paths (one
workgroup per row; split rows for few long rows), causal prefill rows, fewer
visible entries than k, no visible entries and exact ties."""
import numpy as np
import pytest
import torch

import long_context_attention_compressor_amd as lac
import oracle
import synth
from parity import check_topk, check_topk_bf16, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(B, Tq, HI, dI, N, m, k, qpos, fmt, seed, w_zero=False, rows=None, kfmt=None):
    kfmt = fmt if kfmt is None else kfmt
    print(f"indexer B={B} Tq={Tq} HI={HI} dI={dI} N={N} m={m} k={k} {fmt} keys {kfmt}", flush=True)
    q = synth.store(synth.normal(seed, "qI", (B, Tq, HI, dI)), fmt)
    K = synth.store(synth.normal(seed, "KI", (B, N, dI)), kfmt)
    w = synth.uniform(seed, "w", (B, Tq, HI))
    if w_zero:
        w.zero_()
    score = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    idx = lac.indexer_topk(q.to(DEV), w.to(DEV), K.to(DEV), m=m, k=k, q_pos0=qpos,
                           topk_score=score)
    torch.cuda.synchronize()
    g_idx = idx.cpu().numpy().reshape(B * Tq, k)
    g_sc = score.cpu().numpy().reshape(B * Tq, k)
    code = synth.DTYPE_CODES[fmt]
    s, nv = oracle.index_scores(host(q), host(w), host(K), code, B, Tq, HI, dI, N, qpos, m, rows,
                                k_dtype=synth.DTYPE_CODES[kfmt])
    o_idx = oracle.topk(s, nv, k)
    sel = np.arange(B * Tq) if rows is None else np.array([b * Tq + i for b, i in rows])
    g_idx, g_sc = g_idx[sel], g_sc[sel]
    same = check_topk(g_idx, o_idx, s, nv, k)
    for rr in range(len(sel)):
        keff = min(k, int(nv[rr]))
        gi = g_idx[rr, :keff]
        assert (np.diff(gi) > 0).all(), "indices must be ascending"
        # returned scores are the kernel's own fp32 scores of those entries
        assert np.allclose(g_sc[rr, :keff], s[rr, gi], rtol=1e-4, atol=1e-3)
        assert np.isneginf(g_sc[rr, keff:]).all()
    return same


def test_f32_tiny_prefill_all_queries():
    # every query t = 0..255 of a 256-token prefill; t < 64 has fewer than k
    # visible entries, t < 4 has none; ReLU makes exact-zero ties common
    _run(1, 256, 4, 32, 64, 4, 16, [0], "f32", 0)


def test_bf16_decode_prefix_path_ragged():
    # n_vis up to 5003: one workgroup per row holding the row in registers
    _run(4, 1, 64, 128, 5003, 4, 512, [4 * 5003 + 1, 4 * 5003, 4 * 3000 + 3, 40000], "bf16", 1)


def test_bf16_decode_split_path():
    same = _run(2, 1, 64, 128, 40000, 4, 2048, [4 * 40000, 4 * 39001 + 2], "bf16", 2)
    assert len(same) >= 1


def test_bf16_decode_split_path_rows_of_different_lengths():
    # one launch filters every row's chunks and the last chunk of each row to
    # finish resolves it: a row keeping all its visible entries, rows with
    # different chunk counts (ragged last chunks) and one seeing nothing
    _run(4, 1, 64, 128, 20000, 4, 4096, [4 * 3000, 4 * 20000, 4 * 9000 + 1, 2], "bf16", 12)


def test_bf16_decode_split_path_all_tied_takes_lowest_indices():
    B, N, k = 1, 20000, 700
    q = synth.store(synth.normal(3, "qI", (B, 1, 64, 128)), "bf16").to(DEV)
    K = synth.store(synth.normal(3, "KI", (B, N, 128)), "bf16").to(DEV)
    w = torch.zeros((B, 1, 64), device=DEV)
    idx = lac.indexer_topk(q, w, K, m=4, k=k, q_pos0=[4 * N])
    torch.cuda.synchronize()
    assert torch.equal(idx[0, 0].cpu(), torch.arange(k, dtype=torch.int32))


def test_bf16_prefix_path_all_tied_takes_lowest_indices():
    _run(2, 1, 32, 64, 3000, 4, 100, [12000, 12000], "bf16", 4, w_zero=True)


@pytest.mark.parametrize("HI,dI", [(32, 64), (32, 128), (64, 64), (128, 128)])
def test_bf16_head_and_dim_variants(HI, dI):
    _run(2, 1, HI, dI, 2100, 4, 256, [8400, 9000], "bf16", 5 + HI + dI)


def test_bf16_chunked_prefill_causal_rows():
    # 40 queries at positions 20000..20039 (n_vis 5000..5009 at m = 4)
    _run(1, 40, 64, 128, 5010, 4, 300, [20000], "bf16", 6)


def test_bf16_prefill_with_rows_that_see_nothing():
    _run(2, 24, 64, 128, 64, 4, 8, [0, 100], "bf16", 7)


def test_k_covering_everything_and_hca_block():
    _run(2, 3, 64, 128, 300, 128, 400, [128 * 300, 128 * 100], "bf16", 8)


def test_determinism():
    B, N = 3, 30000
    q = synth.store(synth.normal(9, "qI", (B, 1, 64, 128)), "bf16").to(DEV)
    K = synth.store(synth.normal(9, "KI", (B, N, 128)), "bf16").to(DEV)
    w = synth.uniform(9, "w", (B, 1, 64)).to(DEV)
    a = lac.indexer_topk(q, w, K, m=4, k=2048, q_pos0=[4 * N] * B)
    b = lac.indexer_topk(q, w, K, m=4, k=2048, q_pos0=[4 * N] * B)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# E4M3 keys (d_I bytes per key, the mixed row format with no rotated dims),
# bf16 queries: the low-precision indexer key cache.
def test_e4m3_keys_decode_split_path():
    same = _run(2, 1, 64, 128, 40000, 4, 2048, [4 * 40000, 4 * 39001 + 2], "bf16", 21, kfmt="mixed")
    assert len(same) >= 1


def test_e4m3_keys_decode_one_workgroup_per_row():
    _run(4, 1, 64, 128, 5003, 4, 512, [4 * 5003 + 1, 4 * 5003, 4 * 3000 + 3, 40000], "bf16", 22,
         kfmt="mixed")


def test_e4m3_keys_chunked_prefill_causal_rows():
    _run(1, 40, 64, 128, 5010, 4, 300, [20000], "bf16", 23, kfmt="mixed")


@pytest.mark.parametrize("HI,dI", [(32, 64), (128, 128)])
def test_e4m3_keys_head_and_dim_variants(HI, dI):
    _run(2, 3, HI, dI, 2100, 4, 256, [8400, 9000], "bf16", 24 + HI + dI, kfmt="mixed")



# Rows longer than the register-resident kernel holds (16384 visible entries)
# and too many of them for the split path (more than 64 rows): up to 2^19
# visible entries the three-pass kernel (histograms and bitmap in LDS, the row
# re-read per pass), beyond that the 8-bit radix select; one workgroup per
# row.  Drawn on the GPU; the oracle scores sampled rows from a host copy of
# their sequences.
def _run_gpu_drawn(B, Tq, HI, dI, N, m, k, qpos, seed, seqs, rows_per_seq, w_zero=False,
                   min_nv=16384):
    print(f"indexer (long rows) B={B} Tq={Tq} N={N} k={k}", flush=True)
    q = synth.store(synth.normal(seed, "qI", (B, Tq, HI, dI), device=DEV), "bf16")
    K = synth.store(synth.normal(seed, "KI", (B, N, dI), device=DEV), "bf16")
    w = synth.uniform(seed, "w", (B, Tq, HI), device=DEV)
    if w_zero:
        w.zero_()
    score = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    idx = lac.indexer_topk(q, w, K, m=m, k=k, q_pos0=qpos, topk_score=score)
    torch.cuda.synchronize()
    sub = lambda t: host(t[seqs].contiguous())
    rows = [(j, i) for j in range(len(seqs)) for i in rows_per_seq]
    s, nv = oracle.index_scores(sub(q), sub(w), sub(K), synth.BF16, len(seqs), Tq, HI, dI, N,
                                [qpos[b] for b in seqs], m, rows)
    assert (nv > min_nv).all() and B * Tq > 64
    o_idx = oracle.topk(s, nv, k)
    # keys sharing the k-th key's top 12 bits (the long kernel keeps up to
    # 4096 of them in LDS, else reads the row a third time)
    for rr in range(len(rows)):
        u = s[rr, :int(nv[rr])].astype(np.float32).view(np.uint32)
        key = np.where(u >> 31 != 0, ~u, u | np.uint32(0x80000000))
        kth = np.sort(key)[::-1][min(k, int(nv[rr])) - 1]
        print(f"  row {rows[rr]}: {int((key >> 20 == kth >> 20).sum())} keys in the threshold's "
              f"12-bit bucket", flush=True)
    g_idx = np.stack([idx[seqs[j], i].cpu().numpy() for j, i in rows])
    g_sc = np.stack([score[seqs[j], i].cpu().numpy() for j, i in rows])
    check_topk(g_idx, o_idx, s, nv, k)
    for rr in range(len(rows)):
        keff = min(k, int(nv[rr]))
        gi = g_idx[rr, :keff]
        assert (np.diff(gi) > 0).all(), "indices must be ascending"
        assert np.allclose(g_sc[rr, :keff], s[rr, gi], rtol=1e-4, atol=1e-3)
    return idx


def test_bf16_long_kernel_prefill_rows_past_67584():
    # 80 queries at 280000..280079: n_vis 70000..70019, 80 rows > 64
    _run_gpu_drawn(1, 80, 32, 64, 70080, 4, 2048, [280000], 41, [0], [0, 1, 39, 40, 78, 79])


def test_bf16_long_kernel_decode_72_sequences():
    qpos = [4 * 70080 - 8 * b for b in range(72)]
    _run_gpu_drawn(72, 1, 32, 64, 70080, 4, 2048, qpos, 42, [0, 35, 71], [0])


def test_bf16_long_kernel_prefill_chunk_at_1m_tokens():
    # a prefill chunk ending at 2^20 tokens: 262144 entries, ragged row lengths
    _run_gpu_drawn(1, 72, 64, 128, 262144, 4, 2048, [(1 << 20) - 72], 44, [0], [0, 37, 71])


def test_long_kernel_threshold_bucket_past_its_lds_list():
    # Scores spread evenly over [1, 1.1): the f32 queries pick the keys' first
    # dim, so every key lands in the threshold's 12-bit bucket (more keys than
    # the kernel keeps in LDS: the row is read a third time) and about 20
    # share each 24-bit prefix (ranked by key, then index).
    B, Tq, HI, dI, N, m, k, qpos = 1, 80, 4, 32, 70080, 4, 2048, [280000]
    print(f"indexer (long rows, narrow band) B={B} Tq={Tq} N={N} k={k}", flush=True)
    q = torch.zeros((B, Tq, HI, dI))
    q[..., 0] = 1.0
    w = torch.full((B, Tq, HI), 0.25)
    K = torch.zeros((B, N, dI))
    K[..., 0] = 1.0 + 0.1 * synth.uniform(47, "KI", (B, N))
    idx = lac.indexer_topk(q.to(DEV), w.to(DEV), K.to(DEV), m=m, k=k, q_pos0=qpos)
    torch.cuda.synchronize()
    rows = [(0, i) for i in (0, 41, 79)]
    s, nv = oracle.index_scores(host(q), host(w), host(K), synth.F32, B, Tq, HI, dI, N, qpos, m,
                                rows)
    key = s.astype(np.float32).view(np.uint32)
    assert ((key[:, :int(nv.min())] >> 23) == (key[0, 0] >> 23)).all()   # one exponent
    g_idx = np.stack([idx[b, i].cpu().numpy() for b, i in rows])
    check_topk(g_idx, oracle.topk(s, nv, k), s, nv, k)


def test_bf16_long_kernel_threshold_bucket_past_its_lds_list():
    # The same narrow band from bf16 queries and keys, scored by the prefill
    # score kernel: s = k0 + k1 / 64 with k0 in [1, 1.1) and k1 in [0, 1), all
    # in one 12-bit bucket, several dozen keys per distinct score.
    B, Tq, HI, dI, N, m, k, qpos = 1, 80, 32, 64, 70080, 4, 2048, [280000]
    print(f"indexer (long rows, narrow band, bf16) B={B} Tq={Tq} N={N} k={k}", flush=True)
    q = torch.zeros((B, Tq, HI, dI))
    q[..., 0] = 1.0
    q[..., 1] = 1.0 / 64
    w = torch.full((B, Tq, HI), 1.0 / HI)
    K = torch.zeros((B, N, dI))
    K[..., 0] = 1.0 + 0.1 * synth.uniform(48, "KI", (B, N))
    K[..., 1] = synth.uniform(49, "KI", (B, N))
    q, K = q.to(torch.bfloat16), K.to(torch.bfloat16)
    score = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    idx = lac.indexer_topk(q.to(DEV), w.to(DEV), K.to(DEV), m=m, k=k, q_pos0=qpos,
                           topk_score=score)
    torch.cuda.synchronize()
    rows = [(0, i) for i in (0, 41, 79)]
    s, nv = oracle.index_scores(host(q), host(w), host(K), synth.DTYPE_CODES["bf16"], B, Tq, HI,
                                dI, N, qpos, m, rows)
    g_idx = np.stack([idx[b, i].cpu().numpy() for b, i in rows])
    check_topk(g_idx, oracle.topk(s, nv, k), s, nv, k)
    g_sc = np.stack([score[b, i].cpu().numpy() for b, i in rows]).astype(np.float64)
    for rr in range(len(rows)):
        assert np.allclose(g_sc[rr], s[rr, g_idx[rr]], rtol=1e-6, atol=0)


def test_bf16_rowwise_kernel_rows_past_2_19():
    # n_vis 530000.. > 2^19: the 8-bit radix select
    _run_gpu_drawn(1, 80, 32, 64, 530080, 4, 2048, [4 * 530000], 45, [0], [0, 79],
                   min_nv=1 << 19)


def test_bf16_rowwise_kernel_all_tied_takes_lowest_indices():
    idx = _run_gpu_drawn(1, 80, 32, 64, 530080, 4, 2048, [4 * 530000], 46, [0], [0, 79],
                         w_zero=True, min_nv=1 << 19)
    assert torch.equal(idx[0, 0].cpu(), torch.arange(2048, dtype=torch.int32))


def test_bf16_long_kernel_all_tied_takes_lowest_indices():
    idx = _run_gpu_drawn(1, 80, 32, 64, 70080, 4, 2048, [280000], 43, [0], [0, 79], w_zero=True)
    assert torch.equal(idx[0].cpu(), torch.arange(2048, dtype=torch.int32).expand(80, 2048))


# E4M3 queries and E4M3 keys (d_I bytes each): products on the FP8 matrix
# cores, exact per product, summed in fp32.
def test_e4m3_queries_decode_split_path():
    same = _run(2, 1, 64, 128, 40000, 4, 2048, [4 * 40000, 4 * 39001 + 2], "mixed", 31,
                kfmt="mixed")
    assert len(same) >= 1


def test_e4m3_queries_decode_prefix_path_ragged():
    _run(4, 1, 64, 128, 5003, 4, 512, [4 * 5003 + 1, 4 * 5003, 4 * 3000 + 3, 40000], "mixed", 32,
         kfmt="mixed")


def test_e4m3_queries_chunked_prefill_causal_rows():
    _run(1, 40, 64, 128, 5010, 4, 300, [20000], "mixed", 33, kfmt="mixed")


def test_e4m3_queries_prefill_with_rows_that_see_nothing():
    _run(2, 24, 64, 128, 64, 4, 8, [0, 100], "mixed", 34, kfmt="mixed")


@pytest.mark.parametrize("HI,dI", [(32, 64), (32, 128), (64, 64), (128, 128)])
def test_e4m3_queries_head_and_dim_variants(HI, dI):
    _run(2, 1, HI, dI, 2100, 4, 256, [8400, 9000], "mixed", 35 + HI + dI, kfmt="mixed")


@pytest.mark.parametrize("HI,dI", [(32, 64), (128, 128)])
def test_e4m3_queries_prefill_head_and_dim_variants(HI, dI):
    _run(1, 17, HI, dI, 700, 4, 64, [2790], "mixed", 36 + HI + dI, kfmt="mixed")


# Scores rounded to bf16 before the selection (LAC_SCORE_BF16): every path.
def _run_bf16(B, Tq, HI, dI, N, m, k, qpos, fmt, seed, kfmt=None, w_zero=False):
    kfmt = fmt if kfmt is None else kfmt
    print(f"indexer bf16 scores B={B} Tq={Tq} HI={HI} dI={dI} N={N} k={k} {fmt}/{kfmt}", flush=True)
    q = synth.store(synth.normal(seed, "qI", (B, Tq, HI, dI)), fmt)
    K = synth.store(synth.normal(seed, "KI", (B, N, dI)), kfmt)
    w = synth.uniform(seed, "w", (B, Tq, HI))
    if w_zero:
        w.zero_()
    score = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    idx = lac.indexer_topk(q.to(DEV), w.to(DEV), K.to(DEV), m=m, k=k, q_pos0=qpos,
                           topk_score=score, score_bf16=True)
    torch.cuda.synchronize()
    s, nv = oracle.index_scores(host(q), host(w), host(K), synth.DTYPE_CODES[fmt], B, Tq, HI, dI,
                                N, qpos, m, k_dtype=synth.DTYPE_CODES[kfmt], score_bf16=True)
    o_idx = oracle.topk(s, nv, k)
    g_idx = idx.cpu().numpy().reshape(B * Tq, k)
    g_sc = score.cpu().numpy().reshape(B * Tq, k).astype(np.float64)
    return check_topk_bf16(g_idx, g_sc, o_idx, s, nv, k)


def test_bf16_scores_decode_split_path():
    _run_bf16(2, 1, 64, 128, 40000, 4, 2048, [4 * 40000, 4 * 39001 + 2], "bf16", 41)


def test_bf16_scores_decode_prefix_path():
    _run_bf16(4, 1, 64, 128, 5003, 4, 512, [4 * 5003 + 1, 4 * 5003, 4 * 3000 + 3, 40000], "bf16", 42)


def test_bf16_scores_chunked_prefill():
    _run_bf16(1, 40, 64, 128, 5010, 4, 300, [20000], "bf16", 43)


def test_bf16_scores_f32_inputs():
    _run_bf16(1, 256, 4, 32, 64, 4, 16, [0], "f32", 44)


def test_bf16_scores_e4m3_queries_split_path():
    _run_bf16(2, 1, 64, 128, 40000, 4, 2048, [4 * 40000, 4 * 39001 + 2], "mixed", 45,
              kfmt="mixed")


def test_bf16_scores_all_tied_take_the_lowest_indices():
    _run_bf16(2, 1, 32, 64, 30000, 4, 100, [4 * 30000, 4 * 30000], "bf16", 46, w_zero=True)


# MXFP4 keys (E2M1 codes with E8M0 block scales) and bf16 queries: the keys
# are widened exactly to bf16 in LDS.  Random code bytes; scales 2^-3..2^3.
# With E4M3 queries (qfmt "mixed": E4M3 codes) the codes and scales go to the
# block-scaled FP4 matrix cores as stored (LAC_Q_E4M3).
def _run_fp4(B, Tq, HI, dI, N, m, k, qpos, seed, qfmt="bf16"):
    print(f"indexer mxfp4 keys, {qfmt} queries B={B} Tq={Tq} HI={HI} dI={dI} N={N} k={k}",
          flush=True)
    q = synth.store(synth.normal(seed, "qI", (B, Tq, HI, dI)), qfmt)
    K = synth.mxfp4_rows(seed, "KI", (B, N), dI)
    w = synth.uniform(seed, "w", (B, Tq, HI))
    score = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    idx = lac.indexer_topk(q.to(DEV), w.to(DEV), K.to(DEV), m=m, k=k, q_pos0=qpos,
                           topk_score=score)
    torch.cuda.synchronize()
    s, nv = oracle.index_scores(host(q), host(w), host(K), synth.DTYPE_CODES[qfmt], B, Tq, HI,
                                dI, N, qpos, m, k_dtype=synth.DTYPE_CODES["mxfp4"])
    o_idx = oracle.topk(s, nv, k)
    g_idx = idx.cpu().numpy().reshape(B * Tq, k)
    g_sc = score.cpu().numpy().reshape(B * Tq, k)
    same = check_topk(g_idx, o_idx, s, nv, k)
    for rr in range(B * Tq):
        keff = min(k, int(nv[rr]))
        gi = g_idx[rr, :keff]
        assert (np.diff(gi) > 0).all()
        assert np.allclose(g_sc[rr, :keff], s[rr, gi], rtol=1e-4, atol=1e-3)
    return same


def test_mxfp4_keys_decode_split_path():
    _run_fp4(2, 1, 64, 128, 40000, 4, 2048, [4 * 40000, 4 * 39001 + 2], 51)


def test_mxfp4_keys_decode_prefix_path_ragged():
    _run_fp4(4, 1, 64, 128, 5003, 4, 512, [4 * 5003 + 1, 4 * 5003, 4 * 3000 + 3, 40000], 52)


def test_mxfp4_keys_prefill_rows():
    _run_fp4(1, 20, 64, 128, 2010, 4, 300, [8000], 53)


@pytest.mark.parametrize("HI,dI", [(32, 64), (128, 128)])
def test_mxfp4_keys_head_and_dim_variants(HI, dI):
    _run_fp4(2, 1, HI, dI, 2100, 4, 256, [8400, 9000], 54 + HI + dI)


# E4M3 queries against MXFP4 keys on the scaled FP4 matrix cores (d_I = 128).
def test_mxfp4_keys_e4m3_queries_decode_split_path():
    _run_fp4(2, 1, 64, 128, 40000, 4, 2048, [4 * 40000, 4 * 39001 + 2], 61, qfmt="mixed")


def test_mxfp4_keys_e4m3_queries_decode_prefix_path_ragged():
    _run_fp4(4, 1, 64, 128, 5003, 4, 512, [4 * 5003 + 1, 4 * 5003, 4 * 3000 + 3, 40000], 62,
             qfmt="mixed")


def test_mxfp4_keys_e4m3_queries_prefill_rows():
    _run_fp4(1, 20, 64, 128, 2010, 4, 300, [8000], 63, qfmt="mixed")


def test_mxfp4_keys_e4m3_queries_rows_that_see_nothing():
    _run_fp4(2, 9, 64, 128, 40, 4, 8, [0, 100], 64, qfmt="mixed")


def test_mxfp4_keys_e4m3_queries_chunked_prefill_causal_rows():
    # 40 queries: the prefill score kernel (8 queries per wave group share
    # each key tile in LDS), ragged key count
    _run_fp4(1, 40, 64, 128, 5010, 4, 300, [20000], 67, qfmt="mixed")


@pytest.mark.parametrize("HI", [32, 128])
def test_mxfp4_keys_e4m3_queries_prefill_head_variants(HI):
    _run_fp4(1, 17, HI, 128, 700, 4, 64, [2790], 68 + HI, qfmt="mixed")


@pytest.mark.parametrize("HI", [32, 128])
def test_mxfp4_keys_e4m3_queries_head_variants(HI):
    _run_fp4(2, 1, HI, 128, 2100, 4, 256, [8400, 9000], 65 + HI, qfmt="mixed")


def test_mxfp4_keys_e4m3_queries_bf16_scores():
    print("indexer mxfp4 keys, e4m3 queries, bf16 scores", flush=True)
    B, Tq, HI, dI, N, m, k, qpos, seed = 2, 1, 64, 128, 40000, 4, 2048, [4 * 40000, 4 * 39001 + 2], 66
    q = synth.store(synth.normal(seed, "qI", (B, Tq, HI, dI)), "mixed")
    K = synth.mxfp4_rows(seed, "KI", (B, N), dI)
    w = synth.uniform(seed, "w", (B, Tq, HI))
    score = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    idx = lac.indexer_topk(q.to(DEV), w.to(DEV), K.to(DEV), m=m, k=k, q_pos0=qpos,
                           topk_score=score, score_bf16=True)
    torch.cuda.synchronize()
    s, nv = oracle.index_scores(host(q), host(w), host(K), synth.DTYPE_CODES["mixed"], B, Tq, HI,
                                dI, N, qpos, m, k_dtype=synth.DTYPE_CODES["mxfp4"], score_bf16=True)
    o_idx = oracle.topk(s, nv, k)
    g_idx = idx.cpu().numpy().reshape(B * Tq, k)
    g_sc = score.cpu().numpy().reshape(B * Tq, k).astype(np.float64)
    check_topk_bf16(g_idx, g_sc, o_idx, s, nv, k)
