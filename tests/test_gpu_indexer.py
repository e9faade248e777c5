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
from parity import check_topk, host

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


def test_bf16_decode_rowwise_ragged():
    _run(4, 1, 64, 128, 5003, 4, 512, [4 * 5003 + 1, 4 * 5003, 4 * 3000 + 3, 40000], "bf16", 1)


def test_bf16_decode_split_path():
    same = _run(2, 1, 64, 128, 40000, 4, 2048, [4 * 40000, 4 * 39001 + 2], "bf16", 2)
    assert len(same) >= 1


def test_bf16_decode_split_path_all_tied_takes_lowest_indices():
    B, N, k = 1, 20000, 700
    q = synth.store(synth.normal(3, "qI", (B, 1, 64, 128)), "bf16").to(DEV)
    K = synth.store(synth.normal(3, "KI", (B, N, 128)), "bf16").to(DEV)
    w = torch.zeros((B, 1, 64), device=DEV)
    idx = lac.indexer_topk(q, w, K, m=4, k=k, q_pos0=[4 * N])
    torch.cuda.synchronize()
    assert torch.equal(idx[0, 0].cpu(), torch.arange(k, dtype=torch.int32))


def test_bf16_rowwise_all_tied_takes_lowest_indices():
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

