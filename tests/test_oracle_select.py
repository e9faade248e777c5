"""Pins of the oracle's Lightning-Indexer scores and top-k selection.

Indexer (QbitAI rewrite: a light indexer scores each compressed KV block
against each query token): s_j = sum_h w_h * ReLU(q_h . K_j), with strict
causality (a query never sees its own compressed block), so only
j < floor(t/m) is visible.  Top-k (深度解析 DeepSeek-V4, CSA Step 2 Select and
its diagram; DeepSeek V4的4个技巧: top 2048): the k best scores are kept; read
as (score desc, index asc) with -1 padding when fewer than k are visible."""
import json
import os

import numpy as np

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _scores(B=2, Tq=6, HI=4, dI=8, N=20, m=4, qpos0=(0, 40), seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Tq, HI, dI))
    w = rng.uniform(0, 1, (B, Tq, HI)).astype(np.float32)
    K = rng.standard_normal((B, N, dI))
    s, nv = oracle.index_scores(q, w, K, oracle.F64, B, Tq, HI, dI, N, np.array(qpos0), m)
    return q, w, K, s, nv


def test_scores_match_a_library_expression_and_causality():
    B, Tq, HI, dI, N, m = 2, 6, 4, 8, 20, 4
    qpos0 = (0, 40)
    q, w, K, s, nv = _scores(B, Tq, HI, dI, N, m, qpos0)
    dots = np.einsum("bthc,bjc->btjh", q, K)
    ref = (np.maximum(dots, 0.0) * w.astype(np.float64)[:, :, None, :]).sum(-1)
    for b in range(B):
        for i in range(Tq):
            rr = b * Tq + i
            t = qpos0[b] + i
            assert nv[rr] == min(N, t // m)
            assert np.allclose(s[rr, : nv[rr]], ref[b, i, : nv[rr]], rtol=1e-13, atol=1e-12)
            assert np.isneginf(s[rr, nv[rr]:]).all()


def test_scores_with_e4m3_keys_use_the_decoded_key_values():
    # Keys stored as E4M3 codes (the mixed row format with no rotated dims)
    # score exactly as their decoded values would: checked against numpy's
    # expression of the indexer over those values, queries in bf16.
    B, Tq, HI, dI, N, m = 2, 5, 4, 32, 24, 4
    qpos0 = (30, 99)
    rng = np.random.default_rng(7)
    q = oracle.bf16_encode(rng.standard_normal((B, Tq, HI, dI)))
    codes = oracle.e4m3_encode(rng.standard_normal((B, N, dI)) * 2.0)
    w = rng.uniform(0, 1, (B, Tq, HI)).astype(np.float32)
    s, nv = oracle.index_scores(q, w, codes, oracle.BF16, B, Tq, HI, dI, N, np.array(qpos0), m,
                                k_dtype=oracle.MIXED)
    qd = oracle.bf16_decode(q)
    kd = oracle.e4m3_decode(codes)
    dots = np.einsum("bthc,bjc->btjh", qd, kd)
    ref = (np.maximum(dots, 0.0) * w.astype(np.float64)[:, :, None, :]).sum(-1)
    for b in range(B):
        for i in range(Tq):
            rr = b * Tq + i
            assert nv[rr] == min(N, (qpos0[b] + i) // m)
            assert np.allclose(s[rr, : nv[rr]], ref[b, i, : nv[rr]], rtol=1e-13, atol=1e-12)
            assert np.isneginf(s[rr, nv[rr]:]).all()


def test_scores_with_e4m3_queries_and_keys_use_the_decoded_values():
    # Queries and keys both stored as E4M3 codes (the low-precision indexer
    # QK path, 深度解析 DeepSeek-V4, CSA Step 2 Select and section "FP4
    # Quantization-Aware Training"): the codes come from PyTorch's float8
    # conversion and are decoded by PyTorch, so the oracle's own E4M3 decoder
    # is pinned against a library one here.
    import torch
    B, Tq, HI, dI, N, m = 2, 4, 8, 64, 30, 4
    qpos0 = (60, 131)
    rng = np.random.default_rng(11)
    qv = torch.from_numpy(rng.standard_normal((B, Tq, HI, dI)) * 3.0).to(torch.float8_e4m3fn)
    kv = torch.from_numpy(rng.standard_normal((B, N, dI)) * 0.5).to(torch.float8_e4m3fn)
    w = rng.uniform(-0.2, 1, (B, Tq, HI)).astype(np.float32)
    q8 = qv.view(torch.uint8).numpy().copy()
    k8 = kv.view(torch.uint8).numpy().copy()
    s, nv = oracle.index_scores(q8, w, k8, oracle.MIXED, B, Tq, HI, dI, N, np.array(qpos0), m,
                                k_dtype=oracle.MIXED)
    qd = qv.to(torch.float64).numpy()
    kd = kv.to(torch.float64).numpy()
    dots = np.einsum("bthc,bjc->btjh", qd, kd)
    ref = (np.maximum(dots, 0.0) * w.astype(np.float64)[:, :, None, :]).sum(-1)
    for b in range(B):
        for i in range(Tq):
            rr = b * Tq + i
            assert nv[rr] == min(N, (qpos0[b] + i) // m)
            assert np.allclose(s[rr, : nv[rr]], ref[b, i, : nv[rr]], rtol=1e-13, atol=1e-12)
            assert np.isneginf(s[rr, nv[rr]:]).all()


def test_bf16_rounded_scores_match_torch_and_keep_the_lower_index_on_ties():
    # Index scores kept in BF16 (DeepSeek V4 技术架构深度解析, 三、FP4量化): the
    # oracle rounds its double scores to bf16, ties to even.  Checked against
    # PyTorch's bfloat16 conversion (of the float32 value: for random scores
    # the intermediate float rounding never lands on a bf16 midpoint), the
    # half-ulp bound, and the selection's index rule on the ties it creates.
    import torch
    B, Tq, HI, dI, N, m = 1, 3, 4, 16, 300, 4
    rng = np.random.default_rng(12)
    q = rng.standard_normal((B, Tq, HI, dI))
    K = rng.standard_normal((B, N, dI))
    w = rng.uniform(0, 1, (B, Tq, HI)).astype(np.float32)
    qpos0 = np.array([4 * N])
    s, nv = oracle.index_scores(q, w, K, oracle.F64, B, Tq, HI, dI, N, qpos0, m)
    r, nv2 = oracle.index_scores(q, w, K, oracle.F64, B, Tq, HI, dI, N, qpos0, m, score_bf16=True)
    assert (nv == nv2).all()
    fin = np.isfinite(s)
    assert (np.isneginf(r) == ~fin).all()
    ref = torch.from_numpy(s[fin].astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(r[fin], ref)
    half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r[fin]), 1e-300))) - 8)   # 8 bits
    assert (np.abs(r[fin] - s[fin]) <= half_ulp).all()
    # ties: a row whose scores share few bf16 values picks the lowest indices
    t = np.array([[1.0, 1.0039, 1.0, 0.5, 1.0078125, 1.0, 1.0]])    # 1.0039 -> 1.0 in bf16
    tr = oracle.round_scores_bf16(t)
    assert tr[0, 1] == 1.0 and tr[0, 4] == 1.0078125
    idx = oracle.topk(tr, np.array([7], np.int32), 3)
    assert idx[0].tolist() == [4, 0, 1]


def test_worked_example_from_the_pages():
    g = json.load(open(os.path.join(GOLD, "worked_example_select.json")))
    s = np.array([g["scores"]], np.float64)
    idx = oracle.topk(s, np.array([3], np.int32), g["k"])
    assert sorted(idx[0].tolist()) == g["picked"]
    assert not set(g["skipped"]) & set(idx[0].tolist())


def test_topk_is_a_stable_descending_argsort():
    rng = np.random.default_rng(1)
    n, N = 40, 300
    s = rng.standard_normal((n, N))
    s[:, ::3] = np.round(s[:, ::3], 1)        # many exact ties
    s[5] = 0.0                                 # all tied: lowest indices win
    nv = rng.integers(0, N + 1, n).astype(np.int32)
    for k in (1, 16, 64, 400):
        idx = oracle.topk(s, nv, k)
        for rr in range(n):
            ref = np.argsort(-s[rr, : nv[rr]], kind="stable")[:k]
            got = idx[rr]
            assert np.array_equal(got[: len(ref)], ref)
            assert (got[len(ref):] == -1).all()
    assert np.array_equal(oracle.topk(s[5:6], np.array([N], np.int32), 7)[0], np.arange(7))


def test_fewer_visible_than_k_selects_all_visible():
    s = np.array([[3.0, 1.0, 2.0, -np.inf, -np.inf]])
    idx = oracle.topk(s, np.array([3], np.int32), 5)
    assert sorted(idx[0, :3].tolist()) == [0, 1, 2] and (idx[0, 3:] == -1).all()
    idx = oracle.topk(s, np.array([0], np.int32), 2)
    assert (idx == -1).all()


def test_positive_scaling_of_head_weights_keeps_the_selection():
    B, Tq, HI, dI, N, m = 1, 4, 4, 8, 64, 4
    q, w, K, s, nv = _scores(B, Tq, HI, dI, N, m, (300,), seed=3)
    s2, nv2 = oracle.index_scores(q, (w * 3.5).astype(np.float32), K, oracle.F64, B, Tq, HI,
                                  dI, N, np.array([300]), m)
    assert np.array_equal(oracle.topk(s, nv, 10), oracle.topk(s2, nv2, 10))
