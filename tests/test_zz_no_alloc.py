"""The allocation-free indexer entry point (indexer_topk_noalloc) through the
C ABI: on the library's fixed per-device scratch it gives exactly what
indexer_topk gives with a caller workspace, on consecutive calls (a larger
call, then smaller ones on other selection paths, so each call meets the
previous call's leftovers in the scratch), and it refuses calls whose
scratch need exceeds the fixed size before enqueuing anything."""
import pytest
import torch

import long_context_attention_compressor_amd as lac
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(seed, B, Tq, N, HI=64, dI=128, kfmt="bf16"):
    q = synth.store(synth.normal(seed, "qI", (B, Tq, HI, dI)), "bf16").to(DEV)
    K = synth.store(synth.normal(seed, "KI", (B, N, dI)), kfmt).to(DEV)
    w = synth.uniform(seed, "w", (B, Tq, HI)).to(DEV)
    return q, w, K


def _pair(q, w, K, m, k, qpos):
    B, Tq = q.shape[:2]
    sc_ref = torch.empty((B, Tq, k), device=DEV)
    ref_idx = lac.indexer_topk(q, w, K, m=m, k=k, q_pos0=qpos, topk_score=sc_ref)
    idx = torch.full((B, Tq, k), 7, dtype=torch.int32, device=DEV)
    sc = torch.full((B, Tq, k), 3.0, device=DEV)
    lac.indexer_topk_noalloc(q, w, K, m=m, k=k, q_pos0=qpos, topk_idx=idx, topk_score=sc)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx)
    assert torch.equal(sc, sc_ref)


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    # 1) split path, two long decode rows; 2) smaller split path; 3) one
    # workgroup per row (prefill rows) -- each on the scratch the previous left
    print("noalloc: split path B=2 N=40000 k=2048", flush=True)
    q, w, K = _inputs(31, 2, 1, 40000)
    _pair(q, w, K, 4, 2048, [4 * 40000, 4 * 39001 + 2])
    print("noalloc: split path B=1 N=20000 k=700", flush=True)
    q, w, K = _inputs(32, 1, 1, 20000)
    _pair(q, w, K, 4, 700, [4 * 20000])
    print("noalloc: prefill rows B=1 Tq=40 N=5010 k=300", flush=True)
    q, w, K = _inputs(33, 1, 40, 5010)
    _pair(q, w, K, 4, 300, [20000])


def test_noalloc_e4m3_keys_then_smaller_bf16_call():
    print("noalloc: E4M3 keys B=3 N=30000, then bf16 B=2 N=17000", flush=True)
    q, w, K = _inputs(34, 3, 1, 30000, kfmt="mixed")
    _pair(q, w, K, 4, 2048, [4 * 30000] * 3)
    q, w, K = _inputs(35, 2, 1, 17000)
    _pair(q, w, K, 4, 1024, [4 * 17000, 4 * 16000 + 1])


def test_noalloc_refuses_calls_above_the_fixed_scratch():
    B, Tq, N, k = 1, 256, 66560, 2048
    assert lac.indexer_topk_workspace_size(B, Tq, N, k) > 32 << 20
    q = torch.zeros((B, Tq, 64, 128), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((B, Tq, 64), device=DEV)
    K = torch.zeros((B, N, 128), dtype=torch.bfloat16, device=DEV)
    idx = torch.full((B, Tq, k), 5, dtype=torch.int32, device=DEV)
    with pytest.raises(lac.LacError) as e:
        lac.indexer_topk_noalloc(q, w, K, m=4, k=k, q_pos0=[4 * N], topk_idx=idx)
    assert e.value.status == 3 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (idx == 5).all()           # nothing was enqueued
