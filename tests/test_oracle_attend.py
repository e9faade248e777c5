"""Pins of the oracle's core attention (CSA sparse and HCA dense).

Sources: QbitAI rewrite (MQA over the selected compressed blocks; KV entries
act as both key and value, so the output is rotated at -i and keeps only
relative position; strict causality), 深度解析 DeepSeek-V4 (HCA dense over all
compressed entries; Sliding Window Branch of the most recent raw entries;
Attention Sink logits in the denominator let the weights sum below 1).
Readings: one softmax over compressed entries, the window [t-W+1, t] and the
optional sink; scale 1/sqrt(D)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import chain

TH = 10000.0


def _att(q, kv, raw, N, mode, idx=None, k=0, m=4, W=1, sink=None, qpos0=0, raw_pos0=0,
         r=0, rows=None, scale=0.0):
    B, Tq, H, D = q.shape
    T_raw = raw.shape[1] if raw is not None else 0
    return oracle.attend(np.ascontiguousarray(q), oracle.F64, np.ascontiguousarray(kv), oracle.F64,
                         N, mode, idx, k, m,
                         None if raw is None else np.ascontiguousarray(raw), T_raw,
                         raw_pos0, W, sink, scale, B, Tq, H, D, r, TH, qpos0, rows)


def _sdpa_causal(q, x, r):
    """Ordinary causal attention of q [T,H,D] over x [T,D] (K = V = roped x),
    with q roped at t and the output rotated back at -t."""
    T, H, D = q.shape
    qr = np.stack([[oracle.rope(q[t, h], r, TH, t) for h in range(H)] for t in range(T)])
    xr = np.stack([oracle.rope(x[t], r, TH, t) for t in range(T)])
    qt = torch.from_numpy(qr).permute(1, 0, 2)            # [H, T, D]
    kt = torch.from_numpy(xr)[None].expand(H, T, D)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, is_causal=True)
    o = o.permute(1, 0, 2).numpy()
    return np.stack([[oracle.rope(o[t, h], r, TH, -t) for h in range(H)] for t in range(T)])


@pytest.mark.parametrize("r", [0, 8])
def test_hca_with_blocks_of_one_and_window_one_is_causal_attention(r):
    rng = np.random.default_rng(0)
    T, H, D = 12, 3, 16
    x = rng.standard_normal((1, T, D))
    q = rng.standard_normal((1, T, H, D))
    z = rng.standard_normal((1, T, D))
    kv = oracle.compress(x, z, oracle.F64, 1, T, D, 1, r, TH)     # m'=1: rotate at t
    y = _att(q, kv, x, T, 1, m=1, W=1, r=r)
    ref = _sdpa_causal(q[0], x[0], r)
    assert np.allclose(y.reshape(T, H, D), ref, rtol=0, atol=1e-12)


def test_csa_with_k_covering_everything_is_dense_attention():
    rng = np.random.default_rng(1)
    T, H, D, m, W, r = 40, 2, 16, 4, 5, 8
    x = rng.standard_normal((1, T, D))
    z = rng.standard_normal((1, T, D))
    q = rng.standard_normal((1, T, H, D))
    kv = oracle.compress(x, z, oracle.F64, 1, T, D, m, r, TH)
    N = T // m
    K = rng.standard_normal((1, N, 4))
    s, nv = oracle.index_scores(rng.standard_normal((1, T, 2, 4)), np.ones((1, T, 2), np.float32),
                                K, oracle.F64, 1, T, 2, 4, N, 0, m)
    idx = oracle.topk(s, nv, N + 3)
    y_csa = _att(q, kv, x, N, 0, idx=idx, k=N + 3, m=m, W=W, r=r)
    y_hca = _att(q, kv, x, N, 1, m=m, W=W, r=r)
    assert np.allclose(y_csa, y_hca, rtol=0, atol=1e-13)


def test_csa_with_blocks_of_one_and_full_k_is_causal_attention():
    rng = np.random.default_rng(2)
    T, H, D, r = 10, 2, 16, 8
    x = rng.standard_normal((1, T, D))
    q = rng.standard_normal((1, T, H, D))
    kv = oracle.compress(x, np.zeros((1, T, D)), oracle.F64, 1, T, D, 1, r, TH)
    # every earlier entry selected, in a scrambled order, padded with -1
    idx = np.full((T, T + 2), -1, np.int32)
    for t in range(T):
        idx[t, :t] = np.random.default_rng(t).permutation(t)
    y = _att(q, kv, x, T, 0, idx=idx, k=T + 2, m=1, W=1, r=r)
    assert np.allclose(y.reshape(T, H, D), _sdpa_causal(q[0], x[0], r), rtol=0, atol=1e-12)


def test_a_single_entry_comes_back_unrotated():
    rng = np.random.default_rng(3)
    D, H, m, r = 16, 2, 4, 8
    x = rng.standard_normal((1, 4, D))
    q = rng.standard_normal((1, 4, H, D))
    kv = np.zeros((1, 1, D))
    # t < m: no compressed entry is visible; W = 1: only raw token t itself
    y = _att(q, kv, x, 1, 1, m=m, W=1, r=r)
    for t in range(4):
        for h in range(H):
            assert np.allclose(y[t, h], x[0, t], rtol=0, atol=1e-13)


def test_empty_entry_set_gives_zero_and_sink_pins():
    rng = np.random.default_rng(4)
    D, H = 8, 2
    q = rng.standard_normal((1, 1, H, D))
    x = rng.standard_normal((1, 1, D))
    y = _att(q, np.zeros((1, 1, D)), None, 1, 1, m=4, W=0)
    assert (y == 0).all()
    plain = _att(q, np.zeros((1, 1, D)), x, 1, 1, m=4, W=1)
    y = _att(q, np.zeros((1, 1, D)), x, 1, 1, m=4, W=1, sink=np.full(H, -np.inf))
    assert np.array_equal(y, plain)
    sig = np.array([0.3, -1.2])
    y = _att(q, np.zeros((1, 1, D)), x, 1, 1, m=4, W=1, sink=sig)
    for h in range(H):
        logit = (q[0, 0, h] @ x[0, 0]) / math.sqrt(D)
        wgt = math.exp(logit) / (math.exp(logit) + math.exp(sig[h]))
        assert np.allclose(y[0, h], wgt * x[0, 0], rtol=1e-13, atol=1e-15)
    y = _att(q, np.zeros((1, 1, D)), x, 1, 1, m=4, W=1, sink=np.full(H, 1e4))
    assert np.abs(y).max() < 1e-300


def test_outputs_depend_only_on_relative_position():
    rng = np.random.default_rng(5)
    T, H, D, m, W, r, k = 32, 2, 16, 4, 3, 8, 3
    x = rng.standard_normal((1, T, D))
    z = rng.standard_normal((1, T, D))
    q = rng.standard_normal((1, T, H, D))
    N = T // m
    kv = oracle.compress(x, z, oracle.F64, 1, T, D, m, r, TH, 0)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        nv = min(N, t // m)
        sel = np.random.default_rng(10 + t).permutation(nv)[:k]
        idx[t, : len(sel)] = sel
    # queries whose window is not clipped at position 0 (t >= W-1)
    rows = [(0, t) for t in range(W - 1, T)]
    idx = np.ascontiguousarray(idx[W - 1:])          # one index row per listed query
    y0 = _att(q, kv, x, N, 0, idx=idx, k=k, m=m, W=W, r=r, rows=rows)
    for delta in (64, 1 << 20):
        pre = delta // m
        kv_s = np.concatenate([rng.standard_normal((1, pre, D)) * 9,
                               oracle.compress(x, z, oracle.F64, 1, T, D, m, r, TH, delta)], 1)
        idx_s = np.where(idx >= 0, idx + pre, -1).astype(np.int32)
        y1 = _att(q, kv_s, x, N + pre, 0, idx=idx_s, k=k, m=m, W=W, r=r, qpos0=delta,
                  raw_pos0=delta, rows=rows)
        assert np.allclose(y0, y1, rtol=0, atol=1e-9)


def test_no_information_leaks_from_the_future_or_the_own_block():
    rng = np.random.default_rng(6)
    T, D, m, W, r = 64, 32, 4, 2, 8
    inp = dict(B=1, T=T, D=D, m=m, r=r, HI=2, dI=8, H=2, k=5, W=W, theta=TH, q_pos0=0,
               raw_pos0=0, pos0=0)
    base = {n: torch.from_numpy(rng.standard_normal(s).astype(np.float32)) for n, s in
            dict(kv=(1, T, D), z=(1, T, D), kI_raw=(1, T, 8), zI=(1, T, 8), qI=(1, T, 2, 8),
                 q=(1, T, 2, D)).items()}
    base["w"] = torch.from_numpy(rng.uniform(0, 1, (1, T, 2)).astype(np.float32))
    ref = chain.csa_prefill_tiny({**inp, **base})["y"]
    for t in (5, 22, 41):
        own_lo = (t // m) * m
        for name in ("kv", "z", "kI_raw", "zI"):
            pert = {**base, name: base[name].clone()}
            pert[name][0, t + 1:] += 3.0                       # the future
            pert[name][0, own_lo:max(own_lo, t - W + 1)] -= 2.0  # own block, outside the window
            y = chain.csa_prefill_tiny({**inp, **pert})["y"]
            assert np.array_equal(y[t], ref[t]), (t, name)
            assert not np.array_equal(y[T - 1], ref[T - 1])    # a later query does see it


def test_csa_indices_past_the_cache_name_no_entry():
    # An index >= N names no entry: it is skipped like the -1 padding, so a
    # selection padded with such values is still ordinary causal attention.
    rng = np.random.default_rng(7)
    T, H, D, r = 10, 2, 16, 8
    x = rng.standard_normal((1, T, D))
    q = rng.standard_normal((1, T, H, D))
    kv = oracle.compress(x, np.zeros((1, T, D)), oracle.F64, 1, T, D, 1, r, TH)
    idx = np.full((T, T + 3), -1, np.int32)
    for t in range(T):
        idx[t, :t] = np.random.default_rng(t).permutation(t)
        idx[t, t:] = [T, T + 5, 1 << 30][: T + 3 - t] + [-1] * max(0, T - t)
    y = _att(q, kv, x, T, 0, idx=idx, k=T + 3, m=1, W=1, r=r)
    assert np.allclose(y.reshape(T, H, D), _sdpa_causal(q[0], x[0], r), rtol=0, atol=1e-12)
