"""Pins of the oracle's compressor and partial RoPE.

Compressor (深度解析 DeepSeek-V4, CSA Step 1 Compress; HCA section): every m
consecutive KV entries merge into one with learned softmax weights; read as
one softmax over the block's m tokens per channel.  RoPE (QbitAI rewrite,
partial RoPE passage): rotation of the last 64 dims only; the output is
rotated at -i, so R(-p) R(p) = I must hold."""
import json
import math
import os

import numpy as np
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _c(x, z, m, r=0, pos0=0, theta=10000.0, want=False):
    B, T, D = x.shape
    return oracle.compress(np.ascontiguousarray(x, np.float64), np.ascontiguousarray(z, np.float64),
                           oracle.F64, B, T, D, m, r, theta, pos0, want_weights=want)


def test_constant_kv_compresses_to_the_constant():
    rng = np.random.default_rng(0)
    for m in (1, 4, 128):
        x = np.broadcast_to(rng.standard_normal(8), (2, 3 * m, 8)).copy()
        z = rng.standard_normal((2, 3 * m, 8)) * 5
        out = _c(x, z, m)
        assert np.allclose(out, x[:, :3], rtol=0, atol=1e-14)


def test_weights_sum_to_one_per_channel_per_block():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 64, 16))
    z = rng.standard_normal((2, 64, 16)) * 3
    _, alpha = _c(x, z, 4, want=True)
    assert alpha.shape == (2, 16, 4, 16)
    assert np.allclose(alpha.sum(axis=2), 1.0, rtol=0, atol=1e-14)
    assert (alpha > 0).all()


def test_equal_logits_give_the_block_mean():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 32, 8))
    z = np.full((1, 32, 8), 0.7)
    out = _c(x, z, 8)
    assert np.allclose(out[0], x[0].reshape(4, 8, 8).mean(axis=1), atol=1e-14)


def test_block_of_one_is_the_identity():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 10, 8))
    z = rng.standard_normal((2, 10, 8))
    assert np.array_equal(_c(x, z, 1), x)


def test_permuting_tokens_inside_a_block_changes_nothing():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 16, 8))
    z = rng.standard_normal((1, 16, 8))
    perm = np.concatenate([b * 4 + rng.permutation(4) for b in range(4)])
    assert np.allclose(_c(x, z, 4), _c(x[:, perm], z[:, perm], 4), atol=1e-14)


def test_a_dominant_logit_selects_its_token():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 8, 4))
    z = rng.standard_normal((1, 8, 4))
    z[0, 2] += 60.0   # token 2 of block 0
    z[0, 7] += 60.0   # token 3 of block 1
    out = _c(x, z, 4)
    assert np.allclose(out[0, 0], x[0, 2], rtol=1e-20, atol=1e-20 + 1e-24)
    assert np.allclose(out[0, 1], x[0, 7], rtol=0, atol=1e-20)


def test_matches_library_softmax_pooling():
    rng = np.random.default_rng(6)
    B, T, D, m = 2, 48, 12, 4
    x = rng.standard_normal((B, T, D))
    z = rng.standard_normal((B, T, D)) * 2
    xt, zt = torch.from_numpy(x), torch.from_numpy(z)
    ref = (torch.softmax(zt.view(B, T // m, m, D), dim=2) * xt.view(B, T // m, m, D)).sum(2)
    assert np.allclose(_c(x, z, m), ref.numpy(), rtol=0, atol=1e-13)


def test_trailing_partial_block_is_not_emitted_and_page_counts_hold():
    consts = json.load(open(os.path.join(GOLD, "page_constants.json")))
    for c in consts["counts"]:
        T, m = c["tokens"], c["m"]
        x = np.zeros((1, T, 2))
        out = _c(x, x, m)
        if c["exact"]:
            assert out.shape[1] == c["entries"]
        else:
            assert abs(out.shape[1] - c["entries"]) <= c["rel_tol"] * c["entries"]
    out = _c(np.zeros((1, 10, 2)), np.zeros((1, 10, 2)), 4)
    assert out.shape[1] == 2


def test_rope_rotates_only_the_last_r_dims_in_interleaved_pairs():
    D, r, theta = 12, 8, 10000.0
    for i in range(r // 2):
        for pos in (1.0, 7.0, 1048576.0):
            v = np.zeros(D)
            v[D - r + 2 * i] = 1.0
            out = oracle.rope(v, r, theta, pos)
            ang = pos * theta ** (-2.0 * i / r)
            exp = np.zeros(D)
            exp[D - r + 2 * i] = math.cos(ang)
            exp[D - r + 2 * i + 1] = math.sin(ang)
            assert np.allclose(out, exp, atol=1e-12)
    v = np.arange(D, dtype=np.float64) + 1
    assert np.array_equal(oracle.rope(v, r, theta, 123.0)[: D - r], v[: D - r])


def test_rope_inverse_and_norm():
    rng = np.random.default_rng(7)
    D, r = 128, 64
    for pos in (0.0, 3.0, 262144.0, 1048576.0):
        v = rng.standard_normal(D)
        w = oracle.rope(v, r, 10000.0, pos)
        assert abs(np.linalg.norm(w) - np.linalg.norm(v)) < 1e-12
        assert np.allclose(oracle.rope(w, r, 10000.0, -pos), v, atol=1e-12)


def test_compressed_entry_is_rotated_at_its_block_start():
    rng = np.random.default_rng(8)
    B, T, D, m, r = 1, 16, 16, 4, 8
    x = rng.standard_normal((B, T, D))
    z = rng.standard_normal((B, T, D))
    plain = _c(x, z, m, r=0)
    for pos0 in (0, 4096):
        roped = _c(x, z, m, r=r, pos0=pos0)
        for j in range(T // m):
            assert np.allclose(roped[0, j], oracle.rope(plain[0, j], r, 10000.0, pos0 + j * m),
                               atol=1e-13)
