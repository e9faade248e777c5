"""Pins of the oracle's RMSNorm on compressed entries and queries.

深度解析 DeepSeek-V4, section "Attention Sink": V4 applies RMSNorm to the
queries and the compressed KV entries before core attention; the QbitAI
rewrite says the same of CSA and HCA (against exploding attention logits).
Readings: over all D dims of one vector, v / sqrt(mean(v^2) + eps) * gain,
taken before the partial rotation.  The pins below use closed forms (a
constant block pools to its constant, so the output is known), the rotation's
invariance of pair magnitudes (which separates "gain, then rotate" from
"rotate, then gain"), scale invariance, and the reduction to the plain path
when the input already has unit RMS."""
import math

import numpy as np
import pytest

import oracle

TH = 10000.0


def _c(x, z, m, r=0, pos0=0, gain=None, eps=0.0):
    B, T, D = x.shape
    return oracle.compress(np.ascontiguousarray(x, np.float64), np.ascontiguousarray(z, np.float64),
                           oracle.F64, B, T, D, m, r, TH, pos0, norm_gain=gain, norm_eps=eps)


def _att(q, kv, raw, N, mode, m=4, W=1, qpos0=0, raw_pos0=0, r=0, scale=0.0, gain=None,
         eps=0.0, idx=None, k=0):
    B, Tq, H, D = q.shape
    T_raw = raw.shape[1]
    return oracle.attend(np.ascontiguousarray(q), oracle.F64, np.ascontiguousarray(kv), oracle.F64,
                         N, mode, idx, k, m, np.ascontiguousarray(raw), T_raw, raw_pos0, W, None,
                         scale, B, Tq, H, D, r, TH, qpos0, q_norm_gain=gain, norm_eps=eps)


def test_constant_block_at_position_zero_comes_out_as_gain_times_the_unit_vector():
    # A block whose m tokens all equal v pools to v; entry 0 sits at position
    # 0, where the rotation is the identity.  v = (3, 4, 0, ..., 0) has
    # RMS 5 / sqrt(D), so the output is gain * v * sqrt(D) / 5.
    D, m = 8, 4
    v = np.zeros(D)
    v[0], v[1] = 3.0, 4.0
    x = np.broadcast_to(v, (1, 2 * m, D)).copy()
    z = np.random.default_rng(0).standard_normal((1, 2 * m, D)) * 3
    gain = np.linspace(0.5, 2.0, D).astype(np.float32)
    out = _c(x, z, m, r=4, gain=gain)
    want = gain.astype(np.float64) * v * math.sqrt(D) / 5.0
    assert np.allclose(out[0, 0], want, rtol=0, atol=1e-14)


def test_a_constant_unit_block_gives_the_gain_itself():
    D, m = 16, 128
    x = np.full((1, m, D), 2.5)
    z = np.random.default_rng(1).standard_normal((1, m, D))
    gain = np.random.default_rng(2).uniform(0.2, 3.0, D).astype(np.float32)
    out = _c(x, z, m, r=0, gain=gain)
    assert np.allclose(out[0, 0], gain.astype(np.float64), rtol=0, atol=1e-14)


def test_rotated_pairs_keep_the_magnitude_of_the_normalised_gained_pair():
    # Entry 1 of a constant block sits at position m and is rotated; a rotation
    # keeps each pair's length, so |out pair| = |(g_a v_a, g_b v_b)| / rms(v).
    # Gains that differ inside a pair make this fail if the gain were applied
    # after the rotation.  Unrotated dims are gain * v / rms(v).
    D, m, r = 12, 4, 6
    rng = np.random.default_rng(3)
    v = rng.standard_normal(D)
    x = np.broadcast_to(v, (1, 2 * m, D)).copy()
    z = rng.standard_normal((1, 2 * m, D))
    gain = rng.uniform(0.3, 2.0, D).astype(np.float32)
    out = _c(x, z, m, r=r, gain=gain)[0, 1]
    rms = math.sqrt(np.mean(v * v))
    g = gain.astype(np.float64)
    assert np.allclose(out[:D - r], g[:D - r] * v[:D - r] / rms, rtol=0, atol=1e-13)
    for p in range(r // 2):
        a, b = D - r + 2 * p, D - r + 2 * p + 1
        got = math.hypot(out[a], out[b])
        want = math.hypot(g[a] * v[a], g[b] * v[b]) / rms
        assert abs(got - want) < 1e-13
    # ... and the pair is really rotated (position m != 0)
    assert not np.allclose(out[D - r:], g[D - r:] * v[D - r:] / rms, atol=1e-6)


def test_unit_gain_gives_unit_rms_after_rotation():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 64, 32)) * 7
    z = rng.standard_normal((2, 64, 32)) * 2
    out = _c(x, z, 4, r=16, pos0=[40, 1000], gain=np.ones(32, np.float32))
    assert np.allclose(np.mean(out * out, axis=-1), 1.0, rtol=0, atol=1e-12)


def test_scaling_the_values_changes_nothing():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 32, 16))
    z = rng.standard_normal((1, 32, 16))
    gain = rng.uniform(0.5, 1.5, 16).astype(np.float32)
    a = _c(x, z, 4, r=8, gain=gain)
    b = _c(2.0 * x, z, 4, r=8, gain=gain)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_eps_bounds_the_output_of_a_tiny_entry():
    # mean(v^2) = s; with eps the output RMS is sqrt(s / (s + eps)).
    D, m = 8, 4
    v = np.full(D, 1e-3)
    x = np.broadcast_to(v, (1, m, D)).copy()
    z = np.zeros((1, m, D))
    out = _c(x, z, m, gain=np.ones(D, np.float32), eps=1e-6)
    s = 1e-6
    assert abs(math.sqrt(np.mean(out[0, 0] ** 2)) - math.sqrt(s / (s + 1e-6))) < 1e-12
    zero = _c(np.zeros((1, m, D)), z, m, gain=np.ones(D, np.float32), eps=1e-6)
    assert np.array_equal(zero, np.zeros_like(zero))


def _attn_inputs(seed, Tq=3, H=4, D=16, N=8, m=4, W=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Tq, H, D))
    kv = rng.standard_normal((1, N, D))
    qpos0 = N * m
    raw = rng.standard_normal((1, Tq + W - 1, D))
    return q, kv, raw, qpos0, qpos0 - W + 1


@pytest.mark.parametrize("mode", [0, 1])
def test_unit_rms_queries_with_unit_gain_give_the_plain_attention(mode):
    q, kv, raw, qpos0, rpos0 = _attn_inputs(6)
    q = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True))      # each head vector: RMS 1
    D = q.shape[-1]
    idx = np.tile(np.array([0, 3, 5, -1], np.int32), (q.shape[1], 1)) if mode == 0 else None
    k = 4 if mode == 0 else 0
    plain = _att(q, kv, raw, 8, mode, W=3, qpos0=qpos0, raw_pos0=rpos0, r=8, idx=idx, k=k)
    normed = _att(q, kv, raw, 8, mode, W=3, qpos0=qpos0, raw_pos0=rpos0, r=8, idx=idx, k=k,
                  gain=np.ones(D, np.float32))
    assert np.allclose(normed, plain, rtol=0, atol=1e-12)


def test_query_scale_does_not_matter():
    q, kv, raw, qpos0, rpos0 = _attn_inputs(7)
    g = np.random.default_rng(8).uniform(0.5, 1.5, q.shape[-1]).astype(np.float32)
    a = _att(q, kv, raw, 8, 1, W=3, qpos0=qpos0, raw_pos0=rpos0, r=8, gain=g)
    b = _att(3.0 * q, kv, raw, 8, 1, W=3, qpos0=qpos0, raw_pos0=rpos0, r=8, gain=g)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_a_uniform_gain_scales_the_logits():
    # Unit-RMS queries: a gain of 2 everywhere doubles every logit, which is
    # the plain attention with twice the softmax scale.
    q, kv, raw, qpos0, rpos0 = _attn_inputs(9)
    q = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True))
    D = q.shape[-1]
    normed = _att(q, kv, raw, 8, 1, W=3, qpos0=qpos0, raw_pos0=rpos0, r=8,
                  gain=np.full(D, 2.0, np.float32))
    plain = _att(q, kv, raw, 8, 1, W=3, qpos0=qpos0, raw_pos0=rpos0, r=8, scale=2.0 / math.sqrt(D))
    assert np.allclose(normed, plain, rtol=0, atol=1e-12)
