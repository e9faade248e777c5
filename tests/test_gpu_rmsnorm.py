"""GPU parity of the fused RMSNorm variants against the oracle: the RMSNorm of
each compressed entry (csa_compress_rmsnorm / hca_compress_rmsnorm) and of
each query head (csa_attend_rmsnorm / hca_attend_rmsnorm) before the rotation
(深度解析 DeepSeek-V4, section "Attention Sink": RMSNorm of the queries and
compressed KV entries before core attention; the QbitAI rewrite says the same
of CSA and HCA).  Gains are seeded U(0.5, 1.5); values are scaled away from
unit RMS so that the norm matters."""
import numpy as np
import pytest
import torch

import long_context_attention_compressor_amd as lac
import oracle
import synth
from parity import as_f64, check_attention, check_compressed, host

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMTS = {"f32": torch.float32, "bf16": torch.bfloat16}
EPS = 1e-6


def _gain(seed, D):
    return synth.uniform(seed, "gain", (D,)) + 0.5


def _compress(B, T, D, m, r, in_fmt, out_fmt, pos0, seed, hca=False, x_std=3.0):
    print(f"compress+rmsnorm B={B} T={T} D={D} m={m} r={r} {in_fmt}->{out_fmt}", flush=True)
    x = synth.store(synth.normal(seed, "x", (B, T, D), std=x_std), in_fmt)
    z = synth.store(synth.normal(seed, "z", (B, T, D)), in_fmt)
    gain = _gain(seed, D)
    N = T // m
    if out_fmt == "mixed":
        out = torch.full((B, N, D + r), 0x55, dtype=torch.uint8, device=DEV)
    else:
        out = torch.full((B, N, D), 7.0, dtype=FMTS[out_fmt], device=DEV)
    fn = lac.hca_compress if hca else lac.csa_compress
    fn(x.to(DEV), z.to(DEV), out, m=m, rope_dims=r, pos0=pos0, norm_gain=gain.to(DEV),
       norm_eps=EPS)
    torch.cuda.synchronize()
    ref = oracle.compress(host(x), host(z), synth.DTYPE_CODES[in_fmt], B, T, D, m, r, 10000.0,
                          pos0, norm_gain=host(gain), norm_eps=EPS)
    check_compressed(out, ref, out_fmt, D, r)


def test_csa_bf16_to_mixed_ragged_at_1m_positions():
    _compress(2, 4 * 37 + 3, 512, 4, 64, "bf16", "mixed", [0, (1 << 20) - 4 * 40], 20)


def test_hca_bf16_to_mixed():
    _compress(2, 128 * 3 + 17, 512, 128, 64, "bf16", "mixed", [1 << 20, 4096], 21, hca=True)


def test_csa_f32_tiny():
    _compress(1, 256, 128, 4, 64, "f32", "f32", [0], 22)


def test_hca_bf16_prefill_shape():
    _compress(1, 8192, 128, 128, 64, "bf16", "bf16", [0], 23, hca=True)


@pytest.mark.parametrize("D,m", [(256, 256), (64, 8), (8, 4), (512, 1)])
def test_widths_and_block_sizes(D, m):
    _compress(2, m * 5 + 1, D, m, 0 if D < 64 else 64, "bf16", "bf16", [0, 64 * m], 24 + D + m)


def test_width_without_a_power_of_two_channel_count_is_refused():
    x = torch.ones((1, 8, 40), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((1, 2, 40), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(lac.LacError):
        lac.csa_compress(x, x, out, m=4, rope_dims=8,
                         norm_gain=torch.ones(40, dtype=torch.float32, device=DEV))


def _indices(seed, B, Tq, q_pos0, N, m, k):
    rng = np.random.default_rng(seed)
    idx = np.full((B, Tq, k), -1, np.int32)
    for b in range(B):
        for i in range(Tq):
            nv = min(N, (q_pos0[b] + i) // m)
            n = min(k, nv)
            if n:
                idx[b, i, :n] = np.sort(rng.choice(nv, n, replace=False))
    return idx


def _attend(mode, B, Tq, H, D, r, N, k, m, W, q_pos0, fmt, seed, sink=False):
    print(f"attend+rmsnorm mode={mode} B={B} Tq={Tq} H={H} D={D} N={N} k={k} m={m} W={W} {fmt}",
          flush=True)
    q_fmt = "f32" if fmt == "f32" else "bf16"
    q = synth.store(synth.normal(seed, "q", (B, Tq, H, D), std=4.0), q_fmt)
    kv = synth.store(synth.normal(seed, "kv", (B, N, D)), fmt, r)
    raw_pos0 = [max(0, p - W + 1) for p in q_pos0]
    T_raw = max(q_pos0[b] + Tq - raw_pos0[b] for b in range(B)) if W > 0 else 0
    raw = synth.store(synth.normal(seed, "raw", (B, max(T_raw, 1), D)), fmt, r)
    sk = synth.normal(seed, "sink", (H,)) * 2.0 if sink else None
    gain = _gain(seed, D)
    out = torch.empty((B, Tq, H, D), dtype=FMTS[q_fmt], device=DEV)
    idx = None
    if mode == 0:
        idx = _indices(seed, B, Tq, q_pos0, N, m, k)
        lac.csa_attend(q.to(DEV), kv.to(DEV), torch.from_numpy(idx).to(DEV), raw.to(DEV), W,
                       q_pos0=q_pos0, raw_pos0=raw_pos0, rope_dims=r,
                       sink=None if sk is None else sk.to(DEV), out=out,
                       q_norm_gain=gain.to(DEV), norm_eps=EPS)
    else:
        lac.hca_attend(q.to(DEV), kv.to(DEV), raw.to(DEV), W, m=m, q_pos0=q_pos0,
                       raw_pos0=raw_pos0, rope_dims=r, sink=None if sk is None else sk.to(DEV),
                       out=out, q_norm_gain=gain.to(DEV), norm_eps=EPS)
    torch.cuda.synchronize()
    rows = [(b, i) for b in range(B) for i in range(Tq)]
    o_idx = None if idx is None else np.ascontiguousarray(np.stack([idx[b, i] for b, i in rows]))
    ref = oracle.attend(host(q), synth.DTYPE_CODES[q_fmt], host(kv), synth.DTYPE_CODES[fmt], N,
                        mode, o_idx, k, m, host(raw), raw.shape[1], raw_pos0, W,
                        None if sk is None else host(sk).astype(np.float64), 0.0, B, Tq, H, D, r,
                        10000.0, q_pos0, rows, q_norm_gain=host(gain), norm_eps=EPS)
    g = as_f64(out)
    g = np.stack([g[b, i] for b, i in rows])
    check_attention(g, ref, f"rmsnorm mode {mode} {fmt}")


def test_csa_mixed_decode_split_with_query_norm():
    _attend(0, 2, 1, 64, 512, 64, 2000, 512, 4, 128, [8000, 1 << 20], "mixed", 30)


def test_hca_bf16_prefill_grouped_queries_with_query_norm():
    _attend(1, 1, 300, 16, 128, 64, 8, 0, 128, 128, [700], "bf16", 31)


def test_csa_f32_with_sink_and_query_norm():
    _attend(0, 2, 9, 8, 128, 64, 30, 5, 4, 3, [100, 7], "f32", 32, sink=True)


def test_csa_bf16_two_head_tiles_d256_with_query_norm():
    _attend(0, 2, 2, 128, 256, 64, 700, 40, 4, 64, [2790, 300], "bf16", 33)


def test_hca_mixed_decode_with_query_norm():
    _attend(1, 4, 1, 64, 512, 64, 1000, 0, 128, 128, [128 * 1000 + 5, 128 * 600, 64, 128 * 999],
            "mixed", 34)
