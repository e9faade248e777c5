"""Pins of the oracle's MXFP4 indexer keys: E2M1 codes with E8M0 block
scales (DeepSeek V4 技术架构深度解析, 三、FP4量化, bit-layout table: FP4 is E2M1,
2 exponent bits and 1 mantissa bit; 深度解析 DeepSeek-V4, section "FP4
Quantization-Aware Training": the indexer's QK path runs in FP4 and FP4 block
scales fold losslessly into FP8 on dequantisation)."""
import numpy as np
import torch

import oracle


def _minifloat(code, e_bits, m_bits):
    """IEEE-style value of a sign / e_bits / m_bits code (bias 2^(e_bits-1) - 1,
    exponent 0 subnormal); infinities and NaNs are not modelled."""
    bias = 2 ** (e_bits - 1) - 1
    s = (code >> (e_bits + m_bits)) & 1
    e = (code >> m_bits) & (2 ** e_bits - 1)
    m = code & (2 ** m_bits - 1)
    if e == 0:
        v = (m / 2 ** m_bits) * 2.0 ** (1 - bias)
    else:
        v = (1 + m / 2 ** m_bits) * 2.0 ** (e - bias)
    return -v if s else v


def test_generic_minifloat_formula_matches_library_formats():
    # the formula the E2M1 pin uses reproduces PyTorch's E4M3 (all finite
    # codes) and bf16 (normal and subnormal codes) decoders
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert _minifloat(c, 4, 3) == e4[c]
    bf = torch.arange(0, 65536, 97, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).double().numpy()
    for c, v in zip(range(0, 65536, 97), bf):
        if (c >> 7) & 0xFF == 0xFF:
            continue
        assert _minifloat(c, 8, 7) == v


def test_e2m1_decode_follows_the_two_exponent_one_mantissa_layout():
    got = oracle.e2m1_decode(np.arange(16))
    want = np.array([_minifloat(c, 2, 1) for c in range(16)])
    assert np.array_equal(got, want)
    assert got[:8].tolist() == sorted(got[:8].tolist())           # magnitudes ascending
    assert np.array_equal(got[8:], -got[:8])                       # sign bit


def test_e8m0_decode_matches_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    o = oracle.e8m0_decode(np.arange(256))
    assert np.array_equal(np.isnan(o), np.isnan(t))
    assert np.array_equal(o[~np.isnan(o)], t[~np.isnan(t)])


def test_scaled_e2m1_is_exact_in_e4m3_over_the_lossless_range():
    # the pages' claim: FP4 values with their block scale are FP8 values.
    # Every E2M1 value times 2^k, -8 <= k <= 6, survives PyTorch's E4M3
    # conversion unchanged.
    vals = oracle.e2m1_decode(np.arange(16))
    for k in range(-8, 7):
        x = vals * 2.0 ** k
        back = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
        assert np.array_equal(back, x), k


def _decode_rows(rows, d):
    """Test-side MXFP4 row decode from the codes' definition (header layout)."""
    n = rows.shape[0]
    out = np.empty((n, d))
    for i in range(n):
        for c in range(d):
            code = (rows[i, c // 2] >> (4 * (c & 1))) & 15
            out[i, c] = _minifloat(int(code), 2, 1) * 2.0 ** (int(rows[i, d // 2 + c // 32]) - 127)
    return out


def test_scores_with_mxfp4_keys_use_the_decoded_key_values():
    B, Tq, HI, dI, N, m = 1, 3, 4, 64, 20, 4
    rng = np.random.default_rng(21)
    keys = rng.integers(0, 256, (B, N, dI // 2 + dI // 32), dtype=np.uint8)
    keys[..., dI // 2:] = rng.integers(122, 132, (B, N, dI // 32))
    q = oracle.bf16_encode(rng.standard_normal((B, Tq, HI, dI)))
    w = rng.uniform(0, 1, (B, Tq, HI)).astype(np.float32)
    qpos0 = np.array([4 * N + 3])
    s, nv = oracle.index_scores(q, w, keys, oracle.BF16, B, Tq, HI, dI, N, qpos0, m,
                                k_dtype=oracle.MXFP4)
    kd = _decode_rows(keys[0], dI)[None]
    qd = oracle.bf16_decode(q)
    dots = np.einsum("bthc,bjc->btjh", qd, kd)
    ref = (np.maximum(dots, 0.0) * w.astype(np.float64)[:, :, None, :]).sum(-1)
    for i in range(Tq):
        assert nv[i] == min(N, (qpos0[0] + i) // m)
        assert np.allclose(s[i, : nv[i]], ref[0, i, : nv[i]], rtol=1e-13, atol=1e-12)


def test_scores_with_e4m3_queries_and_mxfp4_keys_use_the_decoded_values():
    # The FP4 QK path with FP8 queries: queries are E4M3 codes from PyTorch's
    # float8 conversion, decoded here by PyTorch; keys are MXFP4 rows decoded
    # by the generic minifloat formula and the E8M0 rule.
    B, Tq, HI, dI, N, m = 2, 3, 8, 64, 25, 4
    qpos0 = np.array([4 * N + 1, 70])
    rng = np.random.default_rng(23)
    keys = rng.integers(0, 256, (B, N, dI // 2 + dI // 32), dtype=np.uint8)
    keys[..., dI // 2:] = rng.integers(121, 134, (B, N, dI // 32))
    qv = torch.from_numpy(rng.standard_normal((B, Tq, HI, dI)) * 2.0).to(torch.float8_e4m3fn)
    q8 = qv.view(torch.uint8).numpy().copy()
    w = rng.uniform(-0.3, 1, (B, Tq, HI)).astype(np.float32)
    s, nv = oracle.index_scores(q8, w, keys, oracle.MIXED, B, Tq, HI, dI, N, qpos0, m,
                                k_dtype=oracle.MXFP4)
    kd = np.stack([_decode_rows(keys[b], dI) for b in range(B)])
    qd = qv.to(torch.float64).numpy()
    dots = np.einsum("bthc,bjc->btjh", qd, kd)
    ref = (np.maximum(dots, 0.0) * w.astype(np.float64)[:, :, None, :]).sum(-1)
    for b in range(B):
        for i in range(Tq):
            rr = b * Tq + i
            assert nv[rr] == min(N, (qpos0[b] + i) // m)
            assert np.allclose(s[rr, : nv[rr]], ref[b, i, : nv[rr]], rtol=1e-13, atol=1e-12)
            assert np.isneginf(s[rr, nv[rr]:]).all()


def test_mxfp4_encode_round_trips_rows_whose_blocks_reach_four():
    # a block whose largest code is 4 or 6 times 2^k has shared exponent k,
    # so encoding its decoded values gives the same bytes back
    rng = np.random.default_rng(22)
    d, n = 128, 40
    codes = rng.integers(0, 16, (n, d))
    codes[codes == 8] = 0                               # -0 decodes to 0.0
    for i in range(n):
        for blk in range(d // 32):
            codes[i, 32 * blk + rng.integers(0, 32)] = rng.choice([6, 7, 14, 15])
    rows = np.zeros((n, d // 2 + d // 32), np.uint8)
    for c in range(d):
        rows[:, c // 2] |= (codes[:, c] << (4 * (c & 1))).astype(np.uint8)
    rows[:, d // 2:] = rng.integers(100, 150, (n, d // 32))
    vals = oracle.decode_rows(rows, oracle.MXFP4, d, 0)
    assert np.array_equal(oracle.encode_rows(vals, oracle.MXFP4, 0), rows)


def test_mxfp4_encode_rounds_to_nearest_even_and_saturates():
    # block maximum 7 -> shared exponent 0; the rest are ties of the E2M1
    # grid (0, 0.5, 1, 1.5, 2, 3, 4, 6), which go to the even code
    v = np.zeros((1, 32))
    v[0, :10] = [7.0, 2.5, 0.25, 0.75, 5.0, -1.25, 1.75, 3.5, -0.1, 6.5]
    dec = oracle.decode_rows(oracle.encode_rows(v, oracle.MXFP4, 0), oracle.MXFP4, 32, 0)
    assert dec[0, :10].tolist() == [6.0, 2.0, 0.0, 1.0, 4.0, -1.0, 2.0, 4.0, -0.0, 6.0]
    assert oracle.encode_rows(v, oracle.MXFP4, 0)[0, 16] == 127
    # an all-zero block keeps scale byte 127; a block of 0.3 gets 2^-4 (0.3 = 4.8 x 2^-4)
    z = np.zeros((1, 64))
    z[0, 32:] = 0.3
    b = oracle.encode_rows(z, oracle.MXFP4, 0)
    assert b[0, 32:].tolist() == [127, 123]
    assert np.allclose(oracle.decode_rows(b, oracle.MXFP4, 64, 0)[0, 32:], 0.25)


def test_mxfp4_encode_error_is_within_half_a_grid_step():
    rng = np.random.default_rng(23)
    v = rng.standard_normal((50, 128)) * np.exp(rng.uniform(-4, 4, (50, 1)))
    b = oracle.encode_rows(v, oracle.MXFP4, 0)
    dec = oracle.decode_rows(b, oracle.MXFP4, 128, 0)
    S = 2.0 ** (b[:, 64:].astype(np.int64) - 127)
    S = np.repeat(S, 32, axis=1)
    x = np.abs(v) / S
    assert (x < 8).all() and (np.abs(v).reshape(50, 4, 32).max(-1) / S[:, ::32] >= 4).all()
    gap = np.where(x < 2, 0.5, np.where(x < 4, 1.0, 2.0))
    bound = np.where(x <= 6, 0.5 * gap * S, np.abs(v) - 6 * S)
    assert (np.abs(dec - v) <= bound * (1 + 1e-12)).all()
