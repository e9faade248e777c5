"""Pins of the oracle's number formats against PyTorch's own conversions and
against the bit layouts of the FP8/BF16 table (DeepSeek V4 技术架构深度解析,
section 三、FP4量化: E4M3 = 4 exponent + 3 mantissa bits, BF16 = 8 + 7)."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.decode_rows(codes, oracle.BF16, 1 << 16, 0)[0]
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_encode_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-40, 38, 4000),
        # exact ties between neighbouring bf16 values (even and odd mantissas)
        (1.0 + np.arange(128) / 128.0 + 1.0 / 256.0) * 2.0 ** rng.integers(-20, 20, 128),
        np.array([0.0, -0.0, 1e-40, -1e-41, 3.39e38, -3.4e38]),
    ]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(v).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode_rows(v.reshape(1, -1), oracle.BF16, 0).view(np.uint16).ravel()
    assert (got == ref).all()


def test_bf16_encode_rounds_the_exact_value_not_a_float_copy():
    # 1 + 2^-8 is the tie between bf16 neighbours 1 and 1 + 2^-7; a double just
    # above it must round up (a detour through float32 would land on the tie
    # and round to even, i.e. down).
    v = np.array([[1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -8]])
    got = oracle.decode_rows(oracle.encode_rows(v, oracle.BF16, 0), oracle.BF16, 2, 0)[0]
    assert got[0] == 1.0 + 2.0 ** -7
    assert got[1] == 1.0


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.e4m3_decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    # format facts: largest finite 448, smallest subnormal 2^-9, only S.1111.111 is NaN
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    assert np.isnan(got).sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    finite = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = finite[np.isfinite(finite)]
    srt = np.unique(finite)
    mids = (srt[:-1] + srt[1:]) / 2.0          # exact ties
    v = np.concatenate([
        rng.standard_normal(5000) * 4.0 ** rng.integers(-6, 4, 5000),
        mids, -mids, srt, rng.uniform(-447.0, 447.0, 1000),
    ]).astype(np.float32).astype(np.float64)
    v = v[np.abs(v) < 448.0]
    ref = torch.from_numpy(v).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(v)
    assert (got == ref).all()


def test_e4m3_encode_saturates_and_maps_nan():
    got = oracle.e4m3_encode(np.array([448.0, 460.0, 464.0, 500.0, 1e30, -1e30, math.inf,
                                       -math.inf, math.nan]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F]


def test_e4m3_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes)
    back = oracle.e4m3_encode(vals)
    # -0 and +0 are both exact; compare values
    assert np.array_equal(oracle.e4m3_decode(back), vals)


def test_mixed_row_layout():
    D, r = 16, 8
    v = np.linspace(-3, 3, D).reshape(1, D)
    rowb = oracle.encode_rows(v, oracle.MIXED, r)
    assert rowb.shape == (1, (D - r) + 2 * r)
    lo = torch.from_numpy(v[0, : D - r]).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    hi = torch.from_numpy(v[0, D - r:]).float().to(torch.bfloat16).view(torch.int16).numpy()
    assert (rowb[0, : D - r] == lo).all()
    assert (rowb[0, D - r:].view(np.int16) == hi).all()
