"""Pins of the oracle's overlapping CSA compression windows.

Source: the QbitAI rewrite (futuo-fx-trading.com) says of HCA that its
compression has none of the overlap CSA's has and pools each m' tokens as
one group; the extent of CSA's overlap is not given.  Reading: entry j
(block start p_j = pos0 + j*m) pools positions [max(0, p_j - o), p_j + m)
with one softmax per channel, then is rotated at p_j; o = 0 is plain block
compression.  Input row 0 of sequence b sits at pos0[b] - min(o, pos0[b])."""
import numpy as np
import pytest
import torch

import oracle

TH = 10000.0


def _inputs(seed, B, rows, D):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, rows, D)), rng.standard_normal((B, rows, D))


def test_no_overlap_is_plain_block_compression():
    x, z = _inputs(0, 2, 40, 16)
    a = oracle.compress_overlap(x, z, oracle.F64, 2, 40, 16, 4, 0, r=8, pos0=[0, 12])
    b = oracle.compress(x, z, oracle.F64, 2, 40, 16, 4, r=8, pos0=[0, 12])
    assert np.array_equal(a, b)


@pytest.mark.parametrize("m,o,pos0", [(4, 4, 0), (4, 3, 8), (4, 9, 4), (16, 16, 32)])
def test_constant_kv_gives_the_constant(m, o, pos0):
    lead = min(o, pos0)
    T = 5 * m
    x = np.full((1, T + lead, 8), 0.75)
    z = np.random.default_rng(1).standard_normal((1, T + lead, 8)) * 3
    out = oracle.compress_overlap(x, z, oracle.F64, 1, T, 8, m, o, pos0=[pos0])
    assert np.allclose(out, 0.75, rtol=0, atol=1e-15)


@pytest.mark.parametrize("m,o,pos0", [(4, 4, 0), (4, 3, 8), (4, 9, 4), (8, 8, 16)])
def test_weights_sum_to_one_over_the_window_and_vanish_before_position_zero(m, o, pos0):
    lead = min(o, pos0)
    T = 6 * m
    x, z = _inputs(2, 1, T + lead, 8)
    _, al = oracle.compress_overlap(x, z, oracle.F64, 1, T, 8, m, o, pos0=[pos0],
                                    want_weights=True)
    assert np.allclose(al.sum(axis=2), 1.0, rtol=0, atol=1e-14)
    for j in range(T // m):
        pj = pos0 + j * m
        for i in range(m + o):
            pos = pj - o + i
            if pos < 0:
                assert (al[0, j, i] == 0).all()
            else:
                assert (al[0, j, i] > 0).all()


@pytest.mark.parametrize("m,o,pos0", [(4, 4, 0), (4, 5, 12), (4, 12, 4)])
def test_equal_logits_give_the_mean_of_the_clipped_window(m, o, pos0):
    lead = min(o, pos0)
    T = 4 * m
    x, _ = _inputs(3, 1, T + lead, 8)
    z = np.zeros_like(x)
    out = oracle.compress_overlap(x, z, oracle.F64, 1, T, 8, m, o, pos0=[pos0])
    base = pos0 - lead                                  # position of input row 0
    for j in range(T // m):
        pj = pos0 + j * m
        lo = max(0, pj - o)
        want = x[0, lo - base:pj + m - base].mean(axis=0)
        assert np.allclose(out[0, j], want, rtol=0, atol=1e-14)


def test_matches_torch_softmax_pooling_on_explicit_windows():
    m, o, D, T = 4, 6, 12, 28
    pos0 = [0, 4, 40]
    lead_max = max(min(o, p) for p in pos0)
    x, z = _inputs(4, 3, T + lead_max, D)
    out = oracle.compress_overlap(x, z, oracle.F64, 3, T, D, m, o, pos0=pos0)
    for b, p0 in enumerate(pos0):
        base = p0 - min(o, p0)
        for j in range(T // m):
            pj = p0 + j * m
            lo = max(0, pj - o)
            zw = torch.from_numpy(z[b, lo - base:pj + m - base])
            xw = torch.from_numpy(x[b, lo - base:pj + m - base])
            want = (torch.softmax(zw, dim=0) * xw).sum(dim=0).numpy()
            assert np.allclose(out[b, j], want, rtol=0, atol=1e-13)


def test_a_window_of_two_blocks_is_block_compression_of_twice_the_size():
    # o = m: entry j pools [(j-1)m, (j+1)m), which is the single entry of a
    # plain compression with block 2m over those rows (r = 0: no rotation)
    m, D, T = 4, 8, 24
    x, z = _inputs(5, 1, T, D)
    out = oracle.compress_overlap(x, z, oracle.F64, 1, T, D, m, m, pos0=[0])
    for j in range(1, T // m):
        s = (j - 1) * m
        ref = oracle.compress(np.ascontiguousarray(x[:, s:s + 2 * m]),
                              np.ascontiguousarray(z[:, s:s + 2 * m]), oracle.F64, 1, 2 * m, D,
                              2 * m)
        assert np.allclose(out[0, j], ref[0, 0], rtol=0, atol=1e-14)


def test_only_the_window_reaches_an_entry():
    # entry j depends on positions [p_j - o, p_j + m) and on nothing else: not
    # on the block's future (strict causality), not on older tokens
    m, o, D, T, pos0 = 4, 4, 8, 32, 8
    lead = min(o, pos0)
    x, z = _inputs(6, 1, T + lead, D)
    base = pos0 - lead
    ref = oracle.compress_overlap(x, z, oracle.F64, 1, T, D, m, o, r=8, pos0=[pos0])
    j = 3
    pj = pos0 + j * m
    for pos, changes in ((pj + m, False), (pj + m + 5, False), (pj - o - 1, False),
                         (pj - o, True), (pj + m - 1, True)):
        x2 = x.copy()
        x2[0, pos - base] += 1.0
        out = oracle.compress_overlap(x2, z, oracle.F64, 1, T, D, m, o, r=8, pos0=[pos0])
        assert (not np.array_equal(out[0, j], ref[0, j])) == changes, pos


def test_the_entry_is_rotated_at_its_block_start():
    m, o, D, T, pos0 = 4, 4, 16, 16, 100
    x, z = _inputs(7, 1, T + o, D)
    plain = oracle.compress_overlap(x, z, oracle.F64, 1, T, D, m, o, r=0, pos0=[pos0])
    rot = oracle.compress_overlap(x, z, oracle.F64, 1, T, D, m, o, r=8, pos0=[pos0])
    for j in range(T // m):
        assert np.allclose(rot[0, j], oracle.rope(plain[0, j], 8, TH, pos0 + j * m), rtol=0,
                           atol=1e-14)
