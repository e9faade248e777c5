"""Pins of the oracle's grouped output projection.

QbitAI rewrite (futuo-fx-trading.com), grouped output projection step: with a
head dimension of 512, the n_h heads are split into g groups, each group's
output is projected to an intermediate width d_g, and the concatenation of
the g results is projected back to d.  Readings: group gi holds the H/G
consecutive heads gi*H/G ..; its input is those heads' outputs concatenated in
head order; W1[gi] is [d_g, (H/G)*D] and W2 is [d, G*d_g], both applied as
y = W x.  The pins: selection weights (one 1 per row) whose result is known
element by element, which catches a wrong group offset, a swapped head order
or a transposed weight; small-integer inputs with an exact closed form,
including one whose intermediate is not a bfloat16 value (pins the optional
rounding of y); and the reduction of the grouped product to one dense product
with a block-diagonal first matrix, computed by the library."""
import numpy as np
import pytest

import oracle


def _proj(x, w1, w2, G, d_g, d, y_dtype=oracle.F64):
    T, H, D = x.shape
    return oracle.grouped_projection(np.ascontiguousarray(x, np.float64),
                                     np.ascontiguousarray(w1, np.float64),
                                     np.ascontiguousarray(w2, np.float64), oracle.F64, T, H, D,
                                     G, d_g, d, y_dtype)


def test_selection_weights_pick_the_named_head_elements():
    T, H, D, G, d_g, d = 3, 6, 4, 3, 5, 7
    K1 = (H // G) * D
    rng = np.random.default_rng(0)
    x = rng.standard_normal((T, H, D))
    pick1 = rng.integers(0, K1, (G, d_g))          # y[g, j] = x_g[pick1[g, j]]
    pick2 = rng.integers(0, G * d_g, d)            # out[j] = y[pick2[j]]
    w1 = np.zeros((G, d_g, K1))
    for g in range(G):
        w1[g, np.arange(d_g), pick1[g]] = 1.0
    w2 = np.zeros((d, G * d_g))
    w2[np.arange(d), pick2] = 1.0
    out = _proj(x, w1, w2, G, d_g, d)
    for t in range(T):
        for j in range(d):
            g, jj = divmod(int(pick2[j]), d_g)
            c = int(pick1[g, jj])
            # element c of group g's input is head g*H/G + c // D, dim c % D
            assert out[t, j] == x[t, g * (H // G) + c // D, c % D]


def test_all_ones_gives_the_closed_form():
    T, H, D, G, d_g, d = 2, 4, 8, 2, 3, 5
    K1 = (H // G) * D
    out = _proj(np.ones((T, H, D)), np.ones((G, d_g, K1)), np.ones((d, G * d_g)), G, d_g, d)
    assert np.array_equal(out, np.full((T, d), float(G * d_g * K1)))


def test_bfloat16_intermediate_rounds_to_nearest_even():
    # y = 257 is halfway between the bfloat16 values 256 and 258: it rounds to
    # 256 (even mantissa); y = 259 rounds to 260.
    T, H, D, G, d_g, d = 1, 2, 257, 1, 1, 1
    x = np.zeros((T, H, D))
    x[0, 0, :] = 1.0
    w1 = np.ones((G, d_g, H * D))
    w2 = np.ones((d, G * d_g))
    assert _proj(x, w1, w2, G, d_g, d)[0, 0] == 257.0
    assert _proj(x, w1, w2, G, d_g, d, y_dtype=oracle.BF16)[0, 0] == 256.0
    x[0, 1, :2] = 1.0
    assert _proj(x, w1, w2, G, d_g, d, y_dtype=oracle.BF16)[0, 0] == 260.0


@pytest.mark.parametrize("G", [1, 2, 4])
def test_equals_one_product_with_a_block_diagonal_first_matrix(G):
    T, H, D, d_g, d = 5, 8, 6, 7, 9
    K1 = (H // G) * D
    rng = np.random.default_rng(G)
    x = rng.standard_normal((T, H, D))
    w1 = rng.standard_normal((G, d_g, K1))
    w2 = rng.standard_normal((d, G * d_g))
    big = np.zeros((G * d_g, H * D))
    for g in range(G):
        big[g * d_g:(g + 1) * d_g, g * K1:(g + 1) * K1] = w1[g]
    want = (x.reshape(T, H * D) @ big.T) @ w2.T
    got = _proj(x, w1, w2, G, d_g, d)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_bad_group_count_is_rejected():
    with pytest.raises(ValueError):
        _proj(np.ones((1, 6, 2)), np.ones((4, 1, 3)), np.ones((1, 4)), 4, 1, 1)
