"""Pins of the oracle's Q/K producer step (RMS norm, 3-D rotary embedding,
block means) against closed forms, an independent complex-number form of the
rotation, and invariants (CPU only)."""
import math

import numpy as np
import pytest

from oracle import attention as orc
from oracle import prologue as pro


def test_group_split():
    # D - 4*(D//6) features for the frame axis, 2*(D//6) for rows and columns
    assert pro.rope_split(128) == (44, 42, 42)
    assert pro.rope_split(64) == (24, 20, 20)
    assert pro.rope_split(6) == (2, 2, 2)
    with pytest.raises(ValueError):
        pro.rope_split(7)


def test_closed_form_d6():
    # one pair per axis, theta = 1 for each: token (t, y, x) = (1, 2, 3) of a
    # 2 x 3 x 4 grid; x = [1, 0, 0, 1, 2, 0] has mean square 1, so with gain 1
    # and eps 0 the norm leaves it unchanged
    T, Hg, Wg = 2, 3, 4
    tok = (1 * Hg + 2) * Wg + 3
    x = np.zeros((T * Hg * Wg, 6))
    x[:, 0] = 1.0                       # every token gets x = [1, 0, 0, 1, 2, 0]
    x[:, 3] = 1.0
    x[:, 4] = 2.0
    x[:, 1] = x[:, 2] = x[:, 5] = 0.0
    y = pro.apply_rope(pro.rms_norm(x, np.ones(6), 0.0), pro.rope_angles(T, Hg, Wg, 6, 10000.0))
    expect = [math.cos(1), math.sin(1), -math.sin(2), math.cos(2), 2 * math.cos(3), 2 * math.sin(3)]
    np.testing.assert_allclose(y[tok], expect, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(y[0], [1, 0, 0, 1, 2, 0], atol=1e-15)   # position (0, 0, 0)


def test_closed_form_d12_second_frequency():
    # D = 12: two pairs per axis; base 100 gives theta = (1, 100^(-1/2) = 0.1)
    T, Hg, Wg = 1, 1, 6
    x = np.zeros((6, 12))
    # groups: features 0-3 frame, 4-7 row, 8-11 column (two pairs each)
    x[:, 6:8] = [1.0, 0.0]              # row group, its second pair (theta 0.1)
    x[:, 10:12] = [0.0, 1.0]            # column group, its second pair (theta 0.1)
    g = np.full(12, 2.0)
    y = pro.apply_rope(pro.rms_norm(x, g, 0.0), pro.rope_angles(T, Hg, Wg, 12, 100.0))
    r = math.sqrt(12 / 2)               # 1 / rms: mean square is 2/12
    for col in range(6):
        # column group: features 8, 9 are zero; 10, 11 rotate by 0.1 * column
        np.testing.assert_allclose(y[col, 8:10], [0.0, 0.0], atol=1e-15)
        np.testing.assert_allclose(y[col, 10:12], 2 * r * np.array([-math.sin(0.1 * col), math.cos(0.1 * col)]),
                                   rtol=1e-14, atol=1e-14)
        # the row group sits at row 0 of a one-row grid: unrotated
        np.testing.assert_allclose(y[col, 6:8], [2 * r, 0.0], rtol=1e-14, atol=1e-14)


def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(1)
    T, Hg, Wg, D = 3, 5, 7, 128
    x = rng.normal(size=(T * Hg * Wg, D))
    ang = pro.rope_angles(T, Hg, Wg, D, 10000.0)
    y = pro.apply_rope(x, ang)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * ang)
    np.testing.assert_allclose(y[:, 0::2], z.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[:, 1::2], z.imag, rtol=1e-12, atol=1e-12)
    # per-pair norms are unchanged
    np.testing.assert_allclose(np.hypot(y[:, 0::2], y[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]), rtol=1e-12)


def test_scores_depend_on_relative_position_only():
    # q at token a and k at token b give the same rotated dot product as the
    # same vectors at a + delta and b + delta (delta along each axis)
    rng = np.random.default_rng(2)
    T, Hg, Wg, D = 6, 7, 8, 64
    ang = pro.rope_angles(T, Hg, Wg, D, 10000.0)
    q, k = rng.normal(size=D), rng.normal(size=D)

    def tok(t, y, x):
        return (t * Hg + y) * Wg + x

    def score(a, b):
        return float(pro.apply_rope(q, ang[a]) @ pro.apply_rope(k, ang[b]))
    for (a, b), d in [(((1, 2, 3), (4, 0, 5)), (1, 3, 1)), (((0, 0, 0), (2, 5, 1)), (3, 1, 2))]:
        s0 = score(tok(*a), tok(*b))
        s1 = score(tok(a[0] + d[0], a[1] + d[1], a[2] + d[2]), tok(b[0] + d[0], b[1] + d[1], b[2] + d[2]))
        assert abs(s0 - s1) < 1e-10


def test_rms_norm_scale_invariance_and_unit_mean_square():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(50, 128)) * 3
    y = pro.rms_norm(x, np.ones(128), 0.0)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(pro.rms_norm(7.5 * x, np.ones(128), 0.0), y, rtol=1e-12)


def test_prologue_means_are_block_means_of_rounded_output():
    rng = np.random.default_rng(4)
    T, Hg, Wg, D = 2, 9, 10, 64
    x = rng.normal(size=(T * Hg * Wg, D))
    g = rng.uniform(0.5, 1.5, size=D)
    y, m = pro.qk_prologue(x, g, T, Hg, Wg, eps=1e-6)
    # y holds bf16 values: float32 bit patterns with the low 16 bits clear
    assert not (np.float32(y).view(np.uint32) & 0xFFFF).any()
    np.testing.assert_allclose(m, orc.block_means(y, 64), rtol=1e-13, atol=1e-13)
    order = orc.tile_order(T, Hg, Wg, (1, 8, 8))
    _, mt = pro.qk_prologue(x, g, T, Hg, Wg, eps=1e-6, order=order)
    np.testing.assert_allclose(mt, orc.block_means(y[order], 64), rtol=1e-13, atol=1e-13)
    # and y is the rounded norm + rotation
    ref = pro.apply_rope(pro.rms_norm(x, g, 1e-6), pro.rope_angles(T, Hg, Wg, D, 10000.0))
    assert np.abs(y - ref).max() <= 2.0 ** -8 * np.abs(ref).max()


def test_rms_norm_eps_closed_form():
    # mean square 1 and eps 3: each entry divided by sqrt(1 + 3) = 2
    x = np.array([[1.0, -1.0, 1.0, -1.0, 1.0, -1.0]])
    np.testing.assert_allclose(pro.rms_norm(x, np.full(6, 4.0), 3.0), 2.0 * x, rtol=1e-15)
