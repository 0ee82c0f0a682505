"""Pins for oracle.rope (3D rotary embedding over (t, h, w)).

Checked against: the complex-number statement of rotary embedding (each pair
(a, b) is the complex number a + ib multiplied by exp(i * pos * freq)), an
explicitly built 128 x 128 block-diagonal rotation matrix, norm preservation,
the relative-position property, and the page's theta 256 / split [16, 56, 56]
("Hy-Nomas: an 8.6B world model ...", section "How one segment is made"),
for which the time-band frequencies are exactly 2**-j.
"""

import math

import numpy as np

from oracle import rope

SPLIT = (16, 56, 56)


def test_theta256_time_band_is_powers_of_two():
    w = rope.axis_frequencies(16, 256.0)
    assert np.array_equal(w, 2.0 ** -np.arange(8))


def test_frequencies_first_is_one_and_decreasing():
    for n in SPLIT:
        for th in (256.0, 10000.0):
            w = rope.axis_frequencies(n, th)
            assert w[0] == 1.0 and np.all(np.diff(w) < 0)
            assert np.isclose(w[-1], th ** (-(n - 2) / n), rtol=1e-15)


def test_matches_complex_multiplication():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 128))
    pos = rng.integers(0, 400, (50, 3))
    y = rope.rope3d(x, pos, SPLIT, 10000.0)
    offs = [0, 16, 72]
    for axis, (o, n) in enumerate(zip(offs, SPLIT)):
        z = x[:, :, o:o + n:2] + 1j * x[:, :, o + 1:o + n:2]
        freq = np.array([10000.0 ** (-2.0 * j / n) for j in range(n // 2)])
        rot = np.exp(1j * pos[:, axis][:, None, None] * freq[None, None, :])
        zr = z * rot
        np.testing.assert_allclose(y[:, :, o:o + n:2], zr.real, rtol=0, atol=1e-12)
        np.testing.assert_allclose(y[:, :, o + 1:o + n:2], zr.imag, rtol=0, atol=1e-12)


def _explicit_matrix(pos, theta):
    R = np.zeros((128, 128))
    d = 0
    for axis, n in enumerate(SPLIT):
        for j in range(n // 2):
            ang = pos[axis] * theta ** (-2.0 * j / n)
            c, s = math.cos(ang), math.sin(ang)
            R[d, d], R[d, d + 1] = c, -s
            R[d + 1, d], R[d + 1, d + 1] = s, c
            d += 2
    return R


def test_matches_explicit_rotation_matrix():
    rng = np.random.default_rng(1)
    for theta in (256.0, 10000.0):
        for _ in range(6):
            p = rng.integers(0, 60, 3)
            x = rng.standard_normal(128)
            y = rope.rope3d(x[None, :], p[None, :], SPLIT, theta)[0]
            np.testing.assert_allclose(y, _explicit_matrix(p, theta) @ x, rtol=0, atol=1e-12)


def test_norm_preserved():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((100, 2, 128))
    pos = rng.integers(0, 1000, (100, 3))
    y = rope.rope3d(x, pos)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


def test_dot_product_depends_on_position_difference_only():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((20, 128))
    k = rng.standard_normal((20, 128))
    pq = rng.integers(0, 100, (20, 3))
    pk = rng.integers(0, 100, (20, 3))
    for _ in range(5):
        c = rng.integers(-50, 50, 3)
        a = np.sum(rope.rope3d(q, pq) * rope.rope3d(k, pk), axis=1)
        b = np.sum(rope.rope3d(q, pq + c) * rope.rope3d(k, pk + c), axis=1)
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)


def test_zero_position_is_identity_exactly():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 3, 128))
    assert np.array_equal(rope.rope3d(x, np.zeros((7, 3), np.int64)), x)


def test_axis_bands_are_independent():
    """Moving along one axis only changes that axis's band."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 128))
    base = rope.rope3d(x, np.array([[3, 4, 5]]))
    bands = [(0, 16), (16, 72), (72, 128)]
    for axis in range(3):
        p = np.array([[3, 4, 5]])
        p[0, axis] += 7
        moved = rope.rope3d(x, p)
        for b, (lo, hi) in enumerate(bands):
            same = np.array_equal(moved[:, lo:hi], base[:, lo:hi])
            assert same == (b != axis)


def test_video_positions_raster_order():
    pos = rope.video_positions(5, 2, 4, 6)
    assert pos.shape == (48, 3)
    assert tuple(pos[0]) == (5, 0, 0)
    assert tuple(pos[6]) == (5, 1, 0)          # next row after W = 6 tokens
    assert tuple(pos[23]) == (5, 3, 5)
    assert tuple(pos[24]) == (6, 0, 0)
    fp = rope.frame_positions([9, 2], 4, 6)
    assert tuple(fp[0]) == (9, 0, 0) and tuple(fp[24]) == (2, 0, 0)
