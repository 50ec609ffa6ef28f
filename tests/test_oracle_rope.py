"""Pins of the rotary-embedding oracle (oracle/rope.py) against what the rotation must satisfy."""
import numpy as np

from oracle.rope import bf16_round, rope


def tables(max_pos, d, base=10000.0):
    # float64 tables built here from the angle definition, independent of workloads.rope_tables
    inv = base ** (-np.arange(d // 2) * 2.0 / d)
    ang = np.outer(np.arange(max_pos), inv)
    return np.cos(ang), np.sin(ang)


def test_angle_zero_is_the_identity():
    x = np.random.default_rng(0).standard_normal((3, 2, 8))
    c, s = tables(4, 8)
    assert np.array_equal(rope(x, np.zeros(3, int), c, s), x)


def test_quarter_turn_by_hand():
    # d = 4: pairs (x0, x2) and (x1, x3); cos 0, sin 1 maps (a, b) to (-b, a)
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    c = np.array([[0.0, 0.0]])
    s = np.array([[1.0, 1.0]])
    assert np.array_equal(rope(x, np.array([0]), c, s), np.array([[[-3.0, -4.0, 1.0, 2.0]]]))
    # a general angle on one pair, worked out: (1, 0) by 30 degrees
    c = np.array([[np.sqrt(3) / 2, 1.0]])
    s = np.array([[0.5, 0.0]])
    got = rope(np.array([[[1.0, 5.0, 0.0, 7.0]]]), np.array([0]), c, s)
    assert np.allclose(got, [[[np.sqrt(3) / 2, 5.0, 0.5, 7.0]]], rtol=0, atol=1e-15)


def test_matches_complex_multiplication():
    rng = np.random.default_rng(1)
    T, H, d = 5, 3, 16
    x = rng.standard_normal((T, H, d))
    pos = rng.integers(0, 100, size=T)
    c, s = tables(100, d)
    z = (x[..., :d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * np.arctan2(s, c))[pos][:, None, :]
    got = rope(x, pos, c, s)
    assert np.allclose(got[..., :d // 2], z.real, atol=1e-12) and np.allclose(got[..., d // 2:], z.imag, atol=1e-12)


def test_rotation_keeps_pair_norms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 2, 32))
    c, s = tables(500, 32)
    y = rope(x, rng.integers(0, 500, size=7), c, s)
    n0 = x[..., :16] ** 2 + x[..., 16:] ** 2
    n1 = y[..., :16] ** 2 + y[..., 16:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)


def test_scores_depend_on_the_position_difference_only():
    rng = np.random.default_rng(3)
    d = 64
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    c, s = tables(4096, d)
    def score(m, n):
        return float(np.sum(rope(q, np.array([m]), c, s) * rope(k, np.array([n]), c, s)))
    for m, n, t in [(5, 2, 100), (700, 699, 3000), (0, 31, 17)]:
        assert abs(score(m, n) - score(m + t, n + t)) < 1e-9


def test_angles_add():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 4, 16))
    c, s = tables(300, 16)
    once = rope(x, np.array([250]), c, s)
    twice = rope(rope(x, np.array([100]), c, s), np.array([150]), c, s)
    assert np.allclose(once, twice, atol=1e-12)


def test_bf16_rounding_is_single_round_to_nearest_even():
    # exactly representable values stay; midpoints go to the even neighbour; others to the nearest
    one = 1.0
    ulp = 2.0 ** -7
    v = np.array([one, one + ulp, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2 ** -30, -2.5, 0.0])
    got = bf16_round(v)
    want = np.array([0x3F80, 0x3F81, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000], np.uint16)
    assert np.array_equal(got, want)
