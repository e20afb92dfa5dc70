"""Pins of the oracle's 3D rotary embedding against facts that do not come from
the oracle itself: the textbook rotary embedding written as explicit 2x2
rotation matrices (RoFormer's block-diagonal form), the relative-position
property, norm preservation, the identity at the origin and composition."""
import math

import numpy as np
import pytest

from oracle import rope3d

PAIRS = (12, 10, 10)


def textbook_rope(x: np.ndarray, pos: int, theta: float = 10000.0) -> np.ndarray:
    """RoFormer's rotary embedding of a d-vector at position pos, built as the
    block-diagonal matrix of 2x2 rotations by pos*theta^(-2(i-1)/d), i = 1..d/2."""
    d = x.shape[-1]
    r = np.zeros((d, d))
    for i in range(1, d // 2 + 1):
        a = pos * theta ** (-2.0 * (i - 1) / d)
        c, s = math.cos(a), math.sin(a)
        r[2 * i - 2, 2 * i - 2] = c
        r[2 * i - 2, 2 * i - 1] = -s
        r[2 * i - 1, 2 * i - 2] = s
        r[2 * i - 1, 2 * i - 1] = c
    return r @ x


def rot(x, t, h, w, ntk=1.0):
    tab = rope3d.rotation_table((np.array([t]), np.array([h]), np.array([w])), PAIRS, 10000.0, ntk)
    return rope3d.apply_rotary(x.reshape(1, 1, -1), tab).reshape(-1)


@pytest.mark.parametrize("axis,lo,hi", [(0, 0, 24), (1, 24, 44), (2, 44, 64)])
def test_single_axis_is_textbook_rope(axis, lo, hi):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(64)
    for p in (1, 2, 7, 37, 63, 1023):
        pos = [0, 0, 0]
        pos[axis] = p
        y = rot(x, *pos)
        np.testing.assert_allclose(y[lo:hi], textbook_rope(x[lo:hi], p), rtol=0, atol=1e-12)
        rest = np.r_[0:lo, hi:64]
        np.testing.assert_array_equal(y[rest], x[rest])


def test_first_pair_rotates_by_position():
    # the first pair of each axis turns by exactly `pos` radians, counter-clockwise
    e = np.zeros(64)
    e[0] = 1.0
    y = rot(e, 3, 0, 0)
    assert abs(y[0] - math.cos(3)) < 1e-15 and abs(y[1] - math.sin(3)) < 1e-15
    e = np.zeros(64)
    e[25] = 1.0      # imaginary part of pair 12 (first h pair)
    y = rot(e, 0, 2, 0)
    assert abs(y[24] + math.sin(2)) < 1e-15 and abs(y[25] - math.cos(2)) < 1e-15


def test_relative_position_invariance():
    rng = np.random.default_rng(2)
    for _ in range(50):
        q, k = rng.standard_normal(64), rng.standard_normal(64)
        p = rng.integers(0, 60, 3)
        pp = rng.integers(0, 60, 3)
        dl = rng.integers(0, 900, 3)
        a = rot(q, *p) @ rot(k, *pp)
        b = rot(q, *(p + dl)) @ rot(k, *(pp + dl))
        assert abs(a - b) < 1e-9 * (1 + abs(a))


def test_norm_of_each_pair_preserved_and_identity_at_origin():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3, 64))
    y = rope3d.rotate_frame(x[:, :, :], 17, 1, 4, 1)   # 1 special + 4 patches
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)
    np.testing.assert_array_equal(rot(x[0, 0], 0, 0, 0), x[0, 0])


def test_composition():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(64)
    a, b = np.array([3, 5, 7]), np.array([11, 2, 30])
    np.testing.assert_allclose(rot(rot(x, *a), *b), rot(x, *(a + b)), atol=1e-12)


def test_token_positions_and_specials():
    t, h, w = rope3d.token_positions(9, 3, 4, 6)
    assert list(t) == [9] * 18
    assert list(h[:6]) == [0] * 6 and list(w[:6]) == [0] * 6
    assert list(h[6:]) == [0, 0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 2]
    assert list(w[6:]) == [0, 1, 2, 3] * 3
    rng = np.random.default_rng(5)
    x = rng.standard_normal((18, 2, 64))
    y = rope3d.rotate_frame(x, 9, 3, 4, 6)
    # special tokens: only the 12 temporal pairs move
    np.testing.assert_array_equal(y[:6, :, 24:], x[:6, :, 24:])
    assert np.abs(y[:6, :, :24] - x[:6, :, :24]).max() > 0.1
    # patch (r, c) = (2, 3): all three axes rotate
    np.testing.assert_allclose(y[6 + 11, 1], rot(x[6 + 11, 1], 9, 2, 3), atol=1e-13)


def test_ntk_factor_stretches_theta():
    rng = np.random.default_rng(6)
    x = rng.standard_normal(64)
    y = rot(x, 5, 6, 7, ntk=4.0)
    np.testing.assert_allclose(y[:24], textbook_rope(x[:24], 5, theta=40000.0), atol=1e-12)
    np.testing.assert_allclose(y[24:44], textbook_rope(x[24:44], 6, theta=40000.0), atol=1e-12)


def test_round_bf16_matches_float32_bit_rounding():
    # pin the oracle's bf16 rounding against rounding the float32 bit pattern
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(100000) * 4).astype(np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32).view(np.float32)
    np.testing.assert_array_equal(rope3d.round_bf16(x.astype(np.float64)), r.astype(np.float64))
    # exact ties go to even
    assert rope3d.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert rope3d.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
