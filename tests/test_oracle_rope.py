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


# ---------------------------------------------------------------- half-split layout

PAIRS_2D = (0, 16, 16)


def rot_half(x, t, h, w, pairs=PAIRS_2D, theta=100.0):
    tab = rope3d.rotation_table((np.array([t]), np.array([h]), np.array([w])), pairs, theta, 1.0)
    return rope3d.apply_half_split(x.reshape(1, 1, -1), tab, pairs).reshape(-1)


def rotate_half_rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """A 1D rotary embedding of a d-vector in the split-halves arrangement,
    written as the matrix [[C, -S], [S, C]] with C, S = diag(cos, sin) of
    pos * theta^(-2i/d), i < d/2 -- the rotate-half form of the 2D module."""
    d = x.shape[-1]
    a = pos * theta ** (-2.0 * np.arange(d // 2) / d)
    c, s = np.diag(np.cos(a)), np.diag(np.sin(a))
    r = np.block([[c, -s], [s, c]])
    return r @ x


def test_half_split_unit_vector_closed_form():
    """e_i of the h block turns into cos(h*w_i) e_i + sin(h*w_i) e_{i+16},
    w_i = 100^(-i/16): for i = 0 the angle is h, for i = 8 it is h/10."""
    for i, omega in ((0, 1.0), (8, 0.1), (15, 100.0 ** (-15 / 16))):
        x = np.zeros(64)
        x[i] = 1.0
        y = rot_half(x, 5, 3, 2)
        want = np.zeros(64)
        want[i] = math.cos(3 * omega)
        want[i + 16] = math.sin(3 * omega)
        assert np.allclose(y, want, atol=1e-14), i
        # the w block (channels 32..63) takes the w coordinate
        x = np.zeros(64)
        x[32 + i] = 1.0
        y = rot_half(x, 5, 3, 2)
        want = np.zeros(64)
        want[32 + i] = math.cos(2 * omega)
        want[48 + i] = math.sin(2 * omega)
        assert np.allclose(y, want, atol=1e-14), i


@pytest.mark.parametrize("lo,axis", [(0, 1), (32, 2)])
def test_half_split_block_is_rotate_half_rope(lo, axis):
    rng = np.random.default_rng(5)
    x = rng.standard_normal(64)
    for p in (1, 4, 9, 63):
        pos = [7, 0, 0]
        pos[axis] = p
        y = rot_half(x, *pos)
        assert np.allclose(y[lo:lo + 32], rotate_half_rope(x[lo:lo + 32], p, 100.0), atol=1e-12)
        other = slice(32, 64) if lo == 0 else slice(0, 32)
        # the other block sees its own coordinate only (0 here)
        assert np.allclose(y[other], x[other], atol=1e-12)


def test_half_split_is_interleaved_after_a_channel_permutation():
    """Moving channel (block + i, block + i + pairs_a) to the adjacent pair
    (2(col + i), 2(col + i) + 1) turns the half-split rotation into the
    interleaved one, for any split with a t block."""
    pairs = (16, 8, 8)
    perm = []
    ch = 0
    for n in pairs:
        for i in range(n):
            perm += [ch + i, ch + n + i]
        ch += 2 * n
    perm = np.array(perm)          # interleaved slot k holds half-split channel perm[k]
    rng = np.random.default_rng(6)
    x = rng.standard_normal(64)
    tab = rope3d.rotation_table((np.array([11]), np.array([4]), np.array([9])), pairs, 100.0, 1.0)
    y_half = rope3d.apply_half_split(x.reshape(1, 1, -1), tab, pairs).reshape(-1)
    y_int = rope3d.apply_rotary(x[perm].reshape(1, 1, -1), tab).reshape(-1)
    assert np.allclose(y_half[perm], y_int, atol=1e-12)


def test_half_split_relative_position_and_norm():
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    base = np.dot(rot_half(q, 0, 3, 5), rot_half(k, 0, 1, 2))
    for d in ((0, 4, 1), (0, 10, 20), (0, 60, 33)):
        moved = np.dot(rot_half(q, 0, 3 + d[1], 5 + d[2]), rot_half(k, 0, 1 + d[1], 2 + d[2]))
        assert abs(moved - base) < 1e-10
    y = rot_half(q, 0, 17, 29)
    # norm of every rotating pair (i, i + 16) within each block
    for lo in (0, 32):
        for i in range(16):
            a = np.hypot(q[lo + i], q[lo + i + 16])
            b = np.hypot(y[lo + i], y[lo + i + 16])
            assert abs(a - b) < 1e-12
    assert np.allclose(rot_half(q, 0, 0, 0), q, atol=0)
