"""Pins for the RoPE oracle (CPU only): the fp32 emulation against the fp64
definition within its rounding bound, the identity at angle 0, the
relative-position property, pair norms, the relation between the two pairing
conventions, and a hand-worked case."""
import numpy as np
import pytest

import workloads
from oracle import rope_fp32, rope_fp64


@pytest.mark.parametrize("interleaved", [True, False])
def test_fp32_within_rounding_bound(interleaved):
    x = workloads.gen_random((2, 50, 3, 64), 60)
    c, s = workloads.rope_tables(50, 64)
    y32 = rope_fp32(x, c, s, interleaved).astype(np.float64)
    y64 = rope_fp64(x, c, s, interleaved)
    # two rounded products, one rounded sum: |err| <= 2^-23 (|x_a||c| + |x_b||s|) + 2^-24 |y|
    a = np.abs(np.asarray(x, np.float64))
    i = np.arange(32)
    bound = np.empty_like(y64)
    cc, ss = np.abs(c.astype(np.float64))[None, :, None, :], np.abs(s.astype(np.float64))[None, :, None, :]
    ai, bi = (2 * i, 2 * i + 1) if interleaved else (i, i + 32)
    bound[..., ai] = 2.0 ** -23 * (a[..., ai] * cc + a[..., bi] * ss)
    bound[..., bi] = 2.0 ** -23 * (a[..., ai] * ss + a[..., bi] * cc)
    bound += 2.0 ** -24 * np.abs(y64) + 1e-45
    assert np.all(np.abs(y32 - y64) <= bound)


@pytest.mark.parametrize("interleaved", [True, False])
def test_angle_zero_is_identity(interleaved):
    x = workloads.gen_random((1, 7, 2, 16), 61)
    c, s = np.ones((7, 8), np.float32), np.zeros((7, 8), np.float32)
    np.testing.assert_array_equal(rope_fp32(x, c, s, interleaved), x)


@pytest.mark.parametrize("interleaved", [True, False])
def test_relative_position(interleaved):
    """<R(q, m), R(k, n)> depends on m - n only."""
    d = 32
    q = workloads.gen_random((1, 1, 1, d), 62).astype(np.float64)
    k = workloads.gen_random((1, 1, 1, d), 63).astype(np.float64)
    def at(x, pos):
        c, s = workloads.rope_tables(1, d, offset=pos)
        return rope_fp64(x, c.astype(np.float64), s.astype(np.float64), interleaved)[0, 0, 0]
    ref = at(q, 9) @ at(k, 4)
    for t in (1, 17, 300):
        # tables are fp32-rounded angles' cos/sin: agreement to their precision
        assert abs(at(q, 9 + t) @ at(k, 4 + t) - ref) <= 1e-5 * (np.abs(q).sum() * np.abs(k).max() + 1)


@pytest.mark.parametrize("interleaved", [True, False])
def test_pair_norms_preserved(interleaved):
    x = workloads.gen_random((1, 40, 2, 64), 64)
    c, s = workloads.rope_tables(40, 64)
    # renormalise the fp32 tables so cos^2 + sin^2 = 1 exactly in fp64
    r = np.hypot(c.astype(np.float64), s.astype(np.float64))
    y = rope_fp64(x, c / r, s / r, interleaved)
    i = np.arange(32)
    a, b = (2 * i, 2 * i + 1) if interleaved else (i, i + 32)
    xd = np.asarray(x, np.float64)
    np.testing.assert_allclose(y[..., a] ** 2 + y[..., b] ** 2, xd[..., a] ** 2 + xd[..., b] ** 2,
                               rtol=1e-12)


def test_conventions_related_by_permutation():
    """Half-split RoPE is interleaved RoPE conjugated by the permutation that
    sends dims (i, i + d/2) to (2i, 2i + 1)."""
    d = 64
    x = workloads.gen_random((2, 30, 2, d), 65)
    c, s = workloads.rope_tables(30, d)
    perm = np.empty(d, np.int64)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    inv = np.argsort(perm)
    half = rope_fp32(x, c, s, False)
    inter = rope_fp32(x[..., perm], c, s, True)[..., inv]
    np.testing.assert_array_equal(half, inter)


def test_hand_worked_quarter_turn():
    """d = 4, angles (pi/2, 0): pair 0 turns a quarter, pair 1 stays."""
    x = np.array([1.0, 2.0, 3.0, 4.0], np.float32).reshape(1, 1, 1, 4)
    c = np.array([[0.0, 1.0]], np.float32)
    s = np.array([[1.0, 0.0]], np.float32)
    np.testing.assert_array_equal(rope_fp32(x, c, s, True).ravel(), [-2.0, 1.0, 3.0, 4.0])
    np.testing.assert_array_equal(rope_fp32(x, c, s, False).ravel(), [-3.0, 2.0, 1.0, 4.0])
