"""Pins for the oracle's RoPE (CPU only).

Runway Characters paper, §4.2: keys and queries are rotated once at their own
positions; a position change by Delta is one more rotation by omega_j * Delta
per frequency (the rotation identity).  The references here are closed forms,
an independent complex-number formulation of the same rotation, and the
rotation identity itself.
"""
import math

import numpy as np

from oracle import rope


def rope_complex(x, pos, base=10000.0):
    """RoPE written as multiplication of (x[2j] + i x[2j+1]) by exp(i pos omega_j)."""
    x = np.asarray(x, dtype=np.float64)
    n, h, d = x.shape
    z = x[..., 0::2] + 1j * x[..., 1::2]
    j = np.arange(d // 2)
    w = np.array([base ** (-2.0 * jj / d) for jj in j])
    rot = np.exp(1j * np.outer(np.asarray(pos, dtype=np.float64), w))[:, None, :]
    zr = z * rot
    out = np.empty_like(x)
    out[..., 0::2] = zr.real
    out[..., 1::2] = zr.imag
    return out


def test_omega_closed_forms():
    assert np.allclose(rope.omega(4), [1.0, 0.01], rtol=0, atol=1e-18)
    w = rope.omega(128)
    assert w[0] == 1.0
    assert math.isclose(w[1], 10000 ** (-1 / 64), rel_tol=1e-15)
    assert math.isclose(w[63], 10000 ** (-126 / 128), rel_tol=1e-15)


def test_single_pair_closed_form():
    x = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    y = rope.rope(x, np.array([1, 1]))
    assert np.allclose(y[0, 0], [math.cos(1), math.sin(1)], atol=1e-15)
    assert np.allclose(y[1, 0], [-math.sin(1), math.cos(1)], atol=1e-15)


def test_interleaved_layout():
    # D = 4: pair 0 = elements (0, 1) at omega 1, pair 1 = elements (2, 3) at omega 0.01.
    p = 7
    y = rope.rope(np.array([[[1.0, 0, 0, 0]]]), np.array([p]))
    assert np.allclose(y[0, 0], [math.cos(p), math.sin(p), 0, 0], atol=1e-15)
    y = rope.rope(np.array([[[0, 0, 1.0, 0]]]), np.array([p]))
    assert np.allclose(y[0, 0], [0, 0, math.cos(0.01 * p), math.sin(0.01 * p)], atol=1e-15)


def test_matches_complex_formulation():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 128))
    pos = rng.integers(-40000, 40000, 50)
    assert np.allclose(rope.rope(x, pos), rope_complex(x, pos), atol=1e-9, rtol=0)


def test_zero_position_is_identity():
    x = np.random.default_rng(1).standard_normal((5, 2, 64))
    assert np.array_equal(rope.rope(x, np.zeros(5, dtype=np.int64)), x)


def test_pair_norms_preserved():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((20, 2, 64))
    y = rope.rope(x, rng.integers(0, 30000, 20))
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(nx, ny, rtol=1e-12)


def test_rotation_identity_composes():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((30, 2, 128))
    p = rng.integers(0, 32000, 30)
    for d in (-80, -31794, 5, 1):
        c, s = rope.delta_angles(128, d)
        lhs = rope.rotate_pairs(rope.rope(x, p), c, s)
        rhs = rope.rope(x, p + d)
        assert np.max(np.abs(lhs - rhs)) < 1e-10


def test_relative_position_property():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    base = float(np.sum(rope.rope(q, [100]) * rope.rope(k, [37])))
    for t in (-500, 3, 12345):
        moved = float(np.sum(rope.rope(q, [100 + t]) * rope.rope(k, [37 + t])))
        assert math.isclose(base, moved, rel_tol=1e-9, abs_tol=1e-9)
