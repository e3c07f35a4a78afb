"""Rotary position embedding in float64 (test infrastructure).

Runway Characters paper, §4.2 "RoPE at write, and a delta rotation at reset"
and Appendix G: each new token's queries and keys are rotated once, before
the cache write; a cached key's angle for frequency j is theta_j(t) =
omega_j * (a t + b), so a position change by Delta is one more rotation by
omega_j * a * Delta.

The pages do not fix the pair layout or the frequencies.  Readings taken here
(the RoFormer form the pages cite): pairs are interleaved elements (2j, 2j+1)
of the head dimension; omega_j = base**(-2j/D) with base 10000; token
positions are 1-D integers, so a = 1 and b = 0.  All angles and trigonometry
are float64.
"""
from __future__ import annotations

import numpy as np


def omega(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """Frequencies omega_j = base**(-2j/D), j = 0 .. D/2-1, in float64."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * j / head_dim)


def rotate_pairs(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate each interleaved pair (x[2j], x[2j+1]) by the angle with (cos, sin).

    ``cos``/``sin`` broadcast against x[..., 0::2]:
    y0 = x0 cos - x1 sin,  y1 = x0 sin + x1 cos.
    """
    x = np.asarray(x, dtype=np.float64)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * cos - x1 * sin
    y[..., 1::2] = x0 * sin + x1 * cos
    return y


def rope(x: np.ndarray, pos: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """RoPE of tokens x [n, H, D] at integer positions pos [n] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    n, _, d = x.shape
    w = omega(d, base)
    theta = np.asarray(pos, dtype=np.float64)[:, None] * w[None, :]  # [n, D/2]
    c = np.cos(theta)[:, None, :]
    s = np.sin(theta)[:, None, :]
    return rotate_pairs(x, c, s)


def delta_angles(head_dim: int, delta: int, base: float = 10000.0):
    """(cos, sin) of phi_j = delta * omega_j, float64, shape [D/2]."""
    phi = np.float64(delta) * omega(head_dim, base)
    return np.cos(phi), np.sin(phi)


# ---- 3-D RoPE (global slots and banded positions) ---------------------------
#
# The pages' model places each token at a temporal index t (the latent frame)
# and spatial coordinates; the temporal angle of frequency j is
# theta_j(t) = omega_j (a t + b), spatial angles and global tokens do not
# depend on the window, and a reset rotates only the temporal frequencies
# (§4.2, Appendix G).  The pages do not give the band layout.  Readings taken
# here: the D/2 interleaved pairs of a head form three contiguous bands of
# n_t, n_y and n_x pairs (temporal, height, width; the caller chooses the
# counts, n_t + n_y + n_x = D/2); each band is a RoPE of its own dimension
# 2 n_b, omega_{b,j} = base**(-j / n_b) for its j-th pair, at the token's
# coordinate on that axis; a = 1, b = 0.  With n_y = n_x = 0 this is the 1-D
# RoPE above (omega_j = base**(-2j/D) at position t).


def band_table(head_dim: int, bands, base: float = 10000.0):
    """Per pair j: (axis index 0 = t, 1 = y, 2 = x; omega) as two arrays [D/2]."""
    n_t, n_y, n_x = (int(b) for b in bands)
    if n_t + n_y + n_x != head_dim // 2 or min(n_t, n_y, n_x) < 0:
        raise ValueError("bands must be non-negative pair counts summing to head_dim / 2")
    axis, om = [], []
    for a, nb in enumerate((n_t, n_y, n_x)):
        j = np.arange(nb, dtype=np.float64)
        axis.append(np.full(nb, a, dtype=np.int64))
        om.append(np.power(np.float64(base), -j / nb) if nb else j)
    return np.concatenate(axis), np.concatenate(om)


def rope3d(x: np.ndarray, pos3: np.ndarray, bands, base: float = 10000.0) -> np.ndarray:
    """RoPE of tokens x [n, H, D] at coordinates pos3 [n, 3] = (t, y, x), banded."""
    x = np.asarray(x, dtype=np.float64)
    n, _, d = x.shape
    axis, om = band_table(d, bands, base)
    p = np.asarray(pos3, dtype=np.float64).reshape(n, 3)
    theta = p[:, axis] * om[None, :]  # [n, D/2]
    return rotate_pairs(x, np.cos(theta)[:, None, :], np.sin(theta)[:, None, :])


def delta_angles3d(head_dim: int, bands, delta: int, base: float = 10000.0):
    """(cos, sin) [D/2] of a reset by delta temporal positions: temporal pairs
    rotate by delta * omega_j, spatial pairs not at all (cos 1, sin 0)."""
    axis, om = band_table(head_dim, bands, base)
    phi = np.where(axis == 0, np.float64(delta) * om, 0.0)
    return np.cos(phi), np.sin(phi)
