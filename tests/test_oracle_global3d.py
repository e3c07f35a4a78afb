"""Pins of the oracle's global (sink) slots and 3-D RoPE (Runway Characters
paper, §2 "The step budget": 1,246 global slots written once per session
beside the six-latent window; §4.2 and Appendix G: the temporal angle is
omega_j (a t + b), spatial angles and global tokens do not move at a reset).

References: a complex-number formulation of banded RoPE, the 1-D RoPE as the
one-band special case, the rotation identity per band, permutation
invariance of attention (globals + ring equal a plain ring holding the same
tokens), and a hand-derived bookkeeping case (tests/golden)."""
import os

import numpy as np

from oracle import attend, e4m3, ring, rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_global3d_positions.txt")
BANDS = (22, 21, 21)  # D = 128


def test_one_band_is_the_1d_rope():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((9, 2, 64))
    p = rng.integers(-5000, 40000, 9)
    pos3 = np.stack([p, rng.integers(0, 50, 9), rng.integers(0, 50, 9)], 1)
    assert np.array_equal(rope.rope3d(x, pos3, (32, 0, 0)), rope.rope(x, p))


def test_banded_rope_equals_complex_rotation_per_band():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 3, 128))
    pos3 = rng.integers(-300, 300, (7, 3))
    got = rope.rope3d(x, pos3, BANDS)
    z = x[..., 0::2] + 1j * x[..., 1::2]  # [n, H, 64]
    want = np.empty_like(z)
    k = 0
    for axis, nb in enumerate(BANDS):
        w = 10000.0 ** (-np.arange(nb) / nb)
        want[..., k:k + nb] = z[..., k:k + nb] * np.exp(1j * pos3[:, axis][:, None, None] * w[None, None, :])
        k += nb
    assert np.allclose(got[..., 0::2], want.real, atol=1e-12) and np.allclose(got[..., 1::2], want.imag, atol=1e-12)


def test_relative_position_per_axis():
    """q(p) . k(p') depends only on p - p' on every axis."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    p, pp = np.array([[40, 3, 7]]), np.array([[11, 9, 2]])
    shift = np.array([[-17, 5, 30]])
    a = np.sum(rope.rope3d(q, p, BANDS) * rope.rope3d(k, pp, BANDS))
    b = np.sum(rope.rope3d(q, p + shift, BANDS) * rope.rope3d(k, pp + shift, BANDS))
    assert abs(a - b) < 1e-10


def test_reset_rotates_the_temporal_band_only():
    """The reset rotation of a RoPE'd key equals RoPE at (t + delta, y, x)
    (float64, to 1e-12), and leaves the spatial pairs' values exactly."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 2, 128))
    pos3 = rng.integers(0, 100, (6, 3))
    y = rope.rope3d(x, pos3, BANDS)
    c, s = rope.delta_angles3d(128, BANDS, -42)
    rot = rope.rotate_pairs(y, c, s)
    assert np.allclose(rot, rope.rope3d(x, pos3 + [[-42, 0, 0]], BANDS), atol=1e-12)
    spatial = np.repeat(np.arange(64) >= BANDS[0], 2)
    assert np.array_equal(rot[..., spatial], y[..., spatial])


def session(static=False, seed=4):
    rng = np.random.default_rng(seed)
    st = ring.RingState(40, 2, 128, n_global=12, bands=BANDS)
    toks = []
    for first, n in ((0, 7), (7, 5)):
        k, v = rng.standard_normal((n, 2, 128)), rng.standard_normal((n, 2, 128))
        pos = np.stack([np.full(n, 1000), np.arange(first, first + n) // 4, np.arange(first, first + n) % 4], 1)
        ring.write_global(st, first, k, v, pos)
        toks.append((k, v, pos))
    if static:
        ring.calibrate_static(st, 1.5)
    for c in range(5):  # 5 x 11 tokens into 40 slots: the ring wraps
        k, v = rng.standard_normal((11, 2, 128)), rng.standard_normal((11, 2, 128))
        pos = np.stack([np.full(11, c), np.arange(11) // 4, np.arange(11) % 4], 1)
        ring.write(st, k, v, pos)
        toks.append((k, v, pos))
    return st, toks, rng


def test_globals_are_never_rotated_and_spatial_codes_stay_under_static_scales():
    for static in (False, True):
        st, _, _ = session(static)
        before = st.copy()
        ring.rotate(st, -42)
        g = slice(st.n_slots, st.n_slots + st.n_global)
        for a in ("codes_k", "codes_v", "scale_k", "scale_v"):
            assert np.array_equal(getattr(st, a)[:, g], getattr(before, a)[:, g]), a
        assert np.array_equal(st.slot_pos[g], before.slot_pos[g])
        assert np.array_equal(st.slot_yx, before.slot_yx)
        ringv = ring.ring_valid_slots(st)
        assert np.array_equal(st.slot_pos[ringv], before.slot_pos[ringv] - 42)
        if static:  # the head's scale is kept, so unrotated pairs re-encode to the same codes
            spatial = np.repeat(np.arange(64) >= BANDS[0], 2)
            assert np.array_equal(st.codes_k[:, ringv][..., spatial], before.codes_k[:, ringv][..., spatial])


def test_globals_plus_ring_attend_like_one_plain_ring_of_the_same_tokens():
    """Attention is permutation-invariant: the 12 globals and the 40 valid ring
    slots give the same exact attention as a plain 52-slot ring holding the
    same quantized tokens (their codes and scales copied)."""
    st, _, rng = session()
    slots = ring.valid_slots(st)
    assert slots.size == 52
    flat = ring.RingState(52, 2, 128, bands=BANDS, head=0, n_valid=52)
    for a in ("codes_k", "codes_v", "scale_k", "scale_v"):
        getattr(flat, a)[:] = getattr(st, a)[:, slots]
    q = rng.standard_normal((9, 2, 128))
    qpos = np.stack([np.full(9, 5), np.arange(9), np.arange(9)], 1)
    assert np.allclose(attend.attend_exact(st, q, qpos), attend.attend_exact(flat, q, qpos), atol=1e-12)
    # only the globals written are read: with g_valid 7 the last 5 drop out
    part = st.copy()
    part.g_valid = 7
    sl = ring.valid_slots(part)
    assert sl.size == 47 and sl.max() == st.n_slots + 6


def test_golden_bookkeeping_case():
    want = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if line:
            want[line[0]] = [int(v) for v in line[1:]]
    st = ring.RingState(8, 1, 64, n_global=4, bands=(16, 8, 8))
    rng = np.random.default_rng(5)
    z = lambda n: rng.standard_normal((n, 1, 64))
    ring.write_global(st, 0, z(2), z(2), [(100, 0, 0), (100, 0, 1)])
    ring.write_global(st, 2, z(1), z(1), [(100, 1, 0)])
    ring.write(st, z(3), z(3), [(0, 0, 0), (0, 0, 1), (0, 1, 0)])
    ring.write(st, z(3), z(3), [(1, 0, 0), (1, 0, 1), (1, 1, 0)])
    ring.write(st, z(4), z(4), [(2, 0, 0), (2, 0, 1), (2, 1, 0), (2, 1, 1)])
    assert [st.head, st.n_valid, st.g_valid] == want["head"] + want["n_valid"] + want["g_valid"]
    assert st.slot_pos.tolist() == want["t"]
    assert st.slot_yx[:, 0].tolist() == want["y"] and st.slot_yx[:, 1].tolist() == want["x"]
    assert ring.valid_slots(st).tolist() == want["valid"]
    ring.rotate(st, -5)
    assert st.slot_pos.tolist() == want["t_after"]


def test_global_writes_quantize_like_ring_writes():
    """A token written to a global slot gets the same codes and scales as the
    same token written to the ring."""
    rng = np.random.default_rng(6)
    k, v = rng.standard_normal((3, 2, 128)) * 4, rng.standard_normal((3, 2, 128))
    pos = [(7, 1, 2), (7, 2, 2), (9, 0, 0)]
    a = ring.RingState(16, 2, 128, n_global=5, bands=BANDS)
    ring.write_global(a, 2, k, v, pos)
    b = ring.RingState(16, 2, 128, bands=BANDS)
    ring.write(b, k, v, pos)
    assert np.array_equal(a.codes_k[:, 18:21], b.codes_k[:, 0:3]) and np.array_equal(a.scale_v[:, 18:21], b.scale_v[:, 0:3])
    assert np.array_equal(e4m3.decode(a.codes_v[:, 18:21]), e4m3.decode(b.codes_v[:, 0:3]))
