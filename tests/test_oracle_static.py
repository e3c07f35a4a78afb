"""Pins of the oracle's static-scale mode (the pages' own scale mode: Runway
Characters paper §4.3 "FP8 at write", Appendix G): calibration closed form,
saturation at write, a reset rotation that keeps the scales."""
import numpy as np

from oracle import e4m3, ring
from oracle.rope import rope


def session(n_slots=64, heads=2, d=64, chunks=4, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    st = ring.RingState(n_slots, heads, d)
    for c in range(chunks):
        ring.write(st, rng.standard_normal((16, heads, d)) * scale, rng.standard_normal((16, heads, d)) * scale,
                   np.arange(16 * c, 16 * c + 16))
    return st, rng


def test_calibration_is_margin_times_largest_per_token_scale():
    """Per-token margin-1 rows put their amax element on code 448 exactly, so the
    cache's amax is 448 * max scale and the static scale is fp32(1.5 * max scale)."""
    st, _ = session()
    ring.calibrate_static(st, 1.5)
    for h in range(st.n_heads):
        assert st.static_k[h] == np.float32(1.5 * st.scale_k[h].max())
        assert st.static_v[h] == np.float32(1.5 * st.scale_v[h].max())


def test_static_write_saturates_beyond_the_scale():
    st, rng = session()
    ring.calibrate_static(st, 1.0)
    s_v = st.static_v.copy()
    v = rng.standard_normal((16, 2, 64))
    v[3, 1, 5] = 10 * 448 * s_v[1]      # far beyond the scale: saturates to +448
    v[4, 0, 0] = -448 * s_v[0] * 0.5    # representable: -224 exactly
    ring.write(st, rng.standard_normal((16, 2, 64)), v, np.arange(64, 80))
    first = (st.head - 16) % st.n_slots
    assert e4m3.decode(st.codes_v[1, (first + 3) % 64, 5]) == 448.0
    assert e4m3.decode(st.codes_v[0, (first + 4) % 64, 0]) == -224.0
    assert np.all(st.scale_v[:, (first + np.arange(16)) % 64] == s_v[:, None])


def test_reset_rotation_keeps_static_scales_and_rotates():
    """Keys written with static scales (from data at half the calibration
    range, so nothing clips) keep their scales through a reset rotation, and
    their dequantized values follow RoPE at the shifted positions to within
    the FP8 rounding of the write and of the requantization."""
    st, rng = session(chunks=4, seed=3)
    ring.calibrate_static(st, 1.5)
    k = rng.standard_normal((64, 2, 64)) * 0.5
    pos = np.arange(100, 164)
    for c in range(4):
        ring.write(st, k[16 * c:16 * c + 16], rng.standard_normal((16, 2, 64)), pos[16 * c:16 * c + 16])
    before = st.scale_k.copy()
    ring.rotate(st, -40)
    assert np.array_equal(st.scale_k, before)
    slots = (st.head - 64 + np.arange(64)) % 64  # the 64 keys in write order
    got = e4m3.decode(st.codes_k[:, slots, :]) * st.scale_k[:, slots][..., None]
    want = np.transpose(rope(k, pos - 40), (1, 0, 2))
    # two roundings of at most half a top-binade step (32 / 2) of the scale each
    bound = 32 * st.static_k[:, None, None]
    assert np.all(np.abs(got - want) <= bound)
    assert np.max(np.abs(e4m3.decode(st.codes_k))) < 448  # nothing clipped


def test_reset_returns_to_per_token_scales():
    st, rng = session()
    ring.calibrate_static(st, 1.5)
    ring.reset(st)
    assert st.static_k is None and st.static_v is None
