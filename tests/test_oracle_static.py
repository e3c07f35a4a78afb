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
    sk, sv = st.scale_k.copy(), st.scale_v.copy()
    ring.calibrate_static(st, 1.5)
    for h in range(st.n_heads):
        assert st.static_k[h] == np.float32(1.5 * sk[h].max())
        assert st.static_v[h] == np.float32(1.5 * sv[h].max())


def test_calibration_requantizes_the_valid_cache_with_the_head_scales():
    """After the calibration every valid slot carries its head's scales, each
    element is the pre-calibration value rounded once to the head's e4m3 grid
    (within half an ulp of it), nothing saturates (every value is at most
    amax = 448 s / 1.5), and the value-scale bound is the head's scale."""
    st, _ = session()
    before_k, before_v = ring.dequant_k(st), ring.dequant_v(st)
    ring.calibrate_static(st, 1.5)
    slots = ring.valid_slots(st)
    for before, codes, scales, stat in ((before_k, st.codes_k, st.scale_k, st.static_k),
                                        (before_v, st.codes_v, st.scale_v, st.static_v)):
        assert np.all(scales[:, slots] == stat[:, None])
        c = codes[:, slots]
        got = e4m3.decode(c) * stat[:, None, None]
        half = e4m3.ulp_at(c) * stat[:, None, None] / 2
        assert np.all(np.abs(got - before[:, slots]) <= half * (1 + 1e-12))
        assert np.max(np.abs(e4m3.decode(c))) <= 448 / 1.5 + 16  # at most one step above amax/s
    assert np.array_equal(st.vmax, st.static_v)


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


def test_rotation_right_after_calibration_moves_old_keys_to_the_head_scale():
    """Keys written with per-token scales before the calibration and rotated
    before any rewrite: the rotation requantizes them with the head's static
    scale, which covers every rotated component (pair norm <= sqrt(2) amax <
    1.5 amax), so nothing clips and every key stays within the write's
    rounding plus one requantization of RoPE at the shifted position."""
    rng = np.random.default_rng(7)
    st = ring.RingState(700, 2, 64)
    ks, pos = [], []
    for c in range(2):
        k = rng.standard_normal((300, 2, 64))
        p = np.arange(300 * c, 300 * c + 300)
        ring.write(st, k, rng.standard_normal((300, 2, 64)), p)
        ks.append(k)
        pos.append(p)
    ring.calibrate_static(st, 1.5)
    per_token = st.scale_k.copy()
    ring.rotate(st, -600)
    slots = ring.valid_slots(st)  # the 600 keys in write order
    assert np.all(st.scale_k[:, slots] == st.static_k[:, None])
    assert np.max(np.abs(e4m3.decode(st.codes_k[:, slots]))) < 448  # nothing clipped
    got = e4m3.decode(st.codes_k[:, slots, :]) * st.scale_k[:, slots][..., None]
    want = np.transpose(rope(np.concatenate(ks), np.concatenate(pos) - 600), (1, 0, 2))
    # write rounding: half a top-binade step of the per-token scale, carried
    # through the rotation as a pair (sqrt 2); requantization: half a step of
    # the static scale
    bound = np.sqrt(2) * 16 * per_token[:, slots][..., None] + 16 * st.static_k[:, None, None]
    assert np.all(np.abs(got - want) <= bound * (1 + 1e-9))
    # keeping each key's own per-token scale instead would clip about half of them
    kept = ring.RingState(700, 2, 64)
    rng = np.random.default_rng(7)
    for c in range(2):
        ring.write(kept, rng.standard_normal((300, 2, 64)), rng.standard_normal((300, 2, 64)),
                   np.arange(300 * c, 300 * c + 300))
    x = e4m3.decode(kept.codes_k[:, slots]) * kept.scale_k[:, slots][..., None]
    from oracle.rope import delta_angles, rotate_pairs
    y = rotate_pairs(x, *delta_angles(64, -600))
    clipped = np.any(np.abs(y) > 448 * kept.scale_k[:, slots][..., None], axis=-1)
    assert clipped.mean() > 0.2


def test_zero_amax_head_keeps_per_token_scales():
    """Calibrating a layer with nothing valid (amax 0) gives zero static scales:
    those heads keep the per-(token, head) rule, so later writes store the same
    codes and scales as an uncalibrated ring instead of zero codes."""
    rng = np.random.default_rng(8)
    cal = ring.RingState(64, 2, 64)
    ring.calibrate_static(cal, 1.5)
    assert not cal.static_k.any() and not cal.static_v.any()
    plain = ring.RingState(64, 2, 64)
    k, v = rng.standard_normal((16, 2, 64)), rng.standard_normal((16, 2, 64))
    for st in (cal, plain):
        ring.write(st, k, v, np.arange(16))
        ring.rotate(st, -5)
    assert np.array_equal(cal.codes_k, plain.codes_k) and np.array_equal(cal.codes_v, plain.codes_v)
    assert np.array_equal(cal.scale_k, plain.scale_k) and np.array_equal(cal.scale_v, plain.scale_v)
    assert np.any(cal.codes_k[:, :16] != 0)


def test_zero_key_head_static_values_only():
    """A head whose cached keys are all zero but whose values are not: the keys
    stay per-token (scale 0 static), the values go static."""
    rng = np.random.default_rng(9)
    st = ring.RingState(64, 2, 64)
    k = rng.standard_normal((16, 2, 64))
    k[:, 1] = 0.0
    ring.write(st, k, rng.standard_normal((16, 2, 64)), np.arange(16))
    ring.calibrate_static(st, 1.5)
    assert st.static_k[1] == 0 and st.static_k[0] > 0 and np.all(st.static_v > 0)
    k2 = rng.standard_normal((16, 2, 64))
    v2 = rng.standard_normal((16, 2, 64))
    ring.write(st, k2, v2, np.arange(16, 32))
    new = np.arange(16, 32)
    assert np.all(st.scale_k[0, new] == st.static_k[0])
    assert np.all(st.scale_v[:, new] == st.static_v[:, None])
    # head 1's keys: per-token rule, amax maps to 448
    assert np.all(np.max(np.abs(e4m3.decode(st.codes_k[1, new])), axis=-1) == 448)
    assert np.all(st.scale_k[1, new] == np.float32(np.max(np.abs(rope(k2, new)[:, 1]), axis=-1) / 448))


def test_static_attention_emulation_equals_the_per_token_formula_on_calibrated_heads():
    """On a calibrated cache every valid slot carries its head's scales, so the
    kernel's static attention (s_k folded into the queries, x = 7 P, s_v
    after the product) is the per-token emulation with s_v = vmax: the two
    differ only where folding s_k into Q moves a query code and in the last
    bits (fp32 c against the exact 7), and both sit within the contract of
    exact attention; heads with a zero static scale take the per-token rule."""
    from oracle import attend
    from oracle.bf16 import round_bf16
    st, rng = session(n_slots=200, chunks=10, seed=5)
    ring.calibrate_static(st, 1.5)
    q = rng.standard_normal((40, 2, 64))
    pos = np.arange(100, 140)
    stat = attend.attend_emul(st, q, pos)
    plain = st.copy()
    plain.static_k = plain.static_v = None  # same cache, per-token numerics
    tok = attend.attend_emul(plain, q, pos)
    ex = attend.attend_exact(st, q, pos)
    sig = np.maximum(1, attend.sigma_v(st))[None]
    assert np.max(np.abs(stat - tok) / sig) < 5e-3
    for out in (stat, tok):
        e = np.abs(round_bf16(out) - ex) / sig
        assert e.max() < 2e-2 and e.mean() < 2e-3
    # one value code at 448 (the row max of a one-slot cache): x = 7 exactly
    one = ring.RingState(16, 1, 64)
    ring.write(one, rng.standard_normal((1, 1, 64)), rng.standard_normal((1, 1, 64)), [3])
    ring.calibrate_static(one, 1.5)
    got = attend.attend_emul(one, rng.standard_normal((3, 1, 64)), np.arange(3))
    want = ring.dequant_v(one)[:, 0, :]
    assert np.max(np.abs(got - want[None])) <= 1e-15 * np.max(np.abs(want))
