"""Pins for the oracle's attention (CPU only).

Runway Characters paper: each call attends its new queries over every slot of
its cache, including the chunk just written (§2 "The step budget", Appendix G);
queries get RoPE at their own positions and cached keys are used as stored
(§4.2); only the queries are quantized per call (§4.3).

References: torch's float64 scaled_dot_product_attention (a library routine)
on the dequantized cache, a scalar-loop brute force, closed-form special
cases (one valid slot, identical keys, lossless queries), and the ring's
permutation invariance (a wrapped ring equals a linear cache holding the
same tokens).
"""
import math

import numpy as np
import torch

from oracle import attend, e4m3, ring, rope
from oracle.bf16 import round_bf16
from workloads import TINY, Stream, positions


def tiny_session(n_writes=6):
    st = ring.RingState(TINY.n_slots, TINY.n_heads, TINY.head_dim)
    s = Stream(TINY)
    chunks = []
    for c in range(n_writes):
        q, k, v = s.chunk()
        pos = positions(16 * c, 16)
        ring.write(st, k.f64, v.f64, pos)
        chunks.append((q, k, v, pos))
    return st, chunks


def torch_reference(st, q, q_pos):
    slots = ring.valid_slots(st)
    qr = torch.tensor(rope.rope(q, q_pos)).permute(1, 0, 2)  # [H, n_q, D]
    k = torch.tensor(ring.dequant_k(st)[:, slots, :])
    v = torch.tensor(ring.dequant_v(st)[:, slots, :])
    out = torch.nn.functional.scaled_dot_product_attention(qr, k, v)
    return out.permute(1, 0, 2).numpy()


def brute_force(st, q, q_pos):
    """Scalar loops over heads, queries, slots and channels."""
    qr = rope.rope(q, q_pos)
    kd = ring.dequant_k(st)
    vd = ring.dequant_v(st)
    slots = [int(x) for x in ring.valid_slots(st)]
    n_q, h, d = q.shape
    out = np.zeros((n_q, h, d))
    for hh in range(h):
        for i in range(n_q):
            logits = []
            for sl in slots:
                acc = 0.0
                for c in range(d):
                    acc += qr[i, hh, c] * kd[hh, sl, c]
                logits.append(acc / math.sqrt(d))
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            tot = sum(w)
            for c in range(d):
                out[i, hh, c] = sum(w[j] * vd[hh, slots[j], c] for j in range(len(slots))) / tot
    return out


def test_exact_matches_torch_sdpa_after_each_write():
    st = ring.RingState(TINY.n_slots, TINY.n_heads, TINY.head_dim)
    s = Stream(TINY)
    for c in range(6):
        q, k, v = s.chunk()
        pos = positions(16 * c, 16)
        ring.write(st, k.f64, v.f64, pos)
        got = attend.attend_exact(st, q.f64, pos)
        ref = torch_reference(st, q.f64, pos)
        assert np.max(np.abs(got - ref)) < 1e-12, c


def test_exact_matches_brute_force_after_reset():
    st, chunks = tiny_session()
    ring.rotate(st, -80)
    q, _, _, pos = chunks[5]
    got = attend.attend_exact(st, q.f64[:4], pos[:4] - 80)
    ref = brute_force(st, q.f64[:4], pos[:4] - 80)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_one_valid_slot_returns_its_value():
    rng = np.random.default_rng(3)
    st = ring.RingState(32, 2, 16)
    ring.write(st, rng.standard_normal((1, 2, 16)), rng.standard_normal((1, 2, 16)), np.array([5]))
    q = rng.standard_normal((7, 2, 16)) * 10
    vd = ring.dequant_v(st)[:, 0, :]  # [H, D]
    for fn in (attend.attend_exact, attend.attend_method):
        out = fn(st, q, np.arange(7))
        assert np.max(np.abs(out - vd[None])) < 1e-15, fn.__name__
    # emul: P' = 1 * s_v * c = 448 * 2**-headroom exactly up to the fp32 rounding of c
    for hr in (0, 2, 6):
        out = attend.attend_emul(st, q, np.arange(7), headroom=hr)
        assert np.all(np.abs(out - vd[None]) <= 2 ** -22 * np.abs(vd[None]))


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(4)
    st = ring.RingState(40, 1, 32)
    k = np.repeat(rng.standard_normal((1, 1, 32)), 40, axis=0)
    v = rng.standard_normal((40, 1, 32))
    ring.write(st, k, v, np.zeros(40, dtype=np.int64))  # same key, same position
    q = rng.standard_normal((5, 1, 32))
    mean_v = ring.dequant_v(st)[0].mean(axis=0)
    for fn in (attend.attend_exact, attend.attend_method):
        out = fn(st, q, np.arange(5))
        assert np.max(np.abs(out[:, 0, :] - mean_v[None])) < 1e-13


def test_empty_cache_gives_zeros():
    st = ring.RingState(16, 2, 8)
    q = np.ones((3, 2, 8))
    for fn in (attend.attend_exact, attend.attend_method, attend.attend_emul):
        assert not fn(st, q, np.arange(3)).any()


def test_wrapped_ring_equals_linear_cache():
    """Attention is a function of the valid tokens only, not of where the ring put them."""
    st, chunks = tiny_session()  # head 32: valid data wraps
    lin = ring.RingState(TINY.n_slots, TINY.n_heads, TINY.head_dim)
    for c in (2, 3, 4, 5):  # the resident chunks, written from slot 0 in order
        _, k, v, pos = chunks[c]
        ring.write(lin, k.f64, v.f64, pos)
    assert lin.head == 0 and st.head == 32
    q, _, _, pos = chunks[5]
    for fn in (attend.attend_exact, attend.attend_method, attend.attend_emul):
        a = fn(st, q.f64, pos)
        b = fn(lin, q.f64, pos)
        assert np.max(np.abs(a - b)) < 1e-12, fn.__name__


def test_reset_is_a_global_position_shift():
    """Before vs after a delta rotation with queries moved by the same delta."""
    st, chunks = tiny_session()
    q, _, _, pos = chunks[5]
    before = attend.attend_exact(st, q.f64, pos)
    ring.rotate(st, -80)
    after = attend.attend_exact(st, q.f64, pos - 80)
    # the rotation requantizes each key once: the logits move by a few FP8 steps
    assert np.max(np.abs(after - before)) < 0.05
    assert np.mean(np.abs(after - before)) < 0.005


def test_lossless_queries_make_method_equal_exact():
    """Queries whose scaled RoPE'd values are e4m3 values times 2**e quantize
    without loss: the method is then exact attention, with the float32
    softmax factor in place of log2(e)/sqrt(D)."""
    rng = np.random.default_rng(6)
    st = ring.RingState(48, 2, 16)
    ring.write(st, rng.standard_normal((48, 2, 16)), rng.standard_normal((48, 2, 16)), np.arange(48))
    grid = e4m3.decode(np.arange(0, 0x7F, dtype=np.uint8))
    cs = attend.softmax_scale_log2(16)
    assert abs(cs - math.log2(math.e) / 4.0) <= 2.0 ** -24 * cs  # one float32 rounding
    qg = rng.choice(grid, size=(6, 2, 16)) * rng.choice([-1.0, 1.0], size=(6, 2, 16)) * 2.0 ** -5
    qr = qg / cs  # qr * cs rounds back to qg: well inside half an e4m3 step
    q_pos = np.zeros(6, dtype=np.int64)  # position 0: RoPE is the identity
    b = attend.attend_method(st, qr, q_pos)
    # exact attention of the grid queries in base 2, by explicit loops
    kd, vd = ring.dequant_k(st), ring.dequant_v(st)
    want = np.zeros_like(b)
    for t in range(6):
        for h in range(2):
            s = [sum(qg[t, h, i] * kd[h, j, i] for i in range(16)) for j in range(48)]
            w = [2.0 ** (x - max(s)) for x in s]
            want[t, h] = sum(w[j] * vd[h, j] for j in range(48)) / sum(w)
    assert np.max(np.abs(b - want)) < 1e-13
    # and the factor's rounding moves exact natural-base attention by ~1e-7 at most
    assert np.max(np.abs(attend.attend_exact(st, qr, q_pos) - b)) < 1e-5


def test_quantize_q_pow2_closed_forms():
    q = np.zeros((5, 1, 4))
    q[0, 0, 0] = 448.0  # fits at e = 0
    q[1, 0, 1] = 449.0  # needs e = 1
    q[2, 0, 2] = -224.0  # 224 = 448 * 2**-1
    q[3, 0, 3] = 224.5  # just above: e = 0
    codes, e = attend.quantize_q_pow2(q)
    assert e[:, 0].tolist() == [0, 1, -1, 0, 0]
    assert codes[0, 0, 0] == 0x7E and codes[2, 0, 2] == 0xFE
    assert np.all(codes[4] == 0)


def test_method_and_emul_close_to_exact_on_tiny():
    st, chunks = tiny_session()
    q, _, _, pos = chunks[5]
    ex = attend.attend_exact(st, q.f64, pos)
    me = attend.attend_method(st, q.f64, pos)
    em = attend.attend_emul(st, q.f64, pos)
    # Q in FP8 perturbs each logit by about 2**-5 of |q||k|/sqrt(D); the FP8
    # probabilities add about 2**-5 per term.  Loose sanity bounds.
    assert np.max(np.abs(me - ex)) < 0.15
    assert np.max(np.abs(em - me)) < 0.15
    assert np.mean(np.abs(em - ex)) < 0.02


def test_round_bf16_closed_forms_and_torch():
    one = 1.0
    cases = {
        one + 2 ** -8: 1.0,  # tie between 1 and 1 + 2**-7: even -> 1
        one + 3 * 2 ** -8: one + 2 ** -6,  # tie: 1 + 2**-7 has an odd last bit -> up
        one + 2 ** -8 + 2 ** -30: one + 2 ** -7,  # above the tie (no double rounding)
        -(one + 2 ** -8): -1.0,
        0.0: 0.0,
    }
    for x, want in cases.items():
        assert round_bf16(np.array([x]))[0] == want, x
    rng = np.random.default_rng(8)
    x32 = (rng.standard_normal(100_000) * 10).astype(np.float32)
    ref = torch.tensor(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x32.astype(np.float64)), ref)


def test_vmax_tracks_largest_value_scale_since_reset():
    rng = np.random.default_rng(14)
    st = ring.RingState(20, 2, 8)
    big = rng.standard_normal((5, 2, 8)) * 100
    ring.write(st, rng.standard_normal((5, 2, 8)), big, np.arange(5))
    first = st.vmax.copy()
    assert np.allclose(first, st.scale_v[:, :5].max(axis=1))
    for c in range(6):  # overwrite the ring with small values: vmax stays an upper bound
        ring.write(st, rng.standard_normal((10, 2, 8)), rng.standard_normal((10, 2, 8)), np.arange(10))
    assert np.array_equal(st.vmax, first)
    assert np.all(st.vmax >= st.scale_v.max(axis=1))
    ring.reset(st)
    assert not st.vmax.any()


def test_sigma_v_shape_and_value():
    st, _ = tiny_session()
    sv = attend.sigma_v(st)
    vd = ring.dequant_v(st)
    assert sv.shape == (1, 64)
    assert np.allclose(sv[0], np.sqrt((vd[0] ** 2).mean(axis=0)))


def test_sigma_v_closed_form_on_partial_wrapped_ring():
    """A hand-built 8-slot ring holding 3 valid slots that wrap (head 2,
    n_valid 3: slots 7, 0, 1); every other slot holds huge values.  The codes
    and scales make each dequantized value an exact small number, so the
    per-(head, channel) RMS over the valid slots has a closed form: channel 0
    holds 1, 2, 2 (sqrt 3), channel 1 holds -2, 2, 0 (sqrt(8/3)), channel 2
    holds 0, 0, 0 (0), channel 3 holds 4, 4, 4 (4); head 1 is head 0 times 2.
    Averaging over all slots, over N instead of n_valid, or over the slots
    [0, n_valid) instead of the cyclic range gives other values."""
    st = ring.RingState(8, 2, 4, head=2, n_valid=3)
    one, two, four, mtwo, big = 0x38, 0x40, 0x48, 0xC0, 0x7E  # 1, 2, 4, -2, 448
    st.codes_v[:] = big
    st.scale_v[:] = 1000.0
    rows = {7: [one, mtwo, 0, four], 0: [two, two, 0, four], 1: [two, 0, 0, four]}
    for slot, codes in rows.items():
        st.codes_v[:, slot] = codes
        st.scale_v[0, slot] = 1.0
        st.scale_v[1, slot] = 2.0
    want = np.array([np.sqrt(3.0), np.sqrt(8.0 / 3.0), 0.0, 4.0])
    sv = attend.sigma_v(st)
    assert np.allclose(sv[0], want, rtol=0, atol=1e-15)
    assert np.allclose(sv[1], 2 * want, rtol=0, atol=1e-15)
    # the empty ring normalizes by 1
    assert np.array_equal(attend.sigma_v(ring.RingState(8, 2, 4)), np.ones((2, 4)))

def test_q_term_error_bounds():
    """Power-of-two e4m3 terms: one carries Q to half an ulp of 448 over its
    amax, two to about 2**-8 of it, three to about 2**-12; each term gains
    about 4 bits (e4m3 holds 3 mantissa bits plus the rounding bit)."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((300, 3, 128)) * rng.uniform(0.01, 50, (300, 3, 1))
    amax = np.max(np.abs(q), axis=-1, keepdims=True)
    one = attend.quantize_q_terms(q, 1)
    two = attend.quantize_q_terms(q, 2)
    three = attend.quantize_q_terms(q, 3)
    assert np.all(np.abs(one - q) <= amax * 16 / 224)  # half ulp at 448 over a 224..448 amax
    assert np.all(np.abs(two - q) <= amax / 224)
    assert np.all(np.abs(three - q) <= amax / (224 * 16))
    assert np.max(np.abs(two - q) / amax) < np.max(np.abs(one - q) / amax) / 8
    assert np.max(np.abs(three - q) / amax) < np.max(np.abs(two - q) / amax) / 8
    # each element on its own: two terms within 2**-8 of its magnitude, three
    # within 2**-12 (all these elements are far above the subnormal range)
    big = np.abs(q) > amax * 2 ** -6
    assert np.all(np.abs(two - q)[big] <= np.abs(q)[big] * 2 ** -8)
    assert np.all(np.abs(three - q)[big] <= np.abs(q)[big] * 2 ** -12)


def test_two_term_p_closed_forms_and_bound():
    x = np.array([448.0, 1.0625, 1.1875, 0.0, 3.0 * 2 ** -10])
    two = attend.p_terms_value(x, 2)
    assert np.array_equal(two, x)  # each is hi + a residual that e4m3 holds exactly
    assert np.array_equal(attend.p_terms_value(x, 1), [448.0, 1.0, 1.25, 0.0, 2 ** -8])
    rng = np.random.default_rng(13)
    x = rng.uniform(0.05, 448, 100_000)
    assert np.all(np.abs(attend.p_terms_value(x, 2) - x) <= x * 2 ** -8)


def test_declared_numerics_meet_contract_on_outlier_cache():
    """Precise mode (three-term Q, two-term P) vs exact: normalized 2e-2 max / 2e-3 mean.

    A full 5,788-slot cache written in 757-token chunks with 2% outlier
    channels x8, ring head at slot 3,100; 2 heads and 96 queries keep it fast.
    """
    from workloads import ATTEND, OutlierSpec, Config
    cfg = Config("attend_2h", n_heads=2, head_dim=128, n_slots=5788, chunk=757, seed=1,
                 outliers=OutlierSpec(0.02, 8.0))
    st = ring.RingState(cfg.n_slots, cfg.n_heads, cfg.head_dim)
    s = Stream(cfg)
    p0 = 0
    for c in range(12):
        n = 757 if c < 11 else 561
        _, k, v = s.chunk(n)
        ring.write(st, k.f64, v.f64, positions(p0, n))
        p0 += n
    assert st.head == 3100 and st.n_valid == 5788
    q, _, _ = s.chunk(96)
    qpos = positions(8131, 96)
    ex = attend.attend_exact(st, q.f64, qpos)
    em = round_bf16(attend.attend_emul(st, q.f64, qpos))
    sig = np.maximum(1.0, attend.sigma_v(st))[None]
    e = np.abs(em - ex) / sig
    assert e.max() < 2e-2 and e.mean() < 2e-3


def test_emul_scales_exactly_with_power_of_two_value_scales():
    """Multiplying every value scale (and so vmax) by 2^k leaves each P s_v c
    unchanged (c divides by vmax) and the output scales by exactly 2^k: a
    value scale applied twice, or c missing from the normalization, breaks it."""
    st, chunks = tiny_session()
    q, _, _, pos = chunks[5]
    base = attend.attend_emul(st, q.f64, pos)
    for k in (-3, 5):
        s2 = st.copy()
        s2.scale_v = st.scale_v * 2.0 ** k
        s2.vmax = st.vmax * 2.0 ** k
        got = attend.attend_emul(s2, q.f64, pos)
        assert np.array_equal(got, base * 2.0 ** k), k


def test_emul_exact_when_scaled_probabilities_are_representable():
    """Identical keys make every probability 1; value scales at power-of-two
    fractions of vmax make each P s_v c = 112 * 2^-m an e4m3 value, so both
    terms are exact and the output is the mean of the dequantized values
    (vmax a power of two, so that c = 112 / vmax is exact in fp32)."""
    rng = np.random.default_rng(21)
    n, d = 24, 32
    st = ring.RingState(n, 1, d)
    k = np.repeat(rng.standard_normal((1, 1, d)), n, axis=0)
    v = rng.standard_normal((n, 1, d))
    ring.write(st, k, v, np.zeros(n, dtype=np.int64))
    big = 4.0
    m = rng.integers(0, 9, size=n)
    st.scale_v[0, :] = big * 2.0 ** (-m)
    st.vmax[0] = big
    q = rng.standard_normal((5, 1, d))
    mean_v = (e4m3.decode(st.codes_v[0]) * st.scale_v[0][:, None]).mean(axis=0)
    for terms in (1, 2):
        out = attend.attend_emul(st, q, np.arange(5), p_terms=terms)
        assert np.max(np.abs(out[:, 0, :] - mean_v[None])) <= 1e-14 * np.max(np.abs(mean_v)), terms
    # a value scale above vmax would push P s_v c past 448 * 2**-headroom but
    # stays inside e4m3 for a factor of 4: the same closed form holds
    st.scale_v[0, 0] = big * 4.0
    mean_v = (e4m3.decode(st.codes_v[0]) * st.scale_v[0][:, None]).mean(axis=0)
    out = attend.attend_emul(st, q, np.arange(5))
    assert np.max(np.abs(out[:, 0, :] - mean_v[None])) <= 1e-14 * np.max(np.abs(mean_v))
