"""Pins for the oracle's ring cache: bookkeeping, write values, delta rotation (CPU).

Runway Characters paper: §4.1 (ring slots; each slot keeps the position it
was written with; RoPE applied in physical slot order after a wrap is
invalid), §4.2 and Appendix G (delta rotation at a reset: dequantize, rotate,
requantize; values untouched; the stored key changes by one FP8 rounding),
§4.3 (FP8 at write, only new tokens quantized).

References: a hand-derived worked case (tests/golden/tiny_ring_slot_pos.txt),
a deque model of "the last N tokens" (brute force), the complex-number RoPE
of test_oracle_rope, and error bounds from the e4m3 grid.
"""
import collections
import os

import numpy as np
import pytest

from oracle import e4m3, ring, rope
from tests.test_oracle_rope import rope_complex
from workloads import TINY, Stream, positions

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_ring_slot_pos.txt")


def load_golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(t) for t in line.split()])
    return rows


def tiny_session():
    st = ring.RingState(TINY.n_slots, TINY.n_heads, TINY.head_dim)
    s = Stream(TINY)
    chunks = []
    for c in range(6):
        q, k, v = s.chunk()
        pos = positions(16 * c, 16)
        ring.write(st, k.f64, v.f64, pos)
        chunks.append((q, k, v, pos))
    return st, chunks


def test_tiny_worked_case_bookkeeping():
    (head, n_valid), after_writes, after_reset = load_golden()
    st, _ = tiny_session()
    assert (st.head, st.n_valid) == (head, n_valid)
    assert st.slot_pos.tolist() == after_writes
    ring.rotate(st, -80)
    assert st.slot_pos.tolist() == after_reset
    assert (st.head, st.n_valid) == (head, n_valid)


def test_ring_matches_deque_of_last_n_tokens():
    """Brute force: the valid slots, oldest first, hold the last N tokens written."""
    rng = np.random.default_rng(5)
    n_slots, h, d = 37, 2, 8
    st = ring.RingState(n_slots, h, d)
    model = collections.deque(maxlen=n_slots)
    next_pos = 0
    for _ in range(25):
        n = int(rng.integers(1, n_slots + 1))
        k = rng.standard_normal((n, h, d))
        v = rng.standard_normal((n, h, d))
        pos = np.arange(next_pos, next_pos + n)
        next_pos += n
        ring.write(st, k, v, pos)
        for i in range(n):
            model.append((int(pos[i]), v[i]))
        slots = ring.valid_slots(st)
        assert len(slots) == len(model) == st.n_valid
        assert st.slot_pos[slots].tolist() == [p for p, _ in model]
        # values stored for each valid slot are the ones of the matching token
        vq = ring.dequant_v(st)[:, slots, :]
        for j, (_, vt) in enumerate(model):
            bound = st.scale_v[:, slots[j]][:, None] * 16 * (1 + 1e-12)  # half ulp at 448
            assert np.all(np.abs(vq[:, j, :] - vt) <= bound)


def test_write_values_within_half_ulp_of_rope():
    st, chunks = tiny_session()
    kd = ring.dequant_k(st)
    vd = ring.dequant_v(st)
    for c in (4, 5, 2, 3):  # the chunks still resident
        _, k, v, pos = chunks[c]
        slots = ring.write_slots(ring.RingState(64, 1, 64, head=(16 * c) % 64), 16)
        ref_k = rope_complex(k.f64, pos)  # [16, 1, 64]
        got_k = np.transpose(kd[:, slots, :], (1, 0, 2))
        ck = np.transpose(st.codes_k[:, slots, :], (1, 0, 2))
        sk = st.scale_k[:, slots].T[..., None]
        assert np.all(np.abs(got_k - ref_k) <= sk * e4m3.ulp_at(ck) / 2 + 1e-9 * np.abs(ref_k) + 1e-12)
        got_v = np.transpose(vd[:, slots, :], (1, 0, 2))
        cv = np.transpose(st.codes_v[:, slots, :], (1, 0, 2))
        sv = st.scale_v[:, slots].T[..., None]
        assert np.all(np.abs(got_v - v.f64) <= sv * e4m3.ulp_at(cv) / 2 * (1 + 1e-12))
        # scale rule: amax of the RoPE'd key / 448, stored as fp32
        amax = np.max(np.abs(ref_k), axis=-1)
        assert np.allclose(st.scale_k[:, slots].T, amax / 448, rtol=1e-6)


def test_rope_uses_written_positions_not_slot_order():
    """After a wrap, keys carry their written positions; slot-order RoPE differs (invalid)."""
    st, chunks = tiny_session()
    _, k4, _, pos4 = chunks[4]  # written to slots 0..15 at positions 64..79
    stored = np.transpose(ring.dequant_k(st)[:, 0:16, :], (1, 0, 2))
    right = rope.rope(k4.f64, pos4)
    wrong = rope.rope(k4.f64, np.arange(0, 16))  # physical slot index as position
    err_right = np.max(np.abs(stored - right))
    err_wrong = np.max(np.abs(stored - wrong))
    assert err_right <= np.max(np.abs(right)) * 16 / 448 * (1 + 1e-6)  # half ulp at the amax
    assert err_wrong > 10 * err_right


def test_rotation_invariant_and_bound():
    """rotate(q(RoPE(k, p)), d) ~= RoPE(k, p + d), within the FP8 steps (absolute bound)."""
    st, chunks = tiny_session()
    before_codes = st.codes_k.copy()
    before_scale = st.scale_k.copy()
    v_before = (st.codes_v.copy(), st.scale_v.copy())
    d = -80
    ring.rotate(st, d)
    assert np.array_equal(st.codes_v, v_before[0]) and np.array_equal(st.scale_v, v_before[1])
    kd = ring.dequant_k(st)
    for c in (2, 3, 4, 5):
        _, k, _, pos = chunks[c]
        slots = (16 * c + np.arange(16)) % 64
        ref = rope_complex(k.f64, pos + d)[:, 0, :]  # [16, 64]
        got = kd[0, slots, :]
        c0 = before_codes[0, slots, :]
        s0 = before_scale[0, slots][:, None]
        c1 = st.codes_k[0, slots, :]
        s1 = st.scale_k[0, slots][:, None]
        u0 = e4m3.ulp_at(c0)
        pair_u = np.sqrt(u0[:, 0::2] ** 2 + u0[:, 1::2] ** 2)
        pair_u = np.repeat(pair_u, 2, axis=1)
        bound = s0 * pair_u / 2 + s1 * e4m3.ulp_at(c1) / 2 + 1e-6 * np.abs(ref) + 1e-9
        assert np.all(np.abs(got - ref) <= bound)
        # new scale follows the rule on the rotated key
        assert np.all((np.max(c1 & 0x7F, axis=1)) == 0x7E)


def test_rotate_partial_fill_touches_only_valid_slots():
    rng = np.random.default_rng(9)
    st = ring.RingState(50, 2, 16)
    ring.write(st, rng.standard_normal((20, 2, 16)), rng.standard_normal((20, 2, 16)), np.arange(20))
    frozen = st.copy()
    ring.rotate(st, 7)
    assert st.slot_pos[:20].tolist() == list(range(7, 27))
    assert np.array_equal(st.slot_pos[20:], frozen.slot_pos[20:])
    assert np.array_equal(st.codes_k[:, 20:], frozen.codes_k[:, 20:])
    assert not np.array_equal(st.codes_k[:, :20], frozen.codes_k[:, :20])


def test_rotate_by_zero_is_identity_on_values():
    st, _ = tiny_session()
    before = ring.dequant_k(st).copy()
    ring.rotate(st, 0)
    assert np.array_equal(ring.dequant_k(st), before)


def test_reset_and_argument_checks():
    st, _ = tiny_session()
    ring.reset(st)
    assert st.head == 0 and st.n_valid == 0 and not st.slot_pos.any()
    with pytest.raises(ValueError):
        ring.write(st, np.zeros((65, 1, 64)), np.zeros((65, 1, 64)), np.arange(65))
    with pytest.raises(ValueError):
        ring.write(st, np.zeros((4, 1, 64)), np.zeros((4, 1, 64)), np.arange(3))
