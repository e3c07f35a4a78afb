"""Pins for the oracle's e4m3fn codec and its per-row quantizer (CPU only).

The format is the OCP 8-bit e4m3fn encoding the pages store K and V in
(Runway Characters paper, §4.3 "FP8 at write").  References used here are
not the oracle itself: torch's CPU float8_e4m3fn conversion (a library
routine, which rounds to nearest even but does not saturate, so saturation
is compared after an explicit clamp) and closed-form code values from the
OCP specification, listed in tests/golden/e4m3_closed_forms.txt.
"""
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_closed_forms.txt")


def torch_encode(x):
    t = torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def finite_values():
    tab = e4m3.decode_table()
    pos = tab[:0x7F]
    return pos[np.isfinite(pos)]


def test_decode_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    assert np.isnan(ours).sum() == 2  # 0x7F and 0xFF only
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin], ours[fin])


def test_closed_forms_from_spec():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                val, code, on_grid = line.split()
                rows.append((float(val), int(code, 16), on_grid == "1"))
    assert len(rows) >= 10
    for val, code, on_grid in rows:
        assert int(e4m3.encode(np.array([val]))[0]) == code, (val, hex(code))
        if on_grid:
            assert e4m3.decode(np.array([code], dtype=np.uint8))[0] == val


def test_midpoints_round_to_nearest_even():
    v = finite_values()
    mids = (v[:-1] + v[1:]) / 2
    for x in (mids, -mids):
        assert np.array_equal(e4m3.encode(x), torch_encode(x))
    # Independent of torch: a midpoint goes to the neighbour with an even mantissa.
    enc = e4m3.encode(mids)
    assert np.all((enc & 1) == 0)


def test_random_values_match_torch():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.uniform(-448, 448, 200_000),
        rng.standard_normal(100_000),
        rng.uniform(-2 ** -6, 2 ** -6, 100_000),  # subnormal range
        rng.standard_normal(50_000) * 1e-4,
    ])
    assert np.array_equal(e4m3.encode(x), torch_encode(x))


def test_saturation():
    big = np.array([448.0, 449.0, 463.99, 464.0, 465.0, 480.0, 1e6, 1e30])
    for x in (big, -big):
        ours = e4m3.encode(x)
        ref = torch_encode(np.clip(x, -448, 448))
        assert np.array_equal(ours, ref)
        assert np.all((ours & 0x7F) == 0x7E)


def test_roundtrip_error_is_half_ulp():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-448, 448, 100_000), rng.standard_normal(100_000) * 0.01])
    c = e4m3.encode(x)
    err = np.abs(e4m3.decode(c) - x)
    assert np.all(err <= e4m3.ulp_at(c) / 2 * (1 + 1e-12))


def test_ulp_at_closed_forms():
    c = np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7E, 0xFE], dtype=np.uint8)
    expect = np.array([2 ** -9, 2 ** -9, 2 ** -9, 2 ** -9, 2 ** -3, 32.0, 32.0])
    assert np.array_equal(e4m3.ulp_at(c), expect)


def test_quantize_rows_amax_maps_to_448_and_bound_holds():
    rng = np.random.default_rng(11)
    y = rng.standard_normal((500, 4, 64)) * rng.uniform(0.01, 100, (500, 4, 1))
    codes, s = e4m3.quantize_rows(y)
    assert s.dtype == np.float64
    assert np.array_equal(s, s.astype(np.float32).astype(np.float64))  # fp32 values
    # the amax element of every row is the largest finite code
    idx = np.argmax(np.abs(y), axis=-1)
    top = np.take_along_axis(codes, idx[..., None], axis=-1)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)
    # per element: |code * s - y| <= s * ulp(code) / 2 (plus fp32 scale rounding)
    deq = e4m3.decode(codes) * s[..., None]
    bound = s[..., None] * e4m3.ulp_at(codes) / 2 + np.abs(y) * 2 ** -22
    assert np.all(np.abs(deq - y) <= bound)


def test_quantize_rows_zero_row():
    y = np.zeros((3, 2, 8))
    y[1, 1, 3] = -2.5
    codes, s = e4m3.quantize_rows(y)
    assert s[0, 0] == 0 and np.all(codes[0] == 0) and np.all(codes[1, 0] == 0)
    assert codes[1, 1, 3] == 0xFE and s[1, 1] == np.float32(2.5 / 448)


def test_encode_rejects_nonfinite():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan]))
