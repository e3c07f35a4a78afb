"""OCP float8 e4m3fn codec in float64 (test infrastructure).

The pages store the cache "in float8_e4m3" (Runway Characters paper, §4.3
"FP8 at write"), clamp rotated keys "to the FP8 range" and let values beyond
the scale saturate (§4.3 scale paragraph; Appendix G).  The format is the OCP
8-bit e4m3fn encoding (the ``fn`` variant: no infinities, one NaN pattern per
sign, largest finite value 448):

* bit 7 sign, bits 6..3 biased exponent (bias 7), bits 2..0 mantissa;
* exponent field 0: subnormal, value = m * 2**-9 (m = 0..7);
* exponent field 1..15: value = 2**(e-7) * (1 + m/8), except 0x7F / 0xFF = NaN;
* largest finite 0x7E = 2**8 * 1.75 = 448, smallest normal 0x08 = 2**-6.

Encoding rounds to nearest with ties to even and saturates to +-448 (the
pages' "saturate" / "clamped to the FP8 range").  NaN is never produced.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
MIN_NORMAL = 2.0 ** -6
SUBNORMAL_STEP = 2.0 ** -9


def decode_table() -> np.ndarray:
    """The 256 code values as float64 (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * m * SUBNORMAL_STEP
        else:
            out[code] = sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)
    return out


_TABLE = decode_table()


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode uint8 codes to float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x: np.ndarray) -> np.ndarray:
    """Encode float64 values to e4m3fn codes: nearest-even, saturating at +-448.

    Inputs must be finite.  Negative values that round to zero keep the sign
    bit (0x80), as IEEE conversions do.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3 encode: non-finite input")
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.int64)

    # Subnormal range |x| < 2**-6: mantissa counts steps of 2**-9; a result of
    # 8 steps is the smallest normal, whose code is also 8.
    sub = a < MIN_NORMAL
    code[sub] = np.rint(a[sub] / SUBNORMAL_STEP).astype(np.int64)

    # Normal range: a = f * 2**e with f in [0.5, 1) (exact), i.e.
    # a = 2**(e-1) * (1 + t) with t = 2f - 1 in [0, 1); mantissa = round(8 t).
    nrm = ~sub
    f, e = np.frexp(a[nrm])
    mant = np.rint(16.0 * f - 8.0).astype(np.int64)  # exact product, RNE
    unbiased = e.astype(np.int64) - 1
    carry = mant == 8
    mant[carry] = 0
    unbiased[carry] += 1
    biased = unbiased + 7
    c = (biased << 3) | mant
    c = np.minimum(c, 0x7E)  # saturate: 448 is the largest finite code
    code[nrm] = c
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def ulp_at(code: np.ndarray) -> np.ndarray:
    """Spacing of the e4m3 grid at the magnitude of each code.

    For a code with exponent field e >= 1 the step is 2**(e-7-3); for
    subnormals (and zero) it is 2**-9.
    """
    c = np.asarray(code, dtype=np.uint8) & 0x7F
    e = (c >> 3).astype(np.int64)
    step = np.where(e == 0, SUBNORMAL_STEP, 2.0 ** (np.maximum(e, 1) - 10))
    return step


def quantize_rows(y: np.ndarray, margin: float = 1.0):
    """Per-row scale and codes: s = fp32(margin * amax / 448), code = e4m3(y / s).

    ``y`` has the quantized vector on its last axis (one (token, head) row).
    This is the per-(token, head) amax rule of the hot path; a row of zeros
    gets scale 0 and codes 0.  Returns (codes uint8, scale float64 holding
    fp32 values).
    """
    y = np.asarray(y, dtype=np.float64)
    amax = np.max(np.abs(y), axis=-1)
    s = (margin * amax / E4M3_MAX).astype(np.float32).astype(np.float64)
    safe = np.where(s > 0, s, 1.0)
    codes = encode(y / safe[..., None])
    codes = np.where((s > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, s
