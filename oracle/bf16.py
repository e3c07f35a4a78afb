"""Rounding float64 results to bf16 (test infrastructure).

The attention output is bf16.  A value is rounded once, directly from float64
to the bf16 grid (8 significant bits), with ties to even -- not through an
intermediate float32, which would round twice.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest-even rounding of float64 values to bf16, returned as float64.

    Normal bf16 range only (|x| >= 2**-126 or 0); overflow is not handled
    because the attention outputs are convex combinations of cached values.
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)  # x = f * 2**e, |f| in [0.5, 1)
    # 8 significant bits: scale f to [128, 256) and round to an integer.
    return np.ldexp(np.rint(f * 256.0), e - 8)
