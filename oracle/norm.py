"""RMS normalization of query and key rows in float64 (test infrastructure).

Runway Characters paper, §4.4 "Fused pre-attention" and Appendix G: each
block RMS-normalizes Q and K of the new tokens, then applies RoPE, then
quantizes and writes K and V; values are not normalized.

The pages fix neither the weight shape nor epsilon.  Readings taken here:
each (token, head) row of head_dim elements is normalized on its own,
y_d = x_d * w_d / sqrt(mean over d of x_d^2 + eps), with one learned weight
vector of head_dim entries shared by all heads and a caller-given eps.  The
device computes it in fp32 from bf16 inputs, with no rounding between the
norm and RoPE; here every step is float64 on the exact bf16 values.
"""
from __future__ import annotations

import numpy as np


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x: [..., D] float64; w: [D]; returns x * w / sqrt(mean(x^2) + eps) per row."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)
