"""Attention of new queries over every valid cache slot, float64 (test infrastructure).

Runway Characters paper: §2 "The step budget" and Appendix G (each call
attends over all 5,788 slots of its cache, after writing the new chunk);
§4.2 (queries get RoPE at their own positions and cached keys are used as
they are); §4.3 "FP8 at write" (only the queries are quantized per call; the
FP8 attention takes per-head descales).

Readings where the pages are silent: softmax scale 1/sqrt(D); non-causal;
keys are every valid slot, including the chunk just written; an empty cache
gives zeros; the output is rounded once to bf16 (nearest even).

Three precisions, all on the dequantized cache:

* ``attend_exact``  -- Q unquantized, probabilities exact.
* ``attend_method`` -- Q quantized as the device kernel does, probabilities exact.
* ``attend_emul``   -- ``attend_method`` plus the kernel's FP8 rounding of the
  scaled probabilities that enter the P.V product.

The device kernel's declared numerics, which ``attend_method`` and
``attend_emul`` follow:

* Softmax scale: the kernel multiplies each RoPE'd query by
  c_s = log2(e) / sqrt(D), rounded once to float32, before quantizing it, so
  the logits come out in log2 units and P = 2**(S - m).  (The pages fix FP8
  attention but not where the scale enters; applied to Q it costs no work
  per logit.)
* Q quantization: of the scaled query, per (token, head), a power-of-two
  scale 2**e with e the smallest integer such that amax(q) <= 448 * 2**e;
  codes = e4m3(q / 2**e).
  (A power of two is applied exactly inside the FP8 matrix instruction.)
  With three terms (the default, "precise" mode) the residual
  r = q - decode(codes) * 2**e is quantized the same way, and its residual
  again, and the kernel multiplies K by all three; Q is then known to about
  2**-12 relative.  (Two terms, about 2**-8, are not enough: where a query's
  outlier channels meet a key's, the score error moved single outputs by up
  to 2.9e-2 of the value scale.)
* P.V in FP8: with P = 2**(S - m) (m the row maximum), the kernel feeds
  x = P * s_v[j] * c with c = 448 * 2**-headroom / vmax_h, vmax_h the largest
  value scale written to the head since the last reset (an upper bound of
  every cached s_v), as hi = e4m3(x) and, with two terms, as
  lo = e4m3(16 (x - hi)) / 16; it multiplies them by the V codes and divides
  by c * sum_j P.  The kernel keeps a running row maximum that it raises only
  when a tile exceeds it by more than 6 in log2 units (and then by a whole
  number of log2 units, at least up to the tile's maximum), so its P may
  reach 64: headroom 6 keeps x <= 448.  ``attend_emul`` uses the final row maximum;
  the kernel's running maximum changes which way some codes round, which the
  tolerance covers.
* The single-term ("fast") mode uses one term for Q and one for P.
* Static scales (the pages' per-(layer, head) mode, once calibrated: every
  valid slot of a head carries the head's key scale s_k and value scale
  s_v): the kernel multiplies the scaled query by s_k before quantizing it,
  so the products with the key codes come out in log2 units, and feeds
  x = 7 P (7 = 448 * 2**-6, the headroom) in place of P s_v c; the output is
  s_v times (x . V codes) / sum x.  (A head whose static scales are 0 keeps
  the per-token rule.)
"""
from __future__ import annotations

import math

import numpy as np

from . import e4m3
from .ring import RingState, dequant_k, dequant_v, rope_keys, valid_slots
from .rope import rope


def quantize_q_pow2(q: np.ndarray):
    """Kernel Q rule: per-row power-of-two scale. Returns (codes, exponent e)."""
    q = np.asarray(q, dtype=np.float64)
    amax = np.max(np.abs(q), axis=-1)
    e = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    # smallest integer e with amax <= 448 * 2**e: start from the binary
    # exponent of amax / 448, then settle the boundary with exact ldexp tests.
    _, ex = np.frexp(amax[nz] / e4m3.E4M3_MAX)
    ex = ex.astype(np.int64)
    a = amax[nz]
    ex = ex - (a <= np.ldexp(e4m3.E4M3_MAX, ex - 1))
    ex = ex + (a > np.ldexp(e4m3.E4M3_MAX, ex))
    e[nz] = ex
    codes = e4m3.encode(np.ldexp(q, -e[..., None]))
    return codes, e


def _prepare(st: RingState, q: np.ndarray, q_pos: np.ndarray):
    q = np.asarray(q, dtype=np.float64)
    if q.ndim != 3 or q.shape[1] != st.n_heads or q.shape[2] != st.head_dim:
        raise ValueError("attend: q must be [n_q, H, D]")
    slots = valid_slots(st)
    qr = rope_keys(st, q, q_pos)  # [n_q, H, D], the state's RoPE (1-D or 3-D)
    return qr, slots


def softmax_scale_log2(d: int) -> float:
    """The kernel's query factor c_s = log2(e) / sqrt(D), rounded once to float32."""
    return float(np.float32(math.log2(math.e) / math.sqrt(d)))


def _softmax2_av(sh: np.ndarray, vh: np.ndarray) -> np.ndarray:
    """softmax in base 2 of logits already in log2 units, times v; float64."""
    sh = sh - sh.max(axis=1, keepdims=True)
    p = np.exp2(sh)
    return (p @ vh) / p.sum(axis=1, keepdims=True)


def _softmax_av(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray) -> np.ndarray:
    """Exact softmax(q k^T / sqrt(D)) v for one head, float64."""
    d = qh.shape[-1]
    s = qh @ kh.T / math.sqrt(d)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ vh) / p.sum(axis=1, keepdims=True)


def attend_exact(st: RingState, q: np.ndarray, q_pos: np.ndarray) -> np.ndarray:
    """A-exact: fp64 attention with unquantized (RoPE'd) Q on the dequantized cache."""
    qr, slots = _prepare(st, q, q_pos)
    out = np.zeros(qr.shape, dtype=np.float64)
    if slots.size == 0:
        return out
    kd = dequant_k(st)[:, slots, :]
    vd = dequant_v(st)[:, slots, :]
    for h in range(st.n_heads):
        out[:, h, :] = _softmax_av(qr[:, h, :], kd[h], vd[h])
    return out


def quantize_q_terms(qr: np.ndarray, terms: int):
    """Q as a sum of ``terms`` power-of-two-scaled e4m3 terms; returns float64 value."""
    total = np.zeros_like(qr)
    resid = qr
    for _ in range(terms):
        codes, e = quantize_q_pow2(resid)
        part = np.ldexp(e4m3.decode(codes), e[..., None])
        total = total + part
        resid = qr - total
    return total


def p_terms_value(x: np.ndarray, terms: int) -> np.ndarray:
    """x >= 0 as hi = e4m3(x) (+ lo = e4m3(16 (x - hi)) / 16 with two terms)."""
    hi = e4m3.decode(e4m3.encode(x))
    if terms == 1:
        return hi
    lo = e4m3.decode(e4m3.encode((x - hi) * 16.0)) / 16.0
    return hi + lo


def attend_method(st: RingState, q: np.ndarray, q_pos: np.ndarray, q_terms: int = 3) -> np.ndarray:
    """A-method: Q quantized with the kernel's rule, exact probabilities."""
    qr, slots = _prepare(st, q, q_pos)
    out = np.zeros(qr.shape, dtype=np.float64)
    if slots.size == 0:
        return out
    qd = quantize_q_terms(qr * softmax_scale_log2(st.head_dim), q_terms)
    kd = dequant_k(st)[:, slots, :]
    vd = dequant_v(st)[:, slots, :]
    for h in range(st.n_heads):
        out[:, h, :] = _softmax2_av(qd[:, h, :] @ kd[h].T, vd[h])
    return out


def attend_emul(st: RingState, q: np.ndarray, q_pos: np.ndarray, q_terms: int = 3,
                p_terms: int = 2, headroom: int = 6) -> np.ndarray:
    """A-emul: A-method plus the FP8 rounding of P' = P * s_v[j] * c (see module doc)."""
    qr, slots = _prepare(st, q, q_pos)
    out = np.zeros(qr.shape, dtype=np.float64)
    if slots.size == 0:
        return out
    cs = softmax_scale_log2(st.head_dim)
    qd = quantize_q_terms(qr * cs, q_terms)
    kd = dequant_k(st)[:, slots, :]
    v8 = e4m3.decode(st.codes_v[:, slots, :])  # codes as values
    sv = st.scale_v[:, slots]  # [H, n_valid]
    for h in range(st.n_heads):
        if static_head(st, h):
            sk_h, sv_h = st.static_k[h], st.static_v[h]
            qh = quantize_q_terms(qr[:, h, :] * cs * sk_h, q_terms)
            s = qh @ e4m3.decode(st.codes_k[h, slots, :]).T  # log2 units
            p = np.exp2(s - s.max(axis=1, keepdims=True))
            xq = p_terms_value(7.0 * p, p_terms)  # 7 = 448 * 2**-6
            out[:, h, :] = sv_h * (xq @ v8[h]) / (7.0 * p.sum(axis=1, keepdims=True))
            continue
        s = qd[:, h, :] @ kd[h].T  # log2 units
        p = np.exp2(s - s.max(axis=1, keepdims=True))  # <= 1, row max exactly 1
        l = p.sum(axis=1, keepdims=True)
        smax = st.vmax[h]
        c = (e4m3.E4M3_MAX * 2.0 ** (-headroom) / smax) if smax > 0 else 1.0
        c = float(np.float32(c))
        pq = p_terms_value(p * sv[h][None, :] * c, p_terms)
        out[:, h, :] = (pq @ v8[h]) / (c * l)
    return out


def static_head(st: RingState, h: int) -> bool:
    """True when head h is in the pages' static-scale mode with nonzero key
    and value scales, so every valid slot carries the head's scales (the
    calibration requantizes the valid cache; later writes and rotations use
    them)."""
    return st.static_k is not None and st.static_k[h] > 0 and st.static_v[h] > 0


def sigma_v(st: RingState) -> np.ndarray:
    """RMS of the dequantized V over valid slots, per (head, channel): [H, D].

    Used to normalize attention errors: an output channel whose values are
    large (outlier channels) is compared on its own scale.
    """
    slots = valid_slots(st)
    if slots.size == 0:
        return np.ones((st.n_heads, st.head_dim))
    vd = dequant_v(st)[:, slots, :]
    return np.sqrt(np.mean(vd * vd, axis=1))
