"""Ring KV cache state, write and delta rotation in float64 (test infrastructure).

Runway Characters paper:

* §4.1 "A ring cache with a device-side write position": each new frame goes
  to a circular slot; a ring is correct only if each cached entry keeps the
  position it was written with.
* §4.2 and Appendix G "Cache update and position reset": RoPE is applied to
  each new key once, before the write; at a reset every cached key is
  dequantized, rotated by the position change in fp32, and requantized; the
  values are not touched.
* §4.3 "FP8 at write": K and V are stored in FP8 and only the new tokens are
  quantized.

Readings taken where the pages are silent or differ from the hot path's
statement:

* scale rule: per-(token, head) s = fp32(margin * amax / 448), margin 1.0,
  amax over the RoPE'd K vector (float64, no intermediate rounding) and over
  the raw V vector;
* the reset recomputes the scale from the rotated key's amax, so the scale
  rule holds for every cached key after a reset (keeping the old scale with a
  margin of 1.0 would saturate about half of the keys);
* the valid set is the cyclic slot range [head - n_valid, head); only valid
  slots are rotated and their positions shifted;
* the pages' own scale mode (§4.3, Appendix G) is available after
  ``calibrate_static``: per-head scales from the amax of the dequantized
  cache over the valid slots times a margin, saturating writes with them,
  and reset rotations that requantize every valid key of the head with the
  head's scale and clamp (keys written after the calibration already carry
  it; older keys, quantized with their own per-token scale, move to it --
  the head's scale covers any rotation of them, since a rotated pair's
  component is at most the pair's norm, at most sqrt(2) times the head's
  amax, below the margin of 1.5 the pages use); a head whose amax was 0 at
  calibration keeps per-(token, head) scales (a zero scale would store zero
  codes for every later write); ``reset`` returns to per-(token, head)
  scales.

State layout (canonical, independent of any device layout): codes [H][N][D]
uint8, scales [H][N] float64 holding fp32 values, slot_pos [N] int64, and
vmax [H], the largest value scale written to each head since the last reset
(bookkeeping the device kernels keep so the attention knows an upper bound of
every cached value scale without a pass over the cache).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import e4m3
from .rope import delta_angles, delta_angles3d, rope, rope3d, rotate_pairs


@dataclass
class RingState:
    n_slots: int
    n_heads: int
    head_dim: int
    rope_base: float = 10000.0
    margin: float = 1.0
    head: int = 0
    n_valid: int = 0
    slot_pos: np.ndarray = field(default=None)
    codes_k: np.ndarray = field(default=None)
    codes_v: np.ndarray = field(default=None)
    scale_k: np.ndarray = field(default=None)
    scale_v: np.ndarray = field(default=None)
    vmax: np.ndarray = field(default=None)  # per head: largest s_v written since the reset
    # static per-(layer, head) scales of the pages' own scale mode, [H] each
    # (float64 holding fp32 values); None: per-(token, head) amax scales
    static_k: np.ndarray = field(default=None)
    static_v: np.ndarray = field(default=None)
    # global (sink) slots after the ring: canonical slots n_slots ..
    # n_slots + n_global - 1, written at explicit indices, never rotated;
    # g_valid = 1 + the highest global index written since the reset
    n_global: int = 0
    g_valid: int = 0
    # 3-D RoPE: (n_t, n_y, n_x) pairs per band (rope.band_table); None: 1-D
    # positions.  With bands, slot_pos holds t and slot_yx (y, x).
    bands: tuple = None
    slot_yx: np.ndarray = field(default=None)

    def __post_init__(self):
        h, d = self.n_heads, self.head_dim
        n = self.n_slots + self.n_global
        if self.slot_pos is None:
            self.slot_pos = np.zeros(n, dtype=np.int64)
        if self.slot_yx is None:
            self.slot_yx = np.zeros((n, 2), dtype=np.int64)
        if self.codes_k is None:
            self.codes_k = np.zeros((h, n, d), dtype=np.uint8)
        if self.codes_v is None:
            self.codes_v = np.zeros((h, n, d), dtype=np.uint8)
        if self.scale_k is None:
            self.scale_k = np.zeros((h, n), dtype=np.float64)
        if self.scale_v is None:
            self.scale_v = np.zeros((h, n), dtype=np.float64)
        if self.vmax is None:
            self.vmax = np.zeros(h, dtype=np.float64)

    def copy(self) -> "RingState":
        return RingState(self.n_slots, self.n_heads, self.head_dim, self.rope_base, self.margin,
                         self.head, self.n_valid, self.slot_pos.copy(), self.codes_k.copy(),
                         self.codes_v.copy(), self.scale_k.copy(), self.scale_v.copy(),
                         self.vmax.copy(),
                         None if self.static_k is None else self.static_k.copy(),
                         None if self.static_v is None else self.static_v.copy(),
                         self.n_global, self.g_valid, self.bands, self.slot_yx.copy())


def ring_valid_slots(st: RingState) -> np.ndarray:
    """Ring slots of the valid range, oldest first: (head - n_valid + k) mod N."""
    k = np.arange(st.n_valid, dtype=np.int64)
    return (st.head - st.n_valid + k) % st.n_slots


def valid_slots(st: RingState) -> np.ndarray:
    """Every slot the attention reads: the ring's valid range, oldest first,
    then the global slots written since the reset."""
    return np.concatenate([ring_valid_slots(st), st.n_slots + np.arange(st.g_valid, dtype=np.int64)])


def rope_keys(st: RingState, x: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """RoPE of [n, H, D] rows at the state's position kind: int [n] (1-D) or
    [n, 3] = (t, y, x) with the state's bands."""
    if st.bands is None:
        return rope(x, pos, st.rope_base)
    return rope3d(x, pos, st.bands, st.rope_base)


def _set_positions(st: RingState, slots: np.ndarray, pos: np.ndarray) -> None:
    pos = np.asarray(pos, dtype=np.int64)
    if st.bands is None:
        st.slot_pos[slots] = pos
    else:
        st.slot_pos[slots] = pos[:, 0]
        st.slot_yx[slots] = pos[:, 1:3]


def write_slots(st: RingState, n: int) -> np.ndarray:
    """Slots the next write of n tokens goes to: (head + i) mod N."""
    return (st.head + np.arange(n, dtype=np.int64)) % st.n_slots


def write(st: RingState, k: np.ndarray, v: np.ndarray, pos: np.ndarray) -> None:
    """Write n new tokens into the ring: RoPE on K at their positions, FP8
    quantize K and V.

    k, v: [n, H, D] float64 (bf16 values); pos: [n] integer positions (1-D)
    or [n, 3] (t, y, x) with 3-D RoPE.  Token i goes to slot (head + i) mod N
    and the slot remembers its position.  Then head <- (head + n) mod N and
    n_valid <- min(n_valid + n, N).
    """
    n = np.asarray(k).shape[0]
    if not (0 < n <= st.n_slots):
        raise ValueError("write: n must be in 1..n_slots")
    slots = write_slots(st, n)
    _store(st, slots, k, v, pos)
    st.head = int((st.head + n) % st.n_slots)
    st.n_valid = int(min(st.n_valid + n, st.n_slots))


def write_global(st: RingState, first: int, k: np.ndarray, v: np.ndarray, pos: np.ndarray) -> None:
    """Write n tokens into the global (sink) slots first .. first + n - 1 (the
    pages' global tokens, written once per session, never rotated): RoPE at
    their positions and FP8 quantization as in the ring write.  g_valid
    becomes max(g_valid, first + n)."""
    n = np.asarray(k).shape[0]
    if not (0 < n and 0 <= first and first + n <= st.n_global):
        raise ValueError("write_global: slots out of range")
    slots = st.n_slots + first + np.arange(n, dtype=np.int64)
    _store(st, slots, k, v, pos)
    st.g_valid = int(max(st.g_valid, first + n))


def _store(st: RingState, slots: np.ndarray, k: np.ndarray, v: np.ndarray, pos: np.ndarray) -> None:
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    n = k.shape[0]
    want_pos = (n,) if st.bands is None else (n, 3)
    if k.shape != (n, st.n_heads, st.head_dim) or v.shape != k.shape or pos.shape != want_pos:
        raise ValueError("write: shape mismatch")
    k_rot = rope_keys(st, k, pos)  # [n, H, D]
    if st.static_k is None:
        ck, sk = e4m3.quantize_rows(k_rot, st.margin)  # [n, H, D], [n, H]
        cv, sv = e4m3.quantize_rows(v, st.margin)
    else:
        ck, sk = quantize_static(k_rot, st.static_k, st.margin)
        cv, sv = quantize_static(v, st.static_v, st.margin)
    st.codes_k[:, slots, :] = np.transpose(ck, (1, 0, 2))
    st.codes_v[:, slots, :] = np.transpose(cv, (1, 0, 2))
    st.scale_k[:, slots] = sk.T
    st.scale_v[:, slots] = sv.T
    _set_positions(st, slots, pos)
    st.vmax = np.maximum(st.vmax, sv.max(axis=0))


def rotate(st: RingState, delta: int) -> None:
    """Delta rotation at a position reset, in place, on every valid ring slot.

    Each valid ring key (every head) is dequantized with its scale, each pair
    j is rotated by phi_j = delta * omega_j (with 3-D RoPE only the temporal
    pairs; the spatial ones keep their values), a new scale is taken from the
    rotated key's amax, and the key is requantized.  slot_pos (the temporal
    position) += delta.  V untouched; global slots untouched.
    """
    slots = ring_valid_slots(st)  # global slots never move
    if slots.size == 0:
        return
    if st.bands is None:
        c, s = delta_angles(st.head_dim, delta, st.rope_base)
    else:  # only the temporal band turns; spatial pairs keep their values
        c, s = delta_angles3d(st.head_dim, st.bands, delta, st.rope_base)
    x = e4m3.decode(st.codes_k[:, slots, :]) * st.scale_k[:, slots][..., None]
    y = rotate_pairs(x, c, s)
    ck, sk = e4m3.quantize_rows(y, st.margin)
    if st.static_k is not None:
        # the pages' own mode: requantize with the head's scale, values beyond
        # it saturate; heads calibrated at amax 0 stay per-(token, head)
        for h in np.flatnonzero(st.static_k > 0):
            sh = st.static_k[h]
            ck[h] = e4m3.encode(y[h] / sh)
            sk[h] = sh
    st.codes_k[:, slots, :] = ck
    st.scale_k[:, slots] = sk
    st.slot_pos[slots] = st.slot_pos[slots] + delta


def reset(st: RingState) -> None:
    """Session reset: empty ring and no global slots (head 0, no valid slots,
    positions 0, vmax 0), back to per-(token, head) scales until the next
    calibration."""
    st.head = 0
    st.n_valid = 0
    st.g_valid = 0
    st.slot_pos[:] = 0
    st.slot_yx[:] = 0
    st.vmax[:] = 0
    st.static_k = st.static_v = None


def quantize_static(y: np.ndarray, s_head: np.ndarray, margin: float):
    """Codes of [n, H, D] rows with one fixed scale per head: e4m3(y / s_h),
    saturating at +-448 (values beyond the scale clip).  A head whose static
    scale is 0 (amax 0 at calibration) keeps the per-(token, head) rule.
    Returns (codes, per-row scales [n, H])."""
    codes, s = e4m3.quantize_rows(y, margin)
    for h in np.flatnonzero(np.asarray(s_head) > 0):
        codes[:, h] = e4m3.encode(y[:, h] / s_head[h])
        s[:, h] = s_head[h]
    return codes, s


def calibrate_static(st: RingState, margin: float) -> None:
    """The pages' scale calibration (Appendix G; §4.3 "FP8 at write"): per
    head, s = fp32(margin * amax / 448) with amax the largest magnitude of the
    dequantized keys (values) over the valid slots; the valid cache is
    requantized with these scales, every later write quantizes with them and
    a reset rotation requantizes the head's keys with its key scale.  A scale
    of 0 (amax 0: no valid slot, or all zero) leaves that head's keys
    (values) on per-(token, head) scales."""
    slots = valid_slots(st)
    amk = np.zeros(st.n_heads)
    amv = np.zeros(st.n_heads)
    if slots.size:
        amk = np.max(np.abs(dequant_k(st)[:, slots, :]), axis=(1, 2))
        amv = np.max(np.abs(dequant_v(st)[:, slots, :]), axis=(1, 2))
    st.static_k = (margin * amk / e4m3.E4M3_MAX).astype(np.float32).astype(np.float64)
    st.static_v = (margin * amv / e4m3.E4M3_MAX).astype(np.float32).astype(np.float64)
    # The pages' cache is bf16 until the calibration and FP8 with the head's
    # scales from then on; this cache is FP8 from the first write, so the
    # calibration requantizes every valid key and value of a calibrated head
    # with the head's scale (one more e4m3 rounding of the per-token codes;
    # every element is at most amax = 448 s / margin, so only a margin below
    # 1 saturates, at +-448 as encode does).
    # Every valid slot then carries its head's scales, which is what lets the
    # attention apply them per head.
    for h in range(st.n_heads):
        for sh, codes, scales in ((st.static_k[h], st.codes_k, st.scale_k),
                                  (st.static_v[h], st.codes_v, st.scale_v)):
            if sh > 0 and slots.size:
                x = e4m3.decode(codes[h][slots]) * scales[h][slots][:, None]
                codes[h][slots] = e4m3.encode(x / sh)
                scales[h][slots] = sh
        if st.static_v[h] > 0:
            st.vmax[h] = st.static_v[h]  # every valid value scale is now the head's


def dequant_k(st: RingState) -> np.ndarray:
    """Dequantized keys [H][N][D] float64."""
    return e4m3.decode(st.codes_k) * st.scale_k[..., None]


def dequant_v(st: RingState) -> np.ndarray:
    """Dequantized values [H][N][D] float64."""
    return e4m3.decode(st.codes_v) * st.scale_v[..., None]
