"""CPU oracle for the write-time FP8 ring KV cache (test infrastructure).

This package is test infrastructure, not part of the product.  Only the tests
under ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the device path (no
kernels, headers, tables or helpers); both sides only share the seeded input
generators in ``workloads.py``.

It is a plain, slow NumPy implementation in float64 of what the hot path
computes, written from the pages of "Runway Characters: Serving a 57B Video
Diffusion Transformer for Real-Time Conversation" (arXiv:2611.05642):

* ``e4m3``   -- OCP float8 e4m3fn encode (round to nearest even, saturate at
  +-448) and decode.  The pages store K and V "in float8_e4m3" (§4.3).
* ``rope``   -- rotary position embedding on interleaved pairs, and the pure
  per-pair rotation used by the reset (§4.2, Appendix G).
* ``ring``   -- the ring cache state and its two mutating operations: the write
  with RoPE and per-(token, head) FP8 quantization fused in (§4.1, §4.3, §4.4),
  and the delta rotation of every valid cached key at a position reset
  (§4.2, Appendix G).
* ``norm`` -- RMS normalization of query and key rows before RoPE (the fused
  pre-attention norm, §4.4).
* ``attend`` -- attention of new queries over every valid slot, in three
  precisions: exact (no query quantization), method (queries quantized per
  call, §4.3), and emul (the device kernel's declared numerics).

Pins: every function is checked in ``tests/test_oracle_*.py`` and
``tests/test_codec.py`` against something other than itself (torch's CPU
float8 cast, closed forms, brute-force loops, torch's float64 attention, the
rotation identity).  ``attend.attend_emul`` (the device kernel's declared
numerics, not a rule of the paper) is pinned by exact facts: its output
scales by exactly 2^k when every value scale does; with every scaled
probability an e4m3 value (one valid slot, or identical keys with value
scales at power-of-two fractions of vmax) it equals the closed form; its
two-term probability split has closed forms and an error bound; and its
e4m3 rounding is the codec pinned against torch's cast.
"""

from . import e4m3, rope, ring, attend, bf16, norm  # noqa: F401
