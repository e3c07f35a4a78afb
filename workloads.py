"""Seeded synthetic inputs for the ring-KV hot path.

This module is shared by the tests, the benchmark and the CPU baseline.  It
holds none of the method's arithmetic (no RoPE, no quantization, no
attention): it only draws random tensors with the shapes, value
distributions and position schedules of the workloads described in
"Runway Characters: Serving a 57B Video Diffusion Transformer for Real-Time
Conversation" (§2 "The step budget"; Appendix G): 757 new tokens per write, a
5,788-slot cache, positions that reset every 42 steps.  The pages' real model
and clips are private, so seeded N(0,1) tensors with a fraction of channels
scaled up (outliers) stand in for them.

Every tensor is drawn as fp32 from ``numpy.random.default_rng(seed)`` in a
fixed order and rounded to bf16 with round-to-nearest-even.  The bf16 values
are returned twice: as raw uint16 bit patterns (what the device path
consumes) and as float64 arrays holding exactly the same values (what the
oracle consumes).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f64",
    "Bf16",
    "OutlierSpec",
    "draw_tokens",
    "TINY",
    "ATTEND",
    "WRITE_ROTATE",
    "PER_CHUNK",
    "STRESS",
    "PAGES_LAYOUT",
    "Config",
    "frame_positions",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly."""
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


@dataclass
class Bf16:
    """One bf16 tensor: raw bits for the device, exact float64 for the oracle."""

    bits: np.ndarray  # uint16
    f64: np.ndarray  # float64, same values

    @property
    def shape(self):
        return self.bits.shape


def _bf16(x: np.ndarray) -> Bf16:
    bits = f32_to_bf16_bits(x)
    return Bf16(bits=bits, f64=bf16_bits_to_f64(bits))


@dataclass(frozen=True)
class OutlierSpec:
    """A fraction of the H*D channels is multiplied by ``factor``."""

    frac: float = 0.0
    factor: float = 1.0


def outlier_mask(rng: np.random.Generator, h: int, d: int, spec: OutlierSpec) -> np.ndarray:
    """Per-channel multipliers [h, d]; a seeded subset of channels gets ``factor``."""
    mult = np.ones(h * d, dtype=np.float32)
    n_out = int(round(spec.frac * h * d))
    if n_out > 0 and spec.factor != 1.0:
        idx = rng.choice(h * d, size=n_out, replace=False)
        mult[idx] = np.float32(spec.factor)
    return mult.reshape(h, d)


def draw_tokens(rng: np.random.Generator, n: int, h: int, d: int, mult: np.ndarray) -> Bf16:
    """n tokens of [h, d] N(0,1) fp32 values times the channel multipliers, as bf16."""
    x = rng.standard_normal((n, h, d), dtype=np.float32) * mult[None, :, :]
    return _bf16(x)


@dataclass
class Config:
    """One named workload: sizes, seed, outlier recipe."""

    name: str
    n_heads: int
    head_dim: int
    n_slots: int
    chunk: int
    seed: int
    outliers: OutlierSpec = field(default_factory=OutlierSpec)
    n_layers: int = 1
    rope_base: float = 10000.0
    n_global: int = 0          # global (sink) slots beside the ring
    bands: tuple = None        # 3-D RoPE pairs per band (t, y, x); None: 1-D positions


# Tiny: 1 head, head_dim 64, 64 slots, chunks of 16, 6 writes, reset d=-80.
TINY = Config("tiny", n_heads=1, head_dim=64, n_slots=64, chunk=16, seed=0)

# One attention call at one GPU's head share: 12 heads x 128, 757 queries vs a
# full 5,788-slot cache whose ring head sits at slot 3,100; 2% outliers x8.
ATTEND = Config("attend_757x5788_h12", n_heads=12, head_dim=128, n_slots=5788, chunk=757,
                seed=1, outliers=OutlierSpec(0.02, 8.0))

# Write/rotate path: 42 writes of 757 tokens, then a reset by -42*757 positions.
WRITE_ROTATE = Config("write_rotate_757_h12", n_heads=12, head_dim=128, n_slots=5788, chunk=757,
                      seed=2, outliers=OutlierSpec(0.02, 8.0))

# Per-chunk sequence: 60 layer caches, 4 passes, reset at chunk 42; no outliers.
PER_CHUNK = Config("per_chunk_60x4", n_heads=12, head_dim=128, n_slots=5788, chunk=757,
                   seed=3, n_layers=60)

# The pages' cache layout at one GPU's head share: 1,246 global slots written
# once per session plus a ring of six 757-token latents (4,542 slots), 5,788
# read by every call; 3-D RoPE with the head's 64 pairs in temporal / height /
# width bands of 22 / 21 / 21 (synthetic: the pages give no band layout);
# 2% outlier channels x8.
PAGES_LAYOUT = Config("pages_g1246_r4542_h12", n_heads=12, head_dim=128, n_slots=4542, chunk=757, seed=5,
                      outliers=OutlierSpec(0.02, 8.0), n_global=1246, bands=(22, 21, 21))

# Stress: 48 heads, 11,576 slots, 1% outliers x16.
STRESS = Config("stress_h48_11576", n_heads=48, head_dim=128, n_slots=11576, chunk=757,
                seed=4, outliers=OutlierSpec(0.01, 16.0))


class Stream:
    """Deterministic token stream for one config.

    Draw order: outlier masks for Q, K, V (independent), then per chunk Q, K, V.
    """

    def __init__(self, cfg: Config, seed: int | None = None):
        self.cfg = cfg
        self.rng = np.random.default_rng(cfg.seed if seed is None else seed)
        h, d = cfg.n_heads, cfg.head_dim
        self.mq = outlier_mask(self.rng, h, d, cfg.outliers)
        self.mk = outlier_mask(self.rng, h, d, cfg.outliers)
        self.mv = outlier_mask(self.rng, h, d, cfg.outliers)

    def chunk(self, n: int | None = None):
        """Next (q, k, v) chunk of ``n`` tokens (default: the config's chunk)."""
        c = self.cfg
        n = c.chunk if n is None else n
        q = draw_tokens(self.rng, n, c.n_heads, c.head_dim, self.mq)
        k = draw_tokens(self.rng, n, c.n_heads, c.head_dim, self.mk)
        v = draw_tokens(self.rng, n, c.n_heads, c.head_dim, self.mv)
        return q, k, v


def positions(start: int, n: int) -> np.ndarray:
    """Consecutive int32 token positions start .. start+n-1."""
    return np.arange(start, start + n, dtype=np.int32)


def frame_positions(t: int, n: int, width: int, first: int = 0) -> np.ndarray:
    """3-D positions [n, 3] int32 of tokens first .. first+n-1 of one frame at
    temporal index t, laid row-major on a grid `width` tokens wide:
    (t, i // width, i % width)."""
    i = np.arange(first, first + n)
    return np.stack([np.full(n, t), i // width, i % width], axis=1).astype(np.int32)
