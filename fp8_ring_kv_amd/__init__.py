"""Python binding of librkv.so, the write-time FP8 ring KV cache for MI355X.

Argument marshalling only: every step of the hot path runs in the HIP kernels
behind the C ABI declared in include/rkv.h.  The functions below keep the C
names (ring_cache_bytes, ring_cache_create, ..., cache_attend) and take raw
device pointers and stream handles; ``RingCache`` wraps them for torch
tensors (PyTorch provides device memory and streams, nothing else).

The library binds to the HIP runtime already loaded by torch (same soname),
so torch is imported before the library is opened; there is no CPU
fallback -- a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # noqa: F401  (must precede loading librkv.so: one HIP runtime per process)

__all__ = [
    "RKV_OK", "RKV_EINVAL", "RKV_EHIP", "RKV_PRECISE", "RKV_FAST",
    "rkv_params", "rkv_layout", "RkvError", "lib", "lib_path",
    "ring_cache_bytes", "ring_cache_create", "ring_cache_destroy", "ring_cache_reset",
    "ring_cache_layout", "cache_write_rope_fp8", "cache_write_global", "cache_delta_rotate", "cache_attend",
    "cache_attend_noalloc",
    "cache_write_attend", "ring_cache_set_qk_norm", "ring_cache_calibrate_static",
    "rkv_last_error", "RingCache",
]

RKV_OK, RKV_EINVAL, RKV_EHIP = 0, -1, -2
RKV_PRECISE, RKV_FAST = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "librkv.so")


class rkv_params(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("n_slots", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_queries", ctypes.c_int32),
        ("precision", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("scale_margin", ctypes.c_float),
        ("attn_workgroups", ctypes.c_int32),
        ("attn_merge_wait_us", ctypes.c_int32),
        ("n_global", ctypes.c_int32),
        ("rope_bands", ctypes.c_int32 * 3),
    ]


class rkv_layout(ctypes.Structure):
    _fields_ = [
        ("codes_k", ctypes.c_size_t),
        ("codes_v", ctypes.c_size_t),
        ("scale_k", ctypes.c_size_t),
        ("scale_v", ctypes.c_size_t),
        ("slot_pos", ctypes.c_size_t),
        ("state", ctypes.c_size_t),
        ("vmax", ctypes.c_size_t),
        ("layer_bytes", ctypes.c_size_t),
        ("n_slots_padded", ctypes.c_int32),
        ("slot_yx", ctypes.c_size_t),
        ("n_global", ctypes.c_int32),
        ("global_first_slot", ctypes.c_int32),
    ]


class RkvError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed ({code}): {rkv_last_error()}")
        self.code = code


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Open librkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m fp8_ring_kv_amd.build`")
    L = ctypes.CDLL(path)
    P, I32, SZ, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    L.ring_cache_bytes.argtypes = [P(rkv_params)]
    L.ring_cache_bytes.restype = SZ
    L.ring_cache_create.argtypes = [P(rkv_params), VP, SZ, VP, P(VP)]
    L.ring_cache_create.restype = ctypes.c_int
    L.ring_cache_destroy.argtypes = [VP]
    L.ring_cache_destroy.restype = ctypes.c_int
    L.ring_cache_reset.argtypes = [VP, I32, VP]
    L.ring_cache_reset.restype = ctypes.c_int
    L.ring_cache_layout.argtypes = [VP, I32, P(rkv_layout)]
    L.ring_cache_layout.restype = ctypes.c_int
    L.cache_write_rope_fp8.argtypes = [VP, I32, VP, VP, VP, I32, VP]
    L.cache_write_rope_fp8.restype = ctypes.c_int
    L.cache_delta_rotate.argtypes = [VP, I32, I32, VP]
    L.cache_delta_rotate.restype = ctypes.c_int
    L.cache_attend.argtypes = [VP, I32, VP, VP, I32, VP, VP]
    L.cache_attend.restype = ctypes.c_int
    L.cache_write_global.argtypes = [VP, I32, I32, VP, VP, VP, I32, VP]
    L.cache_write_global.restype = ctypes.c_int
    L.cache_attend_noalloc.argtypes = [VP, I32, VP, VP, I32, VP, VP]
    L.cache_attend_noalloc.restype = ctypes.c_int
    L.cache_write_attend.argtypes = [VP, I32, VP, VP, VP, I32, VP, VP, I32, VP, VP]
    L.cache_write_attend.restype = ctypes.c_int
    L.rkv_last_error.argtypes = []
    L.rkv_last_error.restype = ctypes.c_char_p
    L.ring_cache_set_qk_norm.argtypes = [VP, I32, VP, VP, ctypes.c_float, VP]
    L.ring_cache_calibrate_static.argtypes = [VP, I32, ctypes.c_float, VP]
    L.ring_cache_calibrate_static.restype = ctypes.c_int
    L.ring_cache_set_qk_norm.restype = ctypes.c_int
    _lib = L
    return L


# ---- raw C ABI (same names as include/rkv.h) --------------------------------

def rkv_last_error() -> str:
    return lib().rkv_last_error().decode()


def ring_cache_bytes(params: rkv_params) -> int:
    return int(lib().ring_cache_bytes(ctypes.byref(params)))


def ring_cache_create(params: rkv_params, dev_buf: int, nbytes: int, stream: int) -> int:
    h = ctypes.c_void_p()
    rc = lib().ring_cache_create(ctypes.byref(params), ctypes.c_void_p(dev_buf), nbytes,
                                 ctypes.c_void_p(stream), ctypes.byref(h))
    if rc != RKV_OK:
        raise RkvError(rc, "ring_cache_create")
    return h.value


def ring_cache_destroy(handle: int) -> None:
    lib().ring_cache_destroy(ctypes.c_void_p(handle))


def ring_cache_reset(handle: int, layer: int, stream: int) -> None:
    rc = lib().ring_cache_reset(ctypes.c_void_p(handle), layer, ctypes.c_void_p(stream))
    if rc != RKV_OK:
        raise RkvError(rc, "ring_cache_reset")


def ring_cache_layout(handle: int, layer: int) -> rkv_layout:
    out = rkv_layout()
    rc = lib().ring_cache_layout(ctypes.c_void_p(handle), layer, ctypes.byref(out))
    if rc != RKV_OK:
        raise RkvError(rc, "ring_cache_layout")
    return out


def cache_write_rope_fp8(handle: int, layer: int, k: int, v: int, pos: int, n: int, stream: int) -> None:
    rc = lib().cache_write_rope_fp8(ctypes.c_void_p(handle), layer, ctypes.c_void_p(k),
                                    ctypes.c_void_p(v), ctypes.c_void_p(pos), n, ctypes.c_void_p(stream))
    if rc != RKV_OK:
        raise RkvError(rc, "cache_write_rope_fp8")


def cache_write_global(handle: int, layer: int, first: int, k: int, v: int, pos: int, n: int, stream: int) -> None:
    rc = lib().cache_write_global(ctypes.c_void_p(handle), layer, first, ctypes.c_void_p(k), ctypes.c_void_p(v),
                                  ctypes.c_void_p(pos), n, ctypes.c_void_p(stream))
    if rc != RKV_OK:
        raise RkvError(rc, "cache_write_global")


def cache_delta_rotate(handle: int, layer: int, delta: int, stream: int) -> None:
    rc = lib().cache_delta_rotate(ctypes.c_void_p(handle), layer, delta, ctypes.c_void_p(stream))
    if rc != RKV_OK:
        raise RkvError(rc, "cache_delta_rotate")


def cache_attend(handle: int, layer: int, q: int, q_pos: int, n_q: int, out: int, stream: int) -> None:
    rc = lib().cache_attend(ctypes.c_void_p(handle), layer, ctypes.c_void_p(q), ctypes.c_void_p(q_pos),
                            n_q, ctypes.c_void_p(out), ctypes.c_void_p(stream))
    if rc != RKV_OK:
        raise RkvError(rc, "cache_attend")


def cache_attend_noalloc(handle: int, layer: int, q: int, q_pos: int, n_q: int, out: int, stream: int) -> None:
    rc = lib().cache_attend_noalloc(ctypes.c_void_p(handle), layer, ctypes.c_void_p(q), ctypes.c_void_p(q_pos),
                                    n_q, ctypes.c_void_p(out), ctypes.c_void_p(stream))
    if rc != RKV_OK:
        raise RkvError(rc, "cache_attend_noalloc")


def cache_write_attend(handle: int, layer: int, k: int, v: int, pos: int, n: int, q: int, q_pos: int,
                       n_q: int, out: int, stream: int) -> None:
    rc = lib().cache_write_attend(ctypes.c_void_p(handle), layer, ctypes.c_void_p(k), ctypes.c_void_p(v),
                                  ctypes.c_void_p(pos), n, ctypes.c_void_p(q), ctypes.c_void_p(q_pos), n_q,
                                  ctypes.c_void_p(out), ctypes.c_void_p(stream))
    if rc != RKV_OK:
        raise RkvError(rc, "cache_write_attend")


def ring_cache_set_qk_norm(handle: int, layer: int, wq: int, wk: int, eps: float, stream: int) -> None:
    rc = lib().ring_cache_set_qk_norm(ctypes.c_void_p(handle), layer, ctypes.c_void_p(wq), ctypes.c_void_p(wk),
                                      eps, ctypes.c_void_p(stream))
    if rc != RKV_OK:
        raise RkvError(rc, "ring_cache_set_qk_norm")


def ring_cache_calibrate_static(handle: int, layer: int, margin: float, stream: int) -> None:
    rc = lib().ring_cache_calibrate_static(ctypes.c_void_p(handle), layer, margin, ctypes.c_void_p(stream))
    if rc != RKV_OK:
        raise RkvError(rc, "ring_cache_calibrate_static")


# ---- torch-facing wrapper ---------------------------------------------------

def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check(t: torch.Tensor, dtype, shape, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")


class RingCache:
    """One allocation holding every layer's ring cache plus the attention workspace."""

    def __init__(self, n_layers: int, n_slots: int, n_heads: int, head_dim: int, max_queries: int,
                 precision: int = RKV_PRECISE, rope_base: float = 10000.0, scale_margin: float = 1.0,
                 device: str | torch.device = "cuda", stream=None, attn_workgroups: int = 0,
                 attn_merge_wait_us: int = -1, n_global: int = 0, rope_bands=(0, 0, 0)):
        self.params = rkv_params(n_layers, n_slots, n_heads, head_dim, max_queries, precision,
                                 rope_base, scale_margin, attn_workgroups, attn_merge_wait_us, n_global,
                                 (ctypes.c_int32 * 3)(*rope_bands))
        self.n_global = n_global
        self.rope_bands = tuple(int(b) for b in rope_bands)
        self.pos_width = 3 if any(rope_bands) else 1
        nbytes = ring_cache_bytes(self.params)
        if nbytes == 0:
            raise RkvError(RKV_EINVAL, "ring_cache_bytes")
        self.nbytes = nbytes
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if self.buf.data_ptr() % 256:
            raise RuntimeError("device buffer is not 256-byte aligned")
        self.handle = ring_cache_create(self.params, self.buf.data_ptr(), nbytes, _stream_handle(stream))
        self.n_layers, self.n_slots, self.n_heads, self.head_dim = n_layers, n_slots, n_heads, head_dim
        self.max_queries = max_queries

    def close(self):
        if getattr(self, "handle", None):
            ring_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _pos_shape(self, n: int):
        return (n,) if self.pos_width == 1 else (n, 3)

    # -- hot path --
    def write(self, layer: int, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor, stream=None):
        n = k.shape[0]
        shape = (n, self.n_heads, self.head_dim)
        _check(k, torch.bfloat16, shape, "k")
        _check(v, torch.bfloat16, shape, "v")
        _check(pos, torch.int32, self._pos_shape(n), "pos")
        cache_write_rope_fp8(self.handle, layer, k.data_ptr(), v.data_ptr(), pos.data_ptr(), n,
                             _stream_handle(stream))

    def write_global(self, layer: int, first: int, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor,
                     stream=None):
        """Global (sink) slots first .. first + n - 1 of `layer`."""
        n = k.shape[0]
        shape = (n, self.n_heads, self.head_dim)
        _check(k, torch.bfloat16, shape, "k")
        _check(v, torch.bfloat16, shape, "v")
        _check(pos, torch.int32, self._pos_shape(n), "pos")
        cache_write_global(self.handle, layer, first, k.data_ptr(), v.data_ptr(), pos.data_ptr(), n,
                           _stream_handle(stream))

    def set_qk_norm(self, layer: int, wq: torch.Tensor | None, wk: torch.Tensor | None, eps: float = 1e-6,
                    stream=None):
        """Fused Q/K RMS norm for `layer` (-1: all) with bf16 [head_dim] weights; None, None turns it off.
        The weight tensors are kept alive here until the next call (the copy is asynchronous)."""
        if wq is None and wk is None:
            ring_cache_set_qk_norm(self.handle, layer, 0, 0, eps, _stream_handle(stream))
            return
        for t, nm in ((wq, "wq"), (wk, "wk")):
            _check(t, torch.bfloat16, (self.head_dim,), nm)
        self._norm_refs = (wq, wk)
        ring_cache_set_qk_norm(self.handle, layer, wq.data_ptr(), wk.data_ptr(), eps, _stream_handle(stream))

    def calibrate_static(self, layer: int, margin: float = 1.5, stream=None):
        """Switch `layer` (-1: all) to static per-head scales from the valid cache's amax x margin."""
        ring_cache_calibrate_static(self.handle, layer, margin, _stream_handle(stream))

    def static_scales(self, layer: int) -> torch.Tensor:
        """[2][H] float32: static key and value scales (zeros before calibration)."""
        lay = self.layout(layer)
        base = lay.vmax + ((4 * 8 * self.n_heads + 255) // 256) * 256
        base += ((2 * self.head_dim * 2 + 255) // 256) * 256
        return self._view(base, 4 * 2 * self.n_heads, torch.float32).view(2, self.n_heads)

    def static_flag(self, layer: int) -> bool:
        """True once the layer is calibrated (static scales in use); reads the device."""
        lay = self.layout(layer)
        base = lay.vmax + ((4 * 8 * self.n_heads + 255) // 256) * 256
        base += ((2 * self.head_dim * 2 + 255) // 256) * 256
        return bool(self._view(base + 4 * 2 * self.n_heads, 4, torch.int32).item())

    def rotate(self, layer: int, delta: int, stream=None):
        cache_delta_rotate(self.handle, layer, int(delta), _stream_handle(stream))

    def attend(self, layer: int, q: torch.Tensor, q_pos: torch.Tensor, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
        n_q = q.shape[0]
        shape = (n_q, self.n_heads, self.head_dim)
        _check(q, torch.bfloat16, shape, "q")
        _check(q_pos, torch.int32, self._pos_shape(n_q), "q_pos")
        if out is None:
            out = torch.empty(shape, dtype=torch.bfloat16, device=q.device)
        _check(out, torch.bfloat16, shape, "out")
        cache_attend(self.handle, layer, q.data_ptr(), q_pos.data_ptr(), n_q, out.data_ptr(),
                     _stream_handle(stream))
        return out

    def write_attend(self, layer: int, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor, q: torch.Tensor,
                     q_pos: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """write(layer, k, v, pos) then attend(layer, q, q_pos, out) in one call."""
        n, n_q = k.shape[0], q.shape[0]
        _check(k, torch.bfloat16, (n, self.n_heads, self.head_dim), "k")
        _check(v, torch.bfloat16, (n, self.n_heads, self.head_dim), "v")
        _check(pos, torch.int32, self._pos_shape(n), "pos")
        shape = (n_q, self.n_heads, self.head_dim)
        _check(q, torch.bfloat16, shape, "q")
        _check(q_pos, torch.int32, self._pos_shape(n_q), "q_pos")
        if out is None:
            out = torch.empty(shape, dtype=torch.bfloat16, device=q.device)
        _check(out, torch.bfloat16, shape, "out")
        cache_write_attend(self.handle, layer, k.data_ptr(), v.data_ptr(), pos.data_ptr(), n, q.data_ptr(),
                           q_pos.data_ptr(), n_q, out.data_ptr(), _stream_handle(stream))
        return out

    def reset(self, layer: int = -1, stream=None):
        ring_cache_reset(self.handle, layer, _stream_handle(stream))

    # -- views of the device layout (for checks and tests) --
    def layout(self, layer: int) -> rkv_layout:
        return ring_cache_layout(self.handle, layer)

    def _view(self, off: int, nbytes: int, dtype) -> torch.Tensor:
        return self.buf[off:off + nbytes].view(dtype)

    def state(self, layer: int) -> torch.Tensor:
        """(head, n_valid, ticket counter, g_valid) int32 on device (the third is
        internal to the write kernel, zero between calls)."""
        lay = self.layout(layer)
        return self._view(lay.state, 16, torch.int32)

    def write_counters(self, layer: int) -> torch.Tensor:
        """The write kernel's ticket counters (top, then one per sub-counter line),
        int32 on device; zero between calls."""
        lay = self.layout(layer)
        region = self._view(lay.state, 4 * 64 * 9, torch.int32)
        return torch.cat([region[2:3], region[64::64]])

    def vmax(self, layer: int) -> torch.Tensor:
        """[H] float32: largest value scale written to each head since the reset."""
        lay = self.layout(layer)
        return self._view(lay.vmax, 4 * 8 * self.n_heads, torch.float32).view(self.n_heads, 8).amax(dim=1)

    def _canon(self, t: torch.Tensor, lay: rkv_layout) -> torch.Tensor:
        """Slot axis (dim 1, or 0 for 1-D) in canonical order: the ring's slots,
        then the global slots."""
        g0, ng = lay.global_first_slot, lay.n_global
        if t.dim() == 1:
            return torch.cat([t[: self.n_slots], t[g0:g0 + ng]]) if ng else t[: self.n_slots]
        return torch.cat([t[:, : self.n_slots], t[:, g0:g0 + ng]], dim=1) if ng else t[:, : self.n_slots]

    def slot_pos(self, layer: int) -> torch.Tensor:
        """[N + n_global] int32: each slot's position (3-D RoPE: t), ring then globals."""
        lay = self.layout(layer)
        return self._canon(self._view(lay.slot_pos, 4 * lay.n_slots_padded, torch.int32), lay)

    def slot_yx(self, layer: int) -> torch.Tensor:
        """[N + n_global][2] int32: spatial coordinates (y, x) of each slot (3-D RoPE)."""
        lay = self.layout(layer)
        yx = self._view(lay.slot_yx, 8 * lay.n_slots_padded, torch.int32).view(2, lay.n_slots_padded)
        return self._canon(yx, lay).t()

    def scales(self, layer: int):
        """(scale_k, scale_v) as [H][N + n_global] float32 tensors (ring, then globals)."""
        lay = self.layout(layer)
        n = self.n_heads * lay.n_slots_padded * 4
        sk = self._view(lay.scale_k, n, torch.float32).view(self.n_heads, lay.n_slots_padded)
        sv = self._view(lay.scale_v, n, torch.float32).view(self.n_heads, lay.n_slots_padded)
        return self._canon(sk, lay), self._canon(sv, lay)

    def codes(self, layer: int):
        """(codes_k, codes_v) as [H][N + n_global][D] uint8 tensors in canonical
        slot order (V de-tiled)."""
        lay = self.layout(layer)
        H, D, NP = self.n_heads, self.head_dim, lay.n_slots_padded
        ck = self._view(lay.codes_k, H * NP * D, torch.uint8).view(H, NP, D)
        cv = self._view(lay.codes_v, H * NP * D, torch.uint8).view(H, NP // 16, D, 16)
        cv = cv.permute(0, 1, 3, 2).reshape(H, NP, D)
        return self._canon(ck, lay), self._canon(cv, lay)
