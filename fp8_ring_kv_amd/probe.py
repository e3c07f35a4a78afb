"""Binding of librkv_probe.so, the benchmark's measurement aids (not part of
the cache library's ABI): the FP8 matrix-rate and HBM-stream probes declared
in csrc/probe/rkv_probe.h.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # noqa: F401  (must precede loading the library: one HIP runtime per process)

__all__ = ["ProbeError", "lib", "rkv_probe_fp8_mfma", "rkv_probe_stream", "rkv_probe_last_error"]

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librkv_probe.so")
_lib: Optional[ctypes.CDLL] = None


class ProbeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed ({code}): {rkv_probe_last_error()}")
        self.code = code


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is missing: build it with `python -m fp8_ring_kv_amd.build`")
        L = ctypes.CDLL(_PATH)
        VP = ctypes.c_void_p
        L.rkv_probe_fp8_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, VP, VP]
        L.rkv_probe_fp8_mfma.restype = ctypes.c_int
        L.rkv_probe_stream.argtypes = [VP, ctypes.c_size_t, VP]
        L.rkv_probe_stream.restype = ctypes.c_int
        L.rkv_probe_last_error.argtypes = []
        L.rkv_probe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def rkv_probe_last_error() -> str:
    return lib().rkv_probe_last_error().decode()


def rkv_probe_fp8_mfma(workgroups: int, iters: int, sink: int, stream: int) -> None:
    rc = lib().rkv_probe_fp8_mfma(workgroups, iters, ctypes.c_void_p(sink), ctypes.c_void_p(stream))
    if rc != 0:
        raise ProbeError(rc, "rkv_probe_fp8_mfma")


def rkv_probe_stream(buf: int, nbytes: int, stream: int) -> None:
    rc = lib().rkv_probe_stream(ctypes.c_void_p(buf), nbytes, ctypes.c_void_p(stream))
    if rc != 0:
        raise ProbeError(rc, "rkv_probe_stream")
