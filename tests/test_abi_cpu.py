"""C ABI checks that need no GPU: the library loads into torch's HIP runtime,
exports every function include/rkv.h declares, and rejects host-visible
misuse with RKV_EINVAL before enqueueing anything.  No call here reaches a
kernel launch."""
import ctypes
import os
import re

import pytest

import fp8_ring_kv_amd as rkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text,
                                flags=re.M))
    return sorted(n for n in names if n not in ("if", "defined"))


def test_library_is_built():
    assert os.path.exists(rkv.lib_path()), "run `python -m fp8_ring_kv_amd.build` first"


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) >= {"ring_cache_bytes", "ring_cache_create", "ring_cache_destroy",
                          "ring_cache_reset", "ring_cache_layout", "cache_write_rope_fp8",
                          "cache_delta_rotate", "cache_attend", "cache_write_attend", "rkv_last_error",
                          "cache_attend_noalloc", "ring_cache_calibrate_static", "ring_cache_set_qk_norm"}
    L = rkv.lib()
    for n in names:
        assert hasattr(L, n), n


def test_measurement_probes_live_outside_the_cache_library():
    """The benchmark's probes are a library of their own (librkv_probe.so,
    declared in csrc/probe/rkv_probe.h): exported there, not by librkv.so."""
    from fp8_ring_kv_amd import probe
    path = os.path.join(ROOT, "fp8_ring_kv_amd", "csrc", "probe", "rkv_probe.h")
    text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(rkv_probe_[a-z0-9_]*)\s*\(", text, flags=re.M))
    assert names == {"rkv_probe_fp8_mfma", "rkv_probe_stream", "rkv_probe_last_error"}
    P = probe.lib()
    for n in names:
        assert hasattr(P, n), n
        assert not hasattr(rkv.lib(), n), n


def test_single_hip_runtime_in_process():
    rkv.lib()
    maps = open("/proc/self/maps").read()
    libs = sorted(set(re.findall(r"\S*libamdhip64\.so\S*", maps)))
    assert len(libs) == 1, libs


def params(**kw):
    base = dict(n_layers=1, n_slots=5788, n_heads=12, head_dim=128, max_queries=757,
                precision=rkv.RKV_PRECISE, rope_base=10000.0, scale_margin=1.0, attn_workgroups=0,
                attn_merge_wait_us=-1, n_global=0, rope_bands=(0, 0, 0))
    base.update(kw)
    bands = base.pop("rope_bands")
    p = rkv.rkv_params(**base)
    p.rope_bands[:] = list(bands)
    return p


def test_bytes_cover_the_layout():
    p = params()
    nb = rkv.ring_cache_bytes(p)
    np_ = 5824  # 5788 rounded up to 64
    per_layer = 2 * 12 * np_ * 128 + 2 * 12 * np_ * 4 + np_ * 4 + 16
    assert nb > per_layer
    p60 = params(n_layers=60)
    assert rkv.ring_cache_bytes(p60) - nb >= 59 * per_layer
    assert nb % 256 == 0


@pytest.mark.parametrize("field,value", [
    ("n_layers", 0), ("n_slots", 0), ("n_slots", (1 << 20) + 1), ("n_heads", 0),
    ("head_dim", 96), ("head_dim", 256), ("max_queries", 0), ("precision", 7),
    ("rope_base", 1.0), ("rope_base", float("inf")), ("scale_margin", 0.0),
    ("attn_workgroups", -1), ("attn_workgroups", 4097),
    ("attn_merge_wait_us", -2), ("attn_merge_wait_us", 10001),
])
def test_invalid_params_give_zero_bytes_and_einval(field, value):
    p = params(**{field: value})
    assert rkv.ring_cache_bytes(p) == 0
    assert rkv.rkv_last_error() != ""
    h = ctypes.c_void_p()
    rc = rkv.lib().ring_cache_create(ctypes.byref(p), ctypes.c_void_p(1 << 20), 1 << 40, None, ctypes.byref(h))
    assert rc == rkv.RKV_EINVAL and h.value is None


def test_create_rejects_bad_buffers_without_launching():
    p = params()
    nb = rkv.ring_cache_bytes(p)
    L = rkv.lib()
    h = ctypes.c_void_p()
    assert L.ring_cache_create(ctypes.byref(p), None, nb, None, ctypes.byref(h)) == rkv.RKV_EINVAL
    assert L.ring_cache_create(ctypes.byref(p), ctypes.c_void_p(0x1000 + 16), nb, None,
                               ctypes.byref(h)) == rkv.RKV_EINVAL
    assert "aligned" in rkv.rkv_last_error()
    assert L.ring_cache_create(ctypes.byref(p), ctypes.c_void_p(0x1000), nb - 256, None,
                               ctypes.byref(h)) == rkv.RKV_EINVAL
    assert "too small" in rkv.rkv_last_error()
    assert L.ring_cache_create(ctypes.byref(p), ctypes.c_void_p(0x1000), nb, None, None) == rkv.RKV_EINVAL


def test_calls_on_null_cache_are_einval():
    L = rkv.lib()
    assert L.cache_write_rope_fp8(None, 0, None, None, None, 1, None) == rkv.RKV_EINVAL
    assert L.cache_delta_rotate(None, 0, 5, None) == rkv.RKV_EINVAL
    assert L.cache_attend(None, 0, None, None, 1, None, None) == rkv.RKV_EINVAL
    assert L.ring_cache_reset(None, -1, None) == rkv.RKV_EINVAL
    assert L.ring_cache_layout(None, 0, None) == rkv.RKV_EINVAL
    assert L.ring_cache_destroy(None) == rkv.RKV_OK


def test_probes_reject_misuse_without_launching():
    """The measurement aids validate their arguments on the host: nothing
    below reaches a kernel launch (no GPU here)."""
    from fp8_ring_kv_amd import probe
    L = probe.lib()
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: every call fails validation first
    assert L.rkv_probe_fp8_mfma(1, 1, None, None) == -1
    assert L.rkv_probe_fp8_mfma(0, 1, fake, None) == -1
    assert L.rkv_probe_fp8_mfma(65537, 1, fake, None) == -1
    assert L.rkv_probe_fp8_mfma(1, 0, fake, None) == -1
    assert L.rkv_probe_fp8_mfma(1, (1 << 20) + 1, fake, None) == -1
    assert L.rkv_probe_fp8_mfma(1, 1, ctypes.c_void_p(0x100002), None) == -1
    assert L.rkv_probe_stream(None, 16, None) == -1
    assert L.rkv_probe_stream(ctypes.c_void_p(0x100008), 16, None) == -1
    assert L.rkv_probe_stream(fake, 0, None) == -1
    assert L.rkv_probe_stream(fake, 24, None) == -1
    assert "multiple of 16" in probe.rkv_probe_last_error()


def test_attention_partials_stay_within_their_addressing():
    """The split partials are addressed with 32-bit offsets and a 1 GiB
    past-the-end offset: (units + workgroups) x 128 x head_dim x 2 bytes
    must stay within 1 GiB."""
    assert rkv.ring_cache_bytes(params(n_heads=256, max_queries=1 << 16)) == 0
    assert "partials" in rkv.rkv_last_error()
    assert rkv.ring_cache_bytes(params(n_heads=256, max_queries=1 << 16, head_dim=64)) == 0
    assert rkv.ring_cache_bytes(params(n_heads=48, max_queries=1 << 16)) > 0  # 24,576 units + 4,096
    assert rkv.ring_cache_bytes(params(n_heads=256, max_queries=14336)) > 0  # 28,672 units + 4,096


def test_rope_band_and_global_parameters_are_checked():
    assert rkv.ring_cache_bytes(params(rope_bands=(22, 21, 21), n_global=1246)) > 0
    assert rkv.ring_cache_bytes(params(rope_bands=(22, 21, 20))) == 0  # 63 pairs, not 64
    assert "rope_bands" in rkv.rkv_last_error()
    assert rkv.ring_cache_bytes(params(rope_bands=(70, -3, -3))) == 0
    assert rkv.ring_cache_bytes(params(n_global=-1)) == 0
    assert rkv.ring_cache_bytes(params(n_global=(1 << 20) + 1)) == 0
    # the globals add whole tiles of slot arrays to every layer
    a = rkv.ring_cache_bytes(params(n_layers=2))
    b = rkv.ring_cache_bytes(params(n_layers=2, n_global=1246))
    assert b - a >= 2 * 1280 * 12 * (2 * 128 + 8)
