"""GPU parity of the pages' static-scale mode (Runway Characters paper §4.3
"FP8 at write", Appendix G): calibration from the cache's amax x 1.5, static
writes that saturate, reset rotations that keep the scales.  Bars as for the
plain path: bookkeeping and the calibrated scales bit-exact, dequantized
cache elements within 1 e4m3 ulp, attention within the 2e-2 / 2e-3 gates."""
import ctypes

import numpy as np
import pytest
import torch

import fp8_ring_kv_amd as rkv
from oracle import attend as oatt, ring as oring
from oracle.bf16 import round_bf16
from tests.gpu_common import DEV, assert_cache_matches, check_attention, pos_dev, require_gpu, rotate_checked, to_dev
from workloads import ATTEND, Bf16, Config, OutlierSpec, Stream, positions

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_static_session_matches_oracle():
    cfg = Config("static", n_heads=4, head_dim=128, n_slots=700, chunk=300, seed=31,
                 outliers=OutlierSpec(0.02, 8.0))
    cache = rkv.RingCache(1, cfg.n_slots, cfg.n_heads, cfg.head_dim, cfg.chunk, rkv.RKV_PRECISE, device=DEV)
    st = oring.RingState(cfg.n_slots, cfg.n_heads, cfg.head_dim)
    s = Stream(cfg)
    p0 = 0
    for c in range(2):  # per-token scales first
        _, k, v = s.chunk()
        pos = positions(p0, cfg.chunk)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
        p0 += cfg.chunk
    cache.calibrate_static(0, 1.5)
    oring.calibrate_static(st, 1.5)
    got = cache.static_scales(0).cpu().numpy().astype(np.float64)
    # value scales are bit-exact (per-token value scales are).  A per-token key
    # scale may differ by one ulp (amax of fp32 against float64 RoPE); times
    # the margin 1.5 and rounded once more, that is at most two ulps of the
    # static scale (2^-22 relative)
    assert np.array_equal(got[1], st.static_v), (got[1], st.static_v)
    assert np.all(np.abs(got[0] - st.static_k) <= st.static_k * 2.0 ** -22), (got[0] - st.static_k, st.static_k)
    # the calibration requantized the valid cache with the head scales; the
    # oracle used its own (float64) key scales, the device its own: compare
    # against an oracle state holding the device's static key scales
    st.static_k = got[0].copy()
    st2 = st.copy()
    assert_cache_matches(cache, 0, st2)
    for c in range(3):  # static writes; the ring wraps and every slot is rewritten
        _, k, v = s.chunk()
        pos = positions(p0, cfg.chunk)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
        p0 += cfg.chunk
        assert_cache_matches(cache, 0, st)
    pre = st.copy()
    sk_before = cache.scales(0)[0].clone()
    rotate_checked(cache, 0, -600)
    oring.rotate(st, -600)
    assert_cache_matches(cache, 0, st, pre=pre)
    assert torch.equal(cache.scales(0)[0], sk_before)  # every slot already held its head's scale
    q, _, _ = s.chunk()
    qpos = positions(p0 - 600 - cfg.chunk, cfg.chunk)
    out = cache.attend(0, to_dev(q), pos_dev(qpos)).float().cpu().numpy().astype(np.float64)
    check_attention("static session", cache, 0, st, q.f64, qpos, out)


def test_margin_below_one_saturates_like_the_oracle():
    """A margin below 1 puts the head's largest elements beyond 448 s: the
    calibration's requantization and every later static write clamp them at
    +-448 (code 0x7E / 0xFE), on the device as in the oracle; the attention
    over the clamped cache against exact fp64 attention on the same cache."""
    cfg = Config("static_sat", n_heads=2, head_dim=128, n_slots=500, chunk=200, seed=37,
                 outliers=OutlierSpec(0.02, 8.0))
    cache = rkv.RingCache(1, cfg.n_slots, 2, 128, 200, rkv.RKV_PRECISE, device=DEV)
    st = oring.RingState(cfg.n_slots, 2, 128)
    s = Stream(cfg)
    for c in range(2):
        _, k, v = s.chunk()
        pos = positions(200 * c, 200)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
    cache.calibrate_static(0, 0.75)
    oring.calibrate_static(st, 0.75)
    got = cache.static_scales(0).cpu().numpy().astype(np.float64)
    assert np.array_equal(got[1], st.static_v), (got[1], st.static_v)
    assert np.all(np.abs(got[0] - st.static_k) <= st.static_k * 2.0 ** -22), (got[0] - st.static_k, st.static_k)
    st.static_k = got[0].copy()
    assert_cache_matches(cache, 0, st)
    kc, vc = (t.cpu().numpy() for t in cache.codes(0))
    for name, codes in (("keys", kc), ("values", vc)):  # the clamp was reached
        assert np.any((codes & 0x7F) == 0x7E), f"no saturated {name} after calibrating at 0.75"
    q, k, v = s.chunk()
    pos = positions(400, 200)
    cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))  # static write, saturating
    oring.write(st, k.f64, v.f64, pos)
    assert_cache_matches(cache, 0, st)
    out = cache.attend(0, to_dev(q), pos_dev(pos)).float().cpu().numpy().astype(np.float64)
    check_attention("static scales at margin 0.75", cache, 0, st, q.f64, pos, out)


def test_rotation_right_after_calibration():
    """Keys written with per-token scales, calibrated, then rotated before any
    rewrite: the rotation moves them to the head's static scale, which covers
    every rotated component, so nothing clips (keeping each key's own
    per-token scale would clip about half of them)."""
    cfg = Config("static_rot", n_heads=4, head_dim=128, n_slots=700, chunk=300, seed=33,
                 outliers=OutlierSpec(0.02, 8.0))
    cache = rkv.RingCache(1, cfg.n_slots, cfg.n_heads, cfg.head_dim, cfg.chunk, rkv.RKV_PRECISE, device=DEV)
    st = oring.RingState(cfg.n_slots, cfg.n_heads, cfg.head_dim)
    s = Stream(cfg)
    for c in range(2):
        _, k, v = s.chunk()
        pos = positions(300 * c, 300)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
    cache.calibrate_static(0, 1.5)
    oring.calibrate_static(st, 1.5)
    pre = st.copy()
    rotate_checked(cache, 0, -600)
    oring.rotate(st, -600)
    assert_cache_matches(cache, 0, st, pre=pre)
    ck, _ = cache.codes(0)
    sk, _ = cache.scales(0)
    valid = oring.valid_slots(st)
    from oracle import e4m3
    assert np.max(np.abs(e4m3.decode(ck.cpu().numpy()[:, valid]))) < 448  # nothing clipped
    stat = cache.static_scales(0).cpu()
    vt = torch.from_numpy(valid)
    assert torch.equal(sk.cpu()[:, vt], stat[0][:, None].expand(-1, len(valid)))
    q, _, _ = s.chunk()
    qpos = positions(0, cfg.chunk)
    out = cache.attend(0, to_dev(q), pos_dev(qpos)).float().cpu().numpy().astype(np.float64)
    check_attention("attention after the rotation", cache, 0, st, q.f64, qpos, out)


def test_calibrating_an_empty_layer_keeps_per_token_scales():
    """Layer 1 holds nothing when every layer is calibrated: its static scales
    are 0 and its later writes (and rotations) keep the per-(token, head)
    rule instead of storing zero codes."""
    cfg = Config("static_empty", n_heads=2, head_dim=128, n_slots=300, chunk=100, seed=34,
                 outliers=OutlierSpec(0.02, 8.0))
    cache = rkv.RingCache(2, cfg.n_slots, cfg.n_heads, cfg.head_dim, cfg.chunk, device=DEV)
    s = Stream(cfg)
    _, k, v = s.chunk()
    cache.write(0, to_dev(k), to_dev(v), pos_dev(positions(0, 100)))
    cache.calibrate_static(-1, 1.5)
    assert cache.static_flag(1) and not cache.static_scales(1).cpu().numpy().any()
    st = oring.RingState(cfg.n_slots, cfg.n_heads, cfg.head_dim)
    oring.calibrate_static(st, 1.5)
    for c in range(2):
        _, k, v = s.chunk()
        pos = positions(100 * c, 100)
        cache.write(1, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
        assert_cache_matches(cache, 1, st)
    assert cache.codes(1)[0].cpu().numpy().any()
    rotate_checked(cache, 1, -50)


def test_reset_returns_to_per_token_scales():
    cfg = Config("static_reset", n_heads=2, head_dim=64, n_slots=200, chunk=64, seed=32)
    cache = rkv.RingCache(1, cfg.n_slots, cfg.n_heads, cfg.head_dim, cfg.chunk, device=DEV)
    st = oring.RingState(cfg.n_slots, cfg.n_heads, cfg.head_dim)
    s = Stream(cfg)
    _, k, v = s.chunk()
    cache.write(0, to_dev(k), to_dev(v), pos_dev(positions(0, 64)))
    cache.calibrate_static(-1, 1.5)
    cache.reset(0)
    oring.reset(st)
    assert not cache.static_scales(0).cpu().numpy().any()
    _, k, v = s.chunk()
    cache.write(0, to_dev(k), to_dev(v), pos_dev(positions(0, 64)))
    oring.write(st, k.f64, v.f64, positions(0, 64))
    assert_cache_matches(cache, 0, st)


def test_calibrate_rejects_bad_arguments():
    cache = rkv.RingCache(2, 64, 2, 64, 16, device=DEV)
    L = rkv.lib()
    vp, s = ctypes.c_void_p, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.ring_cache_calibrate_static(None, 0, 1.5, s) == rkv.RKV_EINVAL
    assert L.ring_cache_calibrate_static(vp(cache.handle), 2, 1.5, s) == rkv.RKV_EINVAL
    for m in (0.0, -1.0, 65.0, float("nan")):
        assert L.ring_cache_calibrate_static(vp(cache.handle), 0, m, s) == rkv.RKV_EINVAL, m
    assert "margin" in rkv.rkv_last_error()


def test_static_attention_full_size_every_element():
    """The 757 x 5,788 x 12 workload (ring head at 3,100, 2% outliers x8) after
    the calibration: the attention takes the static path (s_k in the queries,
    s_v after the product, no per-slot scales), through the same split-unit
    merges as the per-token path; every output element against exact fp64
    attention on the device's cache and the kernel's declared numerics."""
    cfg = ATTEND
    cache = rkv.RingCache(1, cfg.n_slots, cfg.n_heads, cfg.head_dim, 757, rkv.RKV_PRECISE, device=DEV)
    st = oring.RingState(cfg.n_slots, cfg.n_heads, cfg.head_dim)
    s = Stream(cfg)
    p0 = 0
    while p0 < 8888:
        n = min(757, 8888 - p0)
        _, k, v = s.chunk(n)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(positions(p0, n)))
        oring.write(st, k.f64, v.f64, positions(p0, n))
        p0 += n
    cache.calibrate_static(0, 1.5)
    oring.calibrate_static(st, 1.5)
    st.static_k = cache.static_scales(0).cpu().numpy().astype(np.float64)[0].copy()
    q, _, _ = s.chunk(757)
    qpos = positions(8131, 757)
    out = cache.attend(0, to_dev(q), pos_dev(qpos)).float().cpu().numpy().astype(np.float64)
    check_attention("static C2 (all 12 heads x 757 rows)", cache, 0, None, q.f64, qpos, out)


def test_static_and_per_token_heads_in_one_layer():
    """Head 1's keys and values are all zero when the layer is calibrated: its
    static scales are 0 and it keeps the per-token rule (and the per-token
    attention) beside head 0's static path; later writes fill both."""
    cfg = Config("static_mixed", n_heads=2, head_dim=128, n_slots=400, chunk=150, seed=35,
                 outliers=OutlierSpec(0.02, 8.0))
    cache = rkv.RingCache(1, cfg.n_slots, 2, 128, 150, device=DEV)
    st = oring.RingState(cfg.n_slots, 2, 128)
    s = Stream(cfg)
    _, k, v = s.chunk()
    kz = Bf16(k.bits.copy(), k.f64.copy())
    vz = Bf16(v.bits.copy(), v.f64.copy())
    for t in (kz, vz):
        t.bits[:, 1] = 0
        t.f64[:, 1] = 0.0
    cache.write(0, to_dev(kz), to_dev(vz), pos_dev(positions(0, 150)))
    oring.write(st, kz.f64, vz.f64, positions(0, 150))
    cache.calibrate_static(0, 1.5)
    oring.calibrate_static(st, 1.5)
    stat = cache.static_scales(0).cpu().numpy()
    assert stat[0, 0] > 0 and stat[1, 0] > 0 and stat[0, 1] == 0 and stat[1, 1] == 0
    st.static_k = stat[0].astype(np.float64).copy()
    for c in (1, 2):
        q, k, v = s.chunk()
        pos = positions(150 * c, 150)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
        out = cache.attend(0, to_dev(q), pos_dev(pos)).float().cpu().numpy().astype(np.float64)
        check_attention(f"mixed static/per-token heads, chunk {c}", cache, 0, st, q.f64, pos, out)
