"""GPU parity of global (sink) slots and 3-D RoPE against the oracle
(Runway Characters paper, §2 "The step budget": each cache holds 1,246
global slots written once per session beside a six-latent window, all read
by attention; §4.2 and Appendix G: the temporal angle is omega_j (a t + b),
and a reset turns only the window's temporal frequencies -- spatial angles
and global tokens do not move).

Bars as for the 1-D ring: bookkeeping (head, n_valid, g_valid, every slot's
(t, y, x)) bit-exact, every dequantized element within 1 e4m3 ulp, the reset
rotation checked in isolation (every rotated key within 1 ulp of the
oracle's rotation of the device's own keys, globals untouched), attention
within 2e-2 max / 2e-3 mean of exact fp64 attention on the device cache."""
import numpy as np
import pytest
import torch

import fp8_ring_kv_amd as rkv
from oracle import ring as oring
from tests.gpu_common import DEV, assert_cache_matches, check_attention, require_gpu, rotate_checked, to_dev
from workloads import PAGES_LAYOUT, Config, OutlierSpec, Stream, frame_positions

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def p3(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


@pytest.mark.parametrize("head_dim,bands", [(128, (22, 21, 21)), (64, (11, 11, 10)), (128, (40, 24, 0))])
def test_globals_and_3d_ring_session(head_dim, bands):
    cfg = Config("g3d", n_heads=4, head_dim=head_dim, n_slots=200, chunk=70, seed=51,
                 outliers=OutlierSpec(0.02, 8.0), n_global=60, bands=bands)
    mk = lambda: rkv.RingCache(1, cfg.n_slots, cfg.n_heads, head_dim, 70, device=DEV, n_global=60, rope_bands=bands)
    cache, split = mk(), mk()
    st = oring.RingState(cfg.n_slots, cfg.n_heads, head_dim, n_global=60, bands=bands)
    s = Stream(cfg)
    for first, n in ((0, 35), (35, 25)):  # the globals, in two calls
        _, k, v = s.chunk(n)
        pos = frame_positions(-1, n, 12, first)
        for c in (cache, split):
            c.write_global(0, first, to_dev(k), to_dev(v), p3(pos))
        oring.write_global(st, first, k.f64, v.f64, pos)
        assert_cache_matches(cache, 0, st)
    for t in range(5):  # 350 tokens into 200 ring slots: wraps
        q, k, v = s.chunk()
        pos = frame_positions(t, 70, 9)
        out = cache.write_attend(0, to_dev(k), to_dev(v), p3(pos), to_dev(q), p3(pos))
        split.write(0, to_dev(k), to_dev(v), p3(pos))
        out_s = split.attend(0, to_dev(q), p3(pos))
        oring.write(st, k.f64, v.f64, pos)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out_s.view(torch.int16)), t  # fused = two calls
        assert_cache_matches(cache, 0, st)
        check_attention(f"globals + 3-D ring, frame {t}", cache, 0, st, q.f64, pos,
                        out.float().cpu().numpy().astype(np.float64))
    # reset: only the ring's temporal pairs turn; the globals stay bit-identical
    gk = [x.clone() for x in cache.codes(0) + cache.scales(0)]
    pre = st.copy()
    rotate_checked(cache, 0, -42)
    oring.rotate(st, -42)
    assert_cache_matches(cache, 0, st, pre=pre)
    for a, b in zip(cache.codes(0) + cache.scales(0), gk):
        assert torch.equal(a[:, 200:], b[:, 200:])
    q, k, v = s.chunk()
    pos = frame_positions(5 - 42, 70, 9)
    cache.write(0, to_dev(k), to_dev(v), p3(pos))
    oring.write(st, k.f64, v.f64, pos)
    out = cache.attend(0, to_dev(q), p3(pos)).float().cpu().numpy().astype(np.float64)
    check_attention("after the reset", cache, 0, st, q.f64, pos, out)
    # the pages' static scales include the globals in the calibration
    cache.calibrate_static(0, 1.5)
    oring.calibrate_static(st, 1.5)
    st.static_k = cache.static_scales(0).cpu().numpy().astype(np.float64)[0].copy()
    assert_cache_matches(cache, 0, st)
    out = cache.attend(0, to_dev(q), p3(pos)).float().cpu().numpy().astype(np.float64)
    check_attention("static scales over globals + ring", cache, 0, st, q.f64, pos, out)


def test_pages_layout_full_size():
    """The pages' cache at one GPU's head share: 1,246 globals + a 4,542-slot
    ring of six 757-token latents (5,788 slots read per call), 12 heads x 128,
    3-D RoPE; eight latents (the ring wraps), attention of the eighth latent's
    757 queries on every element, then a reset by -42 latents and one more."""
    cfg = PAGES_LAYOUT
    cache = rkv.RingCache(1, cfg.n_slots, cfg.n_heads, 128, 757, device=DEV, n_global=cfg.n_global,
                          rope_bands=cfg.bands)
    st = oring.RingState(cfg.n_slots, cfg.n_heads, 128, n_global=cfg.n_global, bands=cfg.bands)
    s = Stream(cfg)
    _, k, v = s.chunk(cfg.n_global)
    gpos = frame_positions(-1, cfg.n_global, 36)
    cache.write_global(0, 0, to_dev(k), to_dev(v), p3(gpos))
    oring.write_global(st, 0, k.f64, v.f64, gpos)
    for t in range(8):
        q, k, v = s.chunk()
        pos = frame_positions(t, 757, 28)
        cache.write(0, to_dev(k), to_dev(v), p3(pos))
        oring.write(st, k.f64, v.f64, pos)
    assert_cache_matches(cache, 0, st)
    assert (st.head, st.n_valid, st.g_valid) == ((8 * 757) % 4542, 4542, 1246)
    out = cache.attend(0, to_dev(q), p3(pos)).float().cpu().numpy().astype(np.float64)
    check_attention("pages layout (12 heads x 757 rows over 1,246 + 4,542 slots)", cache, 0, st, q.f64, pos, out)
    pre = st.copy()
    rotate_checked(cache, 0, -42)
    oring.rotate(st, -42)
    assert_cache_matches(cache, 0, st, pre=pre)
    q, k, v = s.chunk()
    pos = frame_positions(8 - 42, 757, 28)
    cache.write(0, to_dev(k), to_dev(v), p3(pos))
    oring.write(st, k.f64, v.f64, pos)
    out = cache.attend(0, to_dev(q), p3(pos)).float().cpu().numpy().astype(np.float64)
    check_attention("pages layout after the reset", cache, 0, st, q.f64, pos, out)


def test_global_write_rejects_bad_arguments():
    cache = rkv.RingCache(1, 64, 1, 64, 16, device=DEV, n_global=10, rope_bands=(16, 8, 8))
    k = torch.zeros(4, 1, 64, dtype=torch.bfloat16, device=DEV)
    pos = torch.zeros(4, 3, dtype=torch.int32, device=DEV)
    h, s = cache.handle, torch.cuda.current_stream().cuda_stream
    for first, n in ((7, 4), (-1, 4), (0, 0), (10, 1)):
        with pytest.raises(rkv.RkvError) as e:
            rkv.cache_write_global(h, 0, first, k.data_ptr(), k.data_ptr(), pos.data_ptr(), n, s)
        assert e.value.code == rkv.RKV_EINVAL
    torch.cuda.synchronize()
    assert int(cache.state(0)[3]) == 0  # nothing was enqueued
    plain = rkv.RingCache(1, 64, 1, 64, 16, device=DEV)  # no global slots
    with pytest.raises(rkv.RkvError):
        plain.write_global(0, 0, k, k, torch.zeros(4, dtype=torch.int32, device=DEV))
