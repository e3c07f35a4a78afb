"""cache_attend_noalloc -- the attention with its workspace in the library's
fixed device scratch, for callers that cannot allocate -- against
cache_attend on the same cache, through the C ABI: identical output bits on
two calls in a row, the second with fewer queries (a smaller workspace laid
out over what the first left), and a request beyond the fixed size refused
before anything is enqueued."""
import numpy as np
import pytest
import torch

import fp8_ring_kv_amd as rkv
from tests.gpu_common import pos_dev, require_gpu, to_dev
from workloads import ATTEND, Config, OutlierSpec, Stream, positions

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _attend_noalloc(cache, layer, q, qpos, out):
    rkv.cache_attend_noalloc(cache.handle, layer, q.data_ptr(), qpos.data_ptr(), q.shape[0], out.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("precision", [rkv.RKV_PRECISE, rkv.RKV_FAST])
def test_noalloc_attention_equals_cache_attend(precision):
    require_gpu()
    cfg = ATTEND  # 12 heads x 128, 5,788 slots, 2% outliers x8
    cache = rkv.RingCache(2, cfg.n_slots, cfg.n_heads, cfg.head_dim, 757, precision, device=DEV)
    s = Stream(cfg)
    p0 = 0
    while p0 < 8888:  # layer 1: full ring, head at slot 3,100
        n = min(757, 8888 - p0)
        _, k, v = s.chunk(n)
        cache.write(1, to_dev(k), to_dev(v), pos_dev(positions(p0, n)))
        p0 += n
    for n_q, qp0 in ((757, 8131), (200, 8500)):  # the second call smaller
        q, _, _ = s.chunk(n_q)
        qd, qpos = to_dev(q), pos_dev(positions(qp0, n_q))
        want = cache.attend(1, qd, qpos)
        got = torch.full_like(want, float("nan"))
        _attend_noalloc(cache, 1, qd, qpos, got)
        torch.cuda.synchronize()
        print(f"n_q {n_q}: identical bits {torch.equal(got.view(torch.int16), want.view(torch.int16))}", flush=True)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), n_q


def test_noalloc_attention_on_a_wrapped_partial_cache_and_empty_layer():
    require_gpu()
    cfg = Config("noalloc_small", n_heads=3, head_dim=64, n_slots=500, chunk=0, seed=41,
                 outliers=OutlierSpec(0.02, 8.0))
    cache = rkv.RingCache(2, 500, 3, 64, 300, device=DEV)
    s = Stream(cfg)
    for n, p0 in ((300, 0), (350, 300)):  # wraps, 500 valid
        _, k, v = s.chunk(n)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(positions(p0, n)))
    for n_q in (300, 17):
        q, _, _ = s.chunk(n_q)
        qd, qpos = to_dev(q), pos_dev(positions(600, n_q))
        for layer in (0, 1):  # layer 1 is empty: zeros
            want = cache.attend(layer, qd, qpos)
            got = torch.full_like(want, float("nan"))
            _attend_noalloc(cache, layer, qd, qpos, got)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (n_q, layer)
        assert not got.float().abs().sum().item()


def test_noalloc_attention_over_globals_and_3d_ring_with_static_heads():
    """The paper's layout in small (global slots beside a 3-D RoPE ring), then
    with static scales: the fixed-scratch call gives cache_attend's bits."""
    require_gpu()
    from workloads import frame_positions
    bands = (22, 21, 21)
    cfg = Config("noalloc_g3d", n_heads=4, head_dim=128, n_slots=300, chunk=100, seed=43,
                 outliers=OutlierSpec(0.02, 8.0), n_global=90, bands=bands)
    cache = rkv.RingCache(1, 300, 4, 128, 100, device=DEV, n_global=90, rope_bands=bands)
    p3 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)
    s = Stream(cfg)
    _, k, v = s.chunk(90)
    cache.write_global(0, 0, to_dev(k), to_dev(v), p3(frame_positions(-1, 90, 10)))
    for t in range(4):  # 400 tokens into 300 ring slots: wraps
        _, k, v = s.chunk()
        cache.write(0, to_dev(k), to_dev(v), p3(frame_positions(t, 100, 10)))
    for static in (False, True):
        if static:
            cache.calibrate_static(0, 1.5)
        for n_q in (100, 33):
            q, _, _ = s.chunk(n_q)
            qd, qpos = to_dev(q), p3(frame_positions(3, n_q, 10))
            want = cache.attend(0, qd, qpos)
            got = torch.full_like(want, float("nan"))
            _attend_noalloc(cache, 0, qd, qpos, got)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (static, n_q)


def test_noalloc_rejects_a_workspace_beyond_the_fixed_scratch():
    require_gpu()
    # 96 heads x 1,024 queries: (768 + 512) units+workgroups x 34 KiB > 32 MiB
    cache = rkv.RingCache(1, 64, 96, 128, 1024, device=DEV)
    q = torch.zeros(1024, 96, 128, dtype=torch.bfloat16, device=DEV)
    qpos = torch.zeros(1024, dtype=torch.int32, device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(rkv.RkvError) as e:
        _attend_noalloc(cache, 0, q, qpos, out)
    assert e.value.code == rkv.RKV_EINVAL and "scratch" in rkv.rkv_last_error()
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing was enqueued
    _attend_noalloc(cache, 0, q[:100], qpos[:100], out[:100])  # a small call on the same cache works
    torch.cuda.synchronize()
    assert not out[:100].float().abs().sum().item()
