"""GPU parity of the fused pre-attention RMS norm (Runway Characters paper,
§4.4 "Fused pre-attention", Appendix G: RMS-normalize Q and K, then RoPE,
then quantize and write).  The oracle normalizes the exact bf16 inputs in
float64 (oracle.norm) and then runs its ordinary write and attention; the
device does the norm in fp32 inside the write and the query preparation.
Bars as for the plain path: bookkeeping bit-exact, every dequantized cache
element within 1 e4m3 ulp, attention within 2e-2 max / 2e-3 mean of the
sigma_v-normalized error."""
import numpy as np
import pytest
import torch

import fp8_ring_kv_amd as rkv
from oracle import attend as oatt, ring as oring
from oracle.bf16 import round_bf16
from oracle.norm import rms_norm
from tests.gpu_common import DEV, assert_cache_matches, attn_errors, pos_dev, readback, require_gpu, to_dev
from workloads import Config, OutlierSpec, Stream, bf16_bits_to_f64, f32_to_bf16_bits, positions

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def weights(d, seed):
    """bf16 norm weights around 1: (device tensor, exact float64 values)."""
    rng = np.random.default_rng(seed)
    bits = f32_to_bf16_bits((1.0 + 0.25 * rng.standard_normal(d)).astype(np.float32))
    dev = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    return dev, bf16_bits_to_f64(bits)


def gpu_out(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("head_dim", [128, 64])
def test_normed_writes_and_attention_match_oracle(head_dim):
    cfg = Config("norm", n_heads=4, head_dim=head_dim, n_slots=700, chunk=300, seed=21,
                 outliers=OutlierSpec(0.02, 8.0))
    cache = rkv.RingCache(1, cfg.n_slots, cfg.n_heads, cfg.head_dim, cfg.chunk, rkv.RKV_PRECISE, device=DEV)
    st = oring.RingState(cfg.n_slots, cfg.n_heads, cfg.head_dim)
    wq, wq64 = weights(head_dim, 1)
    wk, wk64 = weights(head_dim, 2)
    cache.set_qk_norm(0, wq, wk, EPS)
    s = Stream(cfg)
    for c in range(3):  # 900 tokens into 700 slots: the ring wraps
        _, k, v = s.chunk()
        pos = positions(cfg.chunk * c, cfg.chunk)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, rms_norm(k.f64, wk64, EPS), v.f64, pos)
        assert_cache_matches(cache, 0, st)
    q, _, _ = s.chunk()
    qpos = positions(cfg.chunk * 2, cfg.chunk)
    out = gpu_out(cache.attend(0, to_dev(q), pos_dev(qpos)))
    qn = rms_norm(q.f64, wq64, EPS)
    sig = oatt.sigma_v(st)
    for name, ref in (("emul", round_bf16(oatt.attend_emul(st, qn, qpos))), ("exact", oatt.attend_exact(st, qn, qpos))):
        rmax, rmean, nmax, nmean = attn_errors(out, ref, sig)
        assert nmax < 2e-2 and nmean < 2e-3, (name, rmax, rmean, nmax, nmean)
    # the norm really is applied: without it the oracle's output is far away
    plain = oatt.attend_exact(st, q.f64, qpos)
    assert attn_errors(out, plain, sig)[2] > 0.1


def test_write_attend_with_norm_equals_the_two_calls():
    cfg = Config("normfused", n_heads=6, head_dim=128, n_slots=900, chunk=256, seed=22)
    mk = lambda: rkv.RingCache(1, cfg.n_slots, cfg.n_heads, cfg.head_dim, cfg.chunk, rkv.RKV_PRECISE, device=DEV)
    fused, split = mk(), mk()
    wq, _ = weights(128, 3)
    wk, _ = weights(128, 4)
    for cch in (fused, split):
        cch.set_qk_norm(0, wq, wk, EPS)
    s = Stream(cfg)
    for c in range(4):
        q, k, v = s.chunk()
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        p = pos_dev(positions(cfg.chunk * c, cfg.chunk))
        a = fused.write_attend(0, kd, vd, p, qd, p)
        split.write(0, kd, vd, p)
        b = split.attend(0, qd, p)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), c
        for x, y in zip(fused.codes(0) + fused.scales(0), split.codes(0) + split.scales(0)):
            assert torch.equal(x, y), c


def test_norm_off_restores_the_plain_path():
    cfg = Config("normoff", n_heads=4, head_dim=128, n_slots=500, chunk=200, seed=23)
    mk = lambda: rkv.RingCache(2, cfg.n_slots, cfg.n_heads, cfg.head_dim, cfg.chunk, rkv.RKV_PRECISE, device=DEV)
    toggled, plain = mk(), mk()
    wq, _ = weights(128, 5)
    wk, _ = weights(128, 6)
    toggled.set_qk_norm(-1, wq, wk, EPS)  # every layer
    toggled.set_qk_norm(1, None, None)     # then off again for layer 1
    s = Stream(cfg)
    q, k, v = s.chunk()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    p = pos_dev(positions(0, cfg.chunk))
    for layer in (0, 1):
        toggled.write(0 + layer, kd, vd, p)
        plain.write(layer, kd, vd, p)
    a1, b1 = toggled.attend(1, qd, p), plain.attend(1, qd, p)
    a0, b0 = toggled.attend(0, qd, p), plain.attend(0, qd, p)
    torch.cuda.synchronize()
    assert torch.equal(a1.view(torch.int16), b1.view(torch.int16))  # layer 1: norm off, identical bits
    assert torch.equal(toggled.codes(1)[0], plain.codes(1)[0])
    assert not torch.equal(toggled.codes(0)[0], plain.codes(0)[0])  # layer 0: normalized keys
    assert not torch.equal(a0.view(torch.int16), b0.view(torch.int16))


def test_set_qk_norm_rejects_bad_arguments():
    cache = rkv.RingCache(2, 64, 2, 64, 16, device=DEV)
    wq, _ = weights(64, 7)
    L = rkv.lib()
    h, s = cache.handle, torch.cuda.current_stream().cuda_stream
    import ctypes
    vp = ctypes.c_void_p
    assert L.ring_cache_set_qk_norm(None, 0, vp(wq.data_ptr()), vp(wq.data_ptr()), 1e-6, vp(s)) == rkv.RKV_EINVAL
    assert L.ring_cache_set_qk_norm(vp(h), 2, vp(wq.data_ptr()), vp(wq.data_ptr()), 1e-6, vp(s)) == rkv.RKV_EINVAL
    assert L.ring_cache_set_qk_norm(vp(h), 0, vp(wq.data_ptr()), None, 1e-6, vp(s)) == rkv.RKV_EINVAL
    assert L.ring_cache_set_qk_norm(vp(h), 0, vp(wq.data_ptr()), vp(wq.data_ptr()), 0.0, vp(s)) == rkv.RKV_EINVAL
    assert L.ring_cache_set_qk_norm(vp(h), 0, vp(wq.data_ptr()), vp(wq.data_ptr()), float("inf"), vp(s)) == rkv.RKV_EINVAL
    assert L.ring_cache_set_qk_norm(vp(h), 0, vp(wq.data_ptr() + 1), vp(wq.data_ptr()), 1e-6, vp(s)) == rkv.RKV_EINVAL
    assert "aligned" in rkv.rkv_last_error()
    assert L.ring_cache_set_qk_norm(vp(h), -1, None, None, 1e-6, vp(s)) == rkv.RKV_OK
