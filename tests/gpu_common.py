"""Helpers for the GPU parity tests: device setup, readback, and the contract
checks against the oracle (bit-exact bookkeeping, 1 e4m3 ulp per
dequantized cache element, attention error gates)."""
from __future__ import annotations

import numpy as np
import torch

import fp8_ring_kv_amd as rkv
from oracle import e4m3
from workloads import Bf16

DEV = "cuda:0"


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    rkv.lib()  # fails loudly if the library is missing


def to_dev(x: Bf16) -> torch.Tensor:
    """bf16 bits -> device bf16 tensor."""
    t = torch.from_numpy(x.bits.view(np.int16).copy())
    return t.view(torch.bfloat16).to(DEV)


def pos_dev(p: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.asarray(p, dtype=np.int32)).to(DEV)


def readback(cache: rkv.RingCache, layer: int):
    """Host copies of (head, n_valid), slot_pos, codes_k, codes_v, scale_k, scale_v."""
    torch.cuda.synchronize()
    st = cache.state(layer).cpu().numpy()
    sp = cache.slot_pos(layer).cpu().numpy().astype(np.int64)
    ck, cv = cache.codes(layer)
    sk, sv = cache.scales(layer)
    return ((int(st[0]), int(st[1])), sp, ck.cpu().numpy(), cv.cpu().numpy(),
            sk.cpu().numpy().astype(np.float64), sv.cpu().numpy().astype(np.float64))


def within_one_ulp(cg, sg, co, so, extra=None):
    """Per element |c_g s_g - c_o s_o| <= s_o ulp(max |c|) (1 + 2^-20) (+ fp32 scale slack).

    ``extra`` widens the bound per element.  Returns the boolean mask of
    violations and the worst ratio err / bound.
    """
    dg = e4m3.decode(cg)
    do = e4m3.decode(co)
    vg = dg * sg[..., None]
    vo = do * so[..., None]
    big = np.where(np.abs(dg) >= np.abs(do), cg, co)
    bound = so[..., None] * e4m3.ulp_at(big) * (1 + 2 ** -20) + np.abs(vo) * 2 ** -21 + 1e-30
    if extra is not None:
        bound = bound + extra
    err = np.abs(vg - vo)
    bad = err > bound
    return bad, float(np.max(err / bound)) if err.size else 0.0


def pair_ulp_bound(codes, scale):
    """s * ||(ulp(c_2j), ulp(c_2j+1))|| per element: the largest difference a pair
    can carry through a rotation when each element was allowed 1 ulp before it."""
    u = e4m3.ulp_at(codes)
    pn = np.sqrt(u[..., 0::2] ** 2 + u[..., 1::2] ** 2)
    return np.repeat(pn, 2, axis=-1) * scale[..., None]


def assert_cache_matches(cache, layer, st, slots=None, check_v=True, pre=None):
    """Bit-exact head/n_valid/slot_pos; K (and V) within 1 ulp on valid slots.

    With ``pre`` (the oracle state before a delta rotation), rotated keys may
    also carry the rotated image of the 1-ulp difference allowed before the
    rotation; at most 0.1% of them may exceed the plain 1-ulp bound.
    """
    from oracle import ring as oring
    (head, nv), sp, ck, cv, sk, sv = readback(cache, layer)
    assert (head, nv) == (st.head, st.n_valid), ((head, nv), (st.head, st.n_valid))
    # the write kernel's internal counters are back at zero after every call
    counters = cache.write_counters(layer).cpu().numpy()
    assert len(counters) == 10 and not counters.any(), counters
    # the per-head value-scale bound equals the oracle's (fp32 values)
    vmax = cache.vmax(layer).cpu().numpy().astype(np.float64)
    assert np.array_equal(vmax, st.vmax), (vmax, st.vmax)
    valid = oring.valid_slots(st) if slots is None else slots
    assert np.array_equal(sp[valid], st.slot_pos[valid])
    extra = None
    if pre is not None:
        extra = pair_ulp_bound(pre.codes_k[:, valid], pre.scale_k[:, valid])
        strict, _ = within_one_ulp(ck[:, valid], sk[:, valid], st.codes_k[:, valid], st.scale_k[:, valid])
        assert strict.mean() <= 1e-3, f"K: {strict.mean():.2e} of elements beyond 1 ulp after rotation"
    bad, worst = within_one_ulp(ck[:, valid], sk[:, valid], st.codes_k[:, valid], st.scale_k[:, valid], extra)
    assert not bad.any(), f"K: {int(bad.sum())} elements beyond the bound (worst ratio {worst:.3f})"
    if check_v:
        bad, worst = within_one_ulp(cv[:, valid], sv[:, valid], st.codes_v[:, valid], st.scale_v[:, valid])
        assert not bad.any(), f"V: {int(bad.sum())} elements beyond 1 ulp (worst ratio {worst:.3f})"
    return dict(k_codes_equal=float(np.mean(ck[:, valid] == st.codes_k[:, valid])),
                v_codes_equal=float(np.mean(cv[:, valid] == st.codes_v[:, valid])))


def attn_errors(gpu: np.ndarray, ref: np.ndarray, sigma: np.ndarray):
    """(raw max, raw mean, normalized max, normalized mean) of |gpu - ref|.

    Normalized: divided by max(1, sigma_v[head, channel]), the RMS of the
    dequantized values in that output channel.
    """
    e = np.abs(gpu - ref)
    en = e / np.maximum(1.0, sigma)[None]
    return float(e.max()), float(e.mean()), float(en.max()), float(en.mean())
