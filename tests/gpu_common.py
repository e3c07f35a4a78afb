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
    """Host copies of (head, n_valid), slot_pos, codes_k, codes_v, scale_k, scale_v
    (slot axes in canonical order: the ring's slots, then the global slots)."""
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


def state_from_device(cache: rkv.RingCache, layer: int):
    """The device cache of `layer` as an oracle RingState (codes, scales,
    positions, ring state, value-scale bound and, once calibrated, the static
    scales), so an oracle operation can start from exactly what the device
    holds."""
    from oracle import ring as oring
    (head, nv), sp, ck, cv, sk, sv = readback(cache, layer)
    three_d = cache.pos_width == 3
    st = oring.RingState(cache.n_slots, cache.n_heads, cache.head_dim, rope_base=cache.params.rope_base,
                         margin=cache.params.scale_margin, head=head, n_valid=nv,
                         slot_pos=sp.copy(), codes_k=ck.copy(), codes_v=cv.copy(), scale_k=sk.copy(),
                         scale_v=sv.copy(), vmax=cache.vmax(layer).cpu().numpy().astype(np.float64),
                         n_global=cache.n_global, g_valid=int(cache.state(layer)[3].item()),
                         bands=cache.rope_bands if three_d else None,
                         slot_yx=cache.slot_yx(layer).cpu().numpy().astype(np.int64) if three_d else None)
    if cache.static_flag(layer):
        stat = cache.static_scales(layer).cpu().numpy().astype(np.float64)
        st.static_k, st.static_v = stat[0].copy(), stat[1].copy()
    return st


def check_rotated(cache: rkv.RingCache, layer: int, pre, delta: int):
    """After a delta rotation of `layer` on the device: the oracle rotates
    `pre` (the device's own state before the rotation, from
    state_from_device), and every valid dequantized key of the device must be
    within 1 e4m3 ulp of the oracle's (no exceptions), slot positions and
    ring state bit-exact, values and value scales untouched.  Returns the
    oracle's rotated state."""
    from oracle import ring as oring
    want = pre.copy()
    oring.rotate(want, delta)
    (head, nv), sp, ck, cv, sk, sv = readback(cache, layer)
    assert (head, nv) == (want.head, want.n_valid), (layer, head, nv)
    assert np.array_equal(sp, want.slot_pos), f"layer {layer}: slot positions"
    assert np.array_equal(cv, pre.codes_v) and np.array_equal(sv, pre.scale_v), f"layer {layer}: values touched"
    valid = oring.valid_slots(want)
    bad, worst = within_one_ulp(ck[:, valid], sk[:, valid], want.codes_k[:, valid], want.scale_k[:, valid])
    assert not bad.any(), (f"layer {layer}: {int(bad.sum())} of {bad.size} rotated key elements beyond 1 e4m3 ulp "
                           f"of the oracle's rotation of the device's own keys (worst ratio {worst:.3f})")
    return want


def rotate_checked(cache: rkv.RingCache, layer: int, delta: int):
    """Delta rotation of `layer` (-1: every layer) on the device, checked in
    isolation against the oracle's rotation of the device's own pre-rotation
    state (check_rotated).  Returns the oracle states it compared against."""
    layers = range(cache.n_layers) if layer == -1 else [layer]
    pres = [state_from_device(cache, l) for l in layers]
    cache.rotate(layer, delta)
    return [check_rotated(cache, l, pre, delta) for l, pre in zip(layers, pres)]


def assert_cache_matches(cache, layer, st, slots=None, check_v=True, pre=None):
    """Bit-exact head/n_valid/slot_pos; K (and V) within 1 ulp on valid slots.

    With ``pre`` (the oracle state before a delta rotation), rotated keys may
    also carry the rotated image of the 1-ulp difference allowed before the
    rotation; at most 0.1% of them may exceed the plain 1-ulp bound.
    """
    from oracle import ring as oring
    (head, nv), sp, ck, cv, sk, sv = readback(cache, layer)
    assert (head, nv) == (st.head, st.n_valid), ((head, nv), (st.head, st.n_valid))
    assert int(cache.state(layer)[3].item()) == st.g_valid, (int(cache.state(layer)[3].item()), st.g_valid)
    # the write kernel's internal counters are back at zero after every call
    counters = cache.write_counters(layer).cpu().numpy()
    assert len(counters) == 9 and not counters.any(), counters
    # the per-head value-scale bound equals the oracle's (fp32 values)
    vmax = cache.vmax(layer).cpu().numpy().astype(np.float64)
    assert np.array_equal(vmax, st.vmax), (vmax, st.vmax)
    valid = oring.valid_slots(st) if slots is None else slots
    assert np.array_equal(sp[valid], st.slot_pos[valid])
    if st.bands is not None:
        yx = cache.slot_yx(layer).cpu().numpy().astype(np.int64)
        assert np.array_equal(yx[valid], st.slot_yx[valid])
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


def gate(name, gpu, ref, sigma, max_tol=2e-2, mean_tol=2e-3, raw=False, quiet=False):
    """Attention gate: the error divided by max(1, sigma_v) within max_tol /
    mean_tol (and the raw error too when `raw`); raw and normalized errors
    are printed and carried in the assertion message either way."""
    rmax, rmean, nmax, nmean = attn_errors(gpu, ref, sigma)
    msg = f"{name}: raw max {rmax:.2e} mean {rmean:.2e} | normalized max {nmax:.2e} mean {nmean:.2e}"
    if not quiet:
        print(msg, flush=True)
    assert nmax < max_tol and nmean < mean_tol, msg
    if raw:
        assert rmax < max_tol and rmean < mean_tol, msg + " (raw gate)"
    return rmax, rmean, nmax, nmean


def attn_errors(gpu: np.ndarray, ref: np.ndarray, sigma: np.ndarray):
    """(raw max, raw mean, normalized max, normalized mean) of |gpu - ref|.

    Normalized: divided by max(1, sigma_v[head, channel]), the RMS of the
    dequantized values in that output channel.
    """
    e = np.abs(gpu - ref)
    en = e / np.maximum(1.0, sigma)[None]
    return float(e.max()), float(e.mean()), float(en.max()), float(en.mean())


def check_attention(name, cache, layer, st, q, q_pos, out, raw=False, fast=False, ds=None, quiet=False):
    """The attention gates of one call.

    1. Primary: the device output against exact float64 attention over the
       device's own dequantized cache (state_from_device): errors divided by
       max(1, sigma_v) within 2e-2 max / 2e-3 mean, raw too when `raw`.  (Fast
       mode is gated here only when `raw`: its single-term numerics miss the
       bounds on outlier caches; it is held to its emulation below.)
    2. The kernel's declared numerics (attend_emul: three query terms and two
       probability terms, or one of each in fast mode) on the same cache, same
       bounds.
    3. End to end against the oracle's own session `st`: every cached element
       may differ from the device's by 1 e4m3 ulp, which moves exact attention
       itself (a near-tie key code in an outlier channel that rounds the other
       way changes a dominant score); the device output may differ from the
       oracle's exact attention by that movement plus the 2e-2 / 2e-3 bounds,
       element by element.
    `ds`: the device state when the caller already read it back.  Returns the
    error tuples (device-state exact, end-to-end)."""
    from oracle import attend as oatt
    from oracle.bf16 import round_bf16
    if ds is None:
        ds = state_from_device(cache, layer)
    sig = oatt.sigma_v(ds)
    ex_d = oatt.attend_exact(ds, q, q_pos)
    prim = None
    if not fast or raw:
        prim = gate(f"{name} vs exact on the device cache", out, ex_d, sig, raw=raw, quiet=quiet)
    qt, pt = (1, 1) if fast else (3, 2)
    gate(f"{name} vs emul(q {qt}, p {pt}) on the device cache", out,
         round_bf16(oatt.attend_emul(ds, q, q_pos, qt, pt)), sig, quiet=quiet)
    if st is None:
        return prim, None
    ex_o = oatt.attend_exact(st, q, q_pos)
    norm = np.maximum(1.0, sig)[None]
    e2e = np.abs(out - ex_o) / norm
    move = np.abs(ex_d - ex_o) / norm
    msg = (f"{name} end to end vs the oracle's session: normalized max {e2e.max():.2e} mean {e2e.mean():.2e}; "
           f"exact attention moved by the cache's 1-ulp differences: max {move.max():.2e} mean {move.mean():.2e}")
    if not quiet:
        print(msg, flush=True)
    if not fast or raw:
        assert np.all(e2e <= move + 2e-2) and e2e.mean() <= move.mean() + 2e-3, msg
    return prim, (float(e2e.max()), float(e2e.mean()))
