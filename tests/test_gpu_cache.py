"""GPU parity of the ring write and the delta rotation against the oracle.

Contract (Runway Characters paper §4.1-§4.3, Appendix G, stated as a bar):
ring head, n_valid and every slot position bit-exact; every dequantized
K and V element within 1 e4m3 ulp of the oracle's.

Every rotation is checked twice: in isolation (rotate_checked: the oracle
rotates the device's own pre-rotation keys, and every rotated key element
must be within 1 ulp, with no exceptions), and end to end against the
oracle's own session, where the write's 1-ulp difference before the
rotation is carried through it.
"""
import numpy as np
import pytest
import torch

import fp8_ring_kv_amd as rkv
from oracle import e4m3, ring as oring
from tests.gpu_common import DEV, assert_cache_matches, pos_dev, readback, require_gpu, rotate_checked, to_dev
from workloads import TINY, WRITE_ROTATE, Bf16, Config, OutlierSpec, Stream, f32_to_bf16_bits, bf16_bits_to_f64, positions

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def new_pair(cfg: Config, max_q=64, precision=rkv.RKV_PRECISE, n_layers=1):
    cache = rkv.RingCache(n_layers, cfg.n_slots, cfg.n_heads, cfg.head_dim, max_q, precision,
                          cfg.rope_base, 1.0, device=DEV)
    st = oring.RingState(cfg.n_slots, cfg.n_heads, cfg.head_dim, cfg.rope_base)
    return cache, st


def test_tiny_session_writes_then_reset():
    cache, st = new_pair(TINY)
    s = Stream(TINY)
    for c in range(6):
        _, k, v = s.chunk()
        pos = positions(16 * c, 16)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
        assert_cache_matches(cache, 0, st)
    assert (st.head, st.n_valid) == (32, 64)
    pre = st.copy()
    rotate_checked(cache, 0, -80)
    oring.rotate(st, -80)
    assert_cache_matches(cache, 0, st, pre=pre)


def test_hardware_e4m3_rounding_is_nearest_even_on_every_midpoint():
    """V rows [448, midpoints...] have scale exactly 1, so the stored codes are the
    hardware conversion of the midpoints themselves; they must equal RNE codes."""
    tab = e4m3.decode_table()[:0x7F]
    vals = tab[np.isfinite(tab)]
    mids = (vals[:-1] + vals[1:]) / 2  # 125 positive midpoints, exact in bf16
    cands = np.concatenate([mids, -mids, vals, -vals, [446.0, -446.0]])
    n_rows = int(np.ceil(len(cands) / 127))
    rows = np.zeros((n_rows, 128), dtype=np.float64)
    flat = np.zeros(n_rows * 127)
    flat[: len(cands)] = cands
    rows[:, 0] = 448.0
    rows[:, 1:] = np.clip(flat.reshape(n_rows, 127), -448, 448)
    v_bits = f32_to_bf16_bits(rows.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f64(v_bits), rows)  # representable exactly
    cfg = Config("mid", n_heads=1, head_dim=128, n_slots=64, chunk=n_rows, seed=0)
    cache, st = new_pair(cfg)
    v = Bf16(v_bits.reshape(n_rows, 1, 128), rows.reshape(n_rows, 1, 128))
    k = v
    cache.write(0, to_dev(k), to_dev(v), pos_dev(np.zeros(n_rows, dtype=np.int32)))
    (_, _, _, cv, _, sv) = readback(cache, 0)
    assert np.all(sv[0, :n_rows] == 1.0)
    want = e4m3.encode(rows)
    got = cv[0, :n_rows]
    zero = (want & 0x7F) == 0  # +0 and -0 decode alike; the sign of zero is not kept
    assert np.array_equal(got[~zero], want[~zero]) and np.all((got[zero] & 0x7F) == 0)


@pytest.mark.parametrize("margin", [1.0, 1.5])
def test_value_codes_and_scales_bit_exact(margin):
    """Values are bf16 and their amax times the margin is exact for margins 1
    and 1.5, so the stored value scales equal the oracle's fp32(margin amax /
    448) and every value code is the exact quotient's RNE code, ties included
    (outlier channels x8 put many quotients next to e4m3 midpoints)."""
    cfg = Config("vexact", n_heads=4, head_dim=128, n_slots=700, chunk=500, seed=11,
                 outliers=OutlierSpec(0.05, 8.0))
    cache = rkv.RingCache(1, cfg.n_slots, cfg.n_heads, cfg.head_dim, 64, rkv.RKV_PRECISE,
                          cfg.rope_base, margin, device=DEV)
    st = oring.RingState(cfg.n_slots, cfg.n_heads, cfg.head_dim, cfg.rope_base, margin)
    s = Stream(cfg)
    for c in range(3):  # 1,500 tokens into 700 slots: every slot rewritten, the ring wraps
        _, k, v = s.chunk()
        pos = positions(500 * c, 500)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
    (head, nv), _, _, cv, _, sv = readback(cache, 0)
    assert (head, nv) == (st.head, st.n_valid)
    assert np.array_equal(sv[:, : cfg.n_slots], st.scale_v)
    got, want = cv[:, : cfg.n_slots], st.codes_v
    zero = (want & 0x7F) == 0  # the sign of a zero code is not kept
    assert np.array_equal(got[~zero], want[~zero]) and np.all((got[zero] & 0x7F) == 0)


def test_large_writes_take_two_level_tickets():
    """A 2,000-token write at 12 heads is 762 workgroups, above the 512 that
    count their tickets on one counter: the ring position must still advance
    exactly once per call, with every counter back at zero, before and after
    a small write that uses the single counter.  A 4,000-token write is 1,512
    work items for 1,024 workgroups: some take two, loading the second while
    they store the first (and it wraps the ring)."""
    cfg = Config("bigwrite", n_heads=12, head_dim=128, n_slots=4100, chunk=0, seed=12,
                 outliers=OutlierSpec(0.02, 8.0))
    cache, st = new_pair(cfg)
    s = Stream(cfg)
    p0 = 0
    for n in (2000, 300, 2000, 4000):
        _, k, v = s.chunk(n)
        pos = positions(p0, n)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
        p0 += n
        assert_cache_matches(cache, 0, st)


def test_writes_across_the_heads_per_item_switch():
    """A write takes one head per work item while its items (16-slot groups
    met, n/16 + 2, times heads) fit 1,024 workgroups, two heads per item
    beyond: at 12 heads 1,328 tokens are 85 x 12 = 1,020 one-head items and
    1,344 tokens 86 x 6 = 516 two-head items.  Both sides, at ring offsets
    that leave partial groups at each end and wrap, bit-checked."""
    cfg = Config("hgswitch", n_heads=12, head_dim=128, n_slots=3000, chunk=0, seed=21,
                 outliers=OutlierSpec(0.02, 8.0))
    cache, st = new_pair(cfg)
    s = Stream(cfg)
    p0 = 0
    for n in (7, 1328, 1344, 1344, 1328):
        _, k, v = s.chunk(n)
        pos = positions(p0, n)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
        p0 += n
        assert_cache_matches(cache, 0, st)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_wrapping_writes_of_varied_sizes(head_dim):
    """Random write sizes (1 .. N, including a full-ring write) wrap the ring many times."""
    cfg = Config("vary", n_heads=3, head_dim=head_dim, n_slots=300, chunk=0, seed=5,
                 outliers=OutlierSpec(0.05, 8.0))
    cache, st = new_pair(cfg)
    s = Stream(cfg)
    rng = np.random.default_rng(17)
    p0 = 0
    for n in [1, 299, 300, 17, 16, 15, 64, 65, 250, 3, 128, 300, 1]:
        _, k, v = s.chunk(n)
        pos = positions(p0, n)
        p0 += n + int(rng.integers(0, 5))
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
        assert_cache_matches(cache, 0, st)
    pre = st.copy()
    rotate_checked(cache, 0, -1234)
    oring.rotate(st, -1234)
    assert_cache_matches(cache, 0, st, pre=pre)


def test_partial_fill_rotate_touches_valid_slots_only():
    cfg = Config("partial", n_heads=2, head_dim=128, n_slots=1000, chunk=0, seed=6)
    cache, st = new_pair(cfg)
    s = Stream(cfg)
    _, k, v = s.chunk(333)
    pos = positions(50, 333)
    cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
    oring.write(st, k.f64, v.f64, pos)
    before = readback(cache, 0)
    pre = st.copy()
    rotate_checked(cache, 0, 77)
    oring.rotate(st, 77)
    assert_cache_matches(cache, 0, st, pre=pre)
    after = readback(cache, 0)
    assert np.array_equal(after[1][333:], before[1][333:])  # slot_pos outside the valid range
    assert np.array_equal(after[2][:, 333:], before[2][:, 333:])  # K codes outside


def test_reset_empties_the_ring():
    cache, st = new_pair(TINY)
    s = Stream(TINY)
    _, k, v = s.chunk()
    cache.write(0, to_dev(k), to_dev(v), pos_dev(positions(0, 16)))
    cache.reset(0)
    (hv, sp, *_rest) = readback(cache, 0)
    assert hv == (0, 0) and not sp.any()


def test_write_rotate_workload_full_size():
    """42 writes of 757 tokens (12 heads x 128) into 5,788 slots, then a reset by -42*757."""
    cfg = WRITE_ROTATE
    cache, st = new_pair(cfg)
    s = Stream(cfg)
    for c in range(42):
        _, k, v = s.chunk()
        pos = positions(757 * c, 757)
        cache.write(0, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
        if c in (0, 7, 41):
            assert_cache_matches(cache, 0, st)
    d = -42 * 757
    pre = st.copy()
    rotate_checked(cache, 0, d)
    oring.rotate(st, d)
    stats = assert_cache_matches(cache, 0, st, pre=pre)
    print("codes equal to the oracle's:", stats)
    assert stats["k_codes_equal"] > 0.999 and stats["v_codes_equal"] > 0.99999


def test_rotate_all_layers_in_one_launch():
    cfg = Config("layers", n_heads=2, head_dim=128, n_slots=200, chunk=0, seed=8)
    cache, _ = new_pair(cfg, n_layers=3)
    states = []
    s = Stream(cfg)
    for layer in range(3):
        st = oring.RingState(cfg.n_slots, cfg.n_heads, cfg.head_dim)
        n = [50, 200, 130][layer]
        _, k, v = s.chunk(n)
        pos = positions(10 * layer, n)
        cache.write(layer, to_dev(k), to_dev(v), pos_dev(pos))
        oring.write(st, k.f64, v.f64, pos)
        states.append(st)
    rotate_checked(cache, -1, -9)
    for layer, st in enumerate(states):
        pre = st.copy()
        oring.rotate(st, -9)
        assert_cache_matches(cache, layer, st, pre=pre)


def test_invalid_calls_raise():
    cache, _ = new_pair(TINY)
    k = torch.zeros(65, 1, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rkv.RkvError):
        cache.write(0, k, k, torch.zeros(65, dtype=torch.int32, device=DEV))  # n > N
    with pytest.raises(rkv.RkvError):
        cache.write(1, k[:4], k[:4], torch.zeros(4, dtype=torch.int32, device=DEV))  # layer
    with pytest.raises(rkv.RkvError):
        cache.rotate(5, 1)
