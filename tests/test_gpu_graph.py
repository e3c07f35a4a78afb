"""HIP graph capture of the per-call work (write + attend) through the C ABI.

The device-side write position makes the calls capturable (Runway Characters
paper, §4.1 "A ring cache with a device-side write position"): a graph
recorded once must advance the ring on every replay exactly as eager calls
do.  Each replay is checked bit-exactly against an eager twin cache fed the
same inputs, with the program's own eager work and synchronizations between
replays.
"""
import numpy as np
import pytest
import torch

from tests.gpu_common import require_gpu, to_dev
from workloads import Config, Stream, positions

pytestmark = pytest.mark.gpu


def _pair(cfg, n_q, precision):
    import fp8_ring_kv_amd as rkv
    mk = lambda: rkv.RingCache(1, cfg.n_slots, cfg.n_heads, cfg.head_dim, n_q, precision,
                               device="cuda:0")
    return mk(), mk()


@pytest.mark.parametrize("precision", [0, 1])
def test_captured_write_attend_replays_match_eager(precision):
    require_gpu()
    cfg = Config("graph", n_heads=4, head_dim=128, n_slots=700, chunk=300, seed=11)
    eager, captured = _pair(cfg, cfg.chunk, precision)
    s = Stream(cfg)
    chunks = []
    for c in range(5):  # 1,500 tokens into 700 slots: the ring wraps twice
        q, k, v = s.chunk()
        chunks.append((to_dev(q), to_dev(k), to_dev(v),
                       torch.from_numpy(positions(cfg.chunk * c, cfg.chunk)).to("cuda:0")))
    qb, kb, vb, pb = (torch.empty_like(t) for t in chunks[0])
    out_g = torch.empty_like(qb)
    out_e = torch.empty_like(qb)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            captured.write(0, kb, vb, pb)
            captured.attend(0, qb, pb, out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture records work without running it: the captured cache is still empty
    assert captured.state(0)[:2].cpu().tolist() == [0, 0]

    for c, (q, k, v, p) in enumerate(chunks):
        for dst, src in ((qb, q), (kb, k), (vb, v), (pb, p)):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        eager.write(0, k, v, p)
        eager.attend(0, q, p, out_e)
        torch.cuda.synchronize()
        sg, se = captured.state(0)[:2].cpu().tolist(), eager.state(0)[:2].cpu().tolist()
        assert sg == se, (c, sg, se)
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"replay {c}: output differs"
        for a, b in zip(captured.codes(0) + captured.scales(0), eager.codes(0) + eager.scales(0)):
            assert torch.equal(a, b), f"replay {c}: cache differs"
        assert torch.equal(captured.slot_pos(0), eager.slot_pos(0))
    assert sg == [(5 * cfg.chunk) % cfg.n_slots, cfg.n_slots]


def test_captured_period_with_rotation_replays_match_eager():
    """A multi-step sequence in one graph, as a serving loop would record a
    reset period: a delta rotation, then three fused write+attend calls, each
    from its own input buffers.  Every replay must leave the cache, the ring
    state and the last output bit-identical to the same calls made eagerly."""
    require_gpu()
    import fp8_ring_kv_amd as rkv
    cfg = Config("graph_period", n_heads=6, head_dim=128, n_slots=900, chunk=256, seed=13)
    eager, captured = _pair(cfg, cfg.chunk, rkv.RKV_PRECISE)
    s = Stream(cfg)
    steps = []
    for c in range(3):
        q, k, v = s.chunk()
        steps.append((to_dev(q), to_dev(k), to_dev(v),
                      torch.from_numpy(positions(cfg.chunk * c, cfg.chunk)).to("cuda:0")))
    # fill both caches eagerly first so the first rotation has keys to rotate
    for cache in (eager, captured):
        for q, k, v, p in steps:
            cache.write(0, k, v, p)
    torch.cuda.synchronize()
    out_g = torch.empty_like(steps[0][0])
    out_e = torch.empty_like(steps[0][0])
    delta = -3 * cfg.chunk

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            captured.rotate(0, delta)
            for q, k, v, p in steps:
                captured.write_attend(0, k, v, p, q, p, out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        graph.replay()
        eager.rotate(0, delta)
        for q, k, v, p in steps:
            eager.write_attend(0, k, v, p, q, p, out_e)
        torch.cuda.synchronize()
        sg, se = captured.state(0)[:2].cpu().tolist(), eager.state(0)[:2].cpu().tolist()
        assert sg == se, (rep, sg, se)
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"replay {rep}: output differs"
        for a, b in zip(captured.codes(0) + captured.scales(0), eager.codes(0) + eager.scales(0)):
            assert torch.equal(a, b), f"replay {rep}: cache differs"
        assert torch.equal(captured.slot_pos(0), eager.slot_pos(0))
        assert torch.equal(captured.vmax(0), eager.vmax(0))
