"""The per-chunk sequence on 60 layer caches, captured as HIP graphs and
replayed across a position reset, against the oracle on every layer.

Runway Characters paper: one step runs 4 denoising passes x 60 blocks = 240
attention calls, each layer's cache written once per step and read by every
pass (§2 "The step budget", Appendix G); the write position lives on the
device so the whole step is recorded once and replayed (§4.1); every 42
steps all cached keys are rotated by the position change (§4.2, Appendix G);
bugs that only show under graph capture are why every call is tested there
(§8 "Lessons").

Shape: the per-chunk configuration's 60 layers and 4 passes, at a reduced
head and slot count (2 heads x 128, 600 slots, 128 new tokens per chunk, a
reset every 6 chunks) so that the oracle can follow every layer.  One chunk
(60 cache_write_attend calls for the first pass, then 180 cache_attend
calls) is one graph; the 60-layer rotation is a second graph.  Each replay
reads new inputs from the graphs' input buffers.  Checked on every layer:
every one of the 240 outputs of every chunk against exact attention on the
layer's dequantized device cache (N(0,1) data: raw and normalized gates)
and end to end against the layer's oracle session, the ring
state and slot positions bit-exact after every chunk, every cached element
within 1 e4m3 ulp before the reset, and the captured rotation in isolation
(every rotated key within 1 ulp of the oracle's rotation of the device's own
keys).
"""
import numpy as np
import pytest
import torch

import fp8_ring_kv_amd as rkv
from oracle import attend as oatt, ring as oring
from tests.gpu_common import assert_cache_matches, check_attention, check_rotated, require_gpu, state_from_device, to_dev
from workloads import Config, Stream

pytestmark = pytest.mark.gpu

LAYERS, PASSES, H, D, N, CHUNK, PERIOD, CHUNKS = 60, 4, 2, 128, 600, 128, 6, 9


def test_captured_chunks_across_a_reset_match_the_oracle_on_every_layer():
    require_gpu()
    dev = "cuda:0"
    cfg = Config("per_chunk_reduced", n_heads=H, head_dim=D, n_slots=N, chunk=CHUNK, seed=3, n_layers=LAYERS)
    cache = rkv.RingCache(LAYERS, N, H, D, CHUNK, rkv.RKV_PRECISE, device=dev)
    states = [oring.RingState(N, H, D) for _ in range(LAYERS)]
    streams = [Stream(cfg, seed=1000 + layer) for layer in range(LAYERS)]
    # graph input buffers: per layer k, v and the queries of the 4 passes; one
    # position buffer for the chunk; one output per call
    kb = torch.empty(LAYERS, CHUNK, H, D, dtype=torch.bfloat16, device=dev)
    vb = torch.empty_like(kb)
    qb = torch.empty(LAYERS, PASSES, CHUNK, H, D, dtype=torch.bfloat16, device=dev)
    pb = torch.empty(CHUNK, dtype=torch.int32, device=dev)
    ob = torch.empty(LAYERS, PASSES, CHUNK, H, D, dtype=torch.bfloat16, device=dev)

    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    chunk_graph, reset_graph = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(chunk_graph, stream=side):
            for pas in range(PASSES):
                for layer in range(LAYERS):
                    if pas == 0:
                        cache.write_attend(layer, kb[layer], vb[layer], pb, qb[layer, 0], pb, ob[layer, 0])
                    else:
                        cache.attend(layer, qb[layer, pas], pb, ob[layer, pas])
        with torch.cuda.graph(reset_graph, stream=side):
            cache.rotate(-1, -PERIOD * CHUNK)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    assert cache.state(0)[:2].cpu().tolist() == [0, 0]  # capture ran nothing

    for c in range(CHUNKS):
        if c == PERIOD:  # position reset before the chunk's writes
            pres = [state_from_device(cache, layer) for layer in range(LAYERS)]
            reset_graph.replay()
            torch.cuda.synchronize()
            for layer in range(LAYERS):
                check_rotated(cache, layer, pres[layer], -PERIOD * CHUNK)
                oring.rotate(states[layer], -PERIOD * CHUNK)
            print("reset: captured 60-layer rotation within 1 ulp on every layer", flush=True)
        pos = ((c % PERIOD) * CHUNK + np.arange(CHUNK)).astype(np.int32)
        qs = []
        for layer in range(LAYERS):
            q0, k, v = streams[layer].chunk()
            kb[layer].copy_(to_dev(k))
            vb[layer].copy_(to_dev(v))
            lq = [q0] + [streams[layer].chunk()[0] for _ in range(PASSES - 1)]
            for pas in range(PASSES):
                qb[layer, pas].copy_(to_dev(lq[pas]))
            oring.write(states[layer], k.f64, v.f64, pos)
            qs.append(lq)
        pb.copy_(torch.from_numpy(pos))
        torch.cuda.synchronize()
        chunk_graph.replay()
        torch.cuda.synchronize()
        out = ob.float().cpu().numpy().astype(np.float64)
        worst = np.zeros(4)
        for layer in range(LAYERS):
            st = states[layer]
            got_state = cache.state(layer)[:2].cpu().tolist()
            assert got_state == [st.head, st.n_valid], (c, layer, got_state)
            assert np.array_equal(cache.slot_pos(layer).cpu().numpy(), st.slot_pos), (c, layer)
            ds = state_from_device(cache, layer)
            for pas in range(PASSES):
                prim, e2e = check_attention(f"chunk {c} layer {layer} pass {pas}", cache, layer, st, qs[layer][pas].f64,
                                            pos, out[layer, pas], raw=True, ds=ds, quiet=True)
                worst = np.maximum(worst, [prim[0], prim[2], e2e[0], e2e[1]])
        print(f"chunk {c}: 60 writes + 240 attention calls replayed; worst vs exact on the device caches: raw max "
              f"{worst[0]:.2e}, normalized max {worst[1]:.2e}; end to end normalized max {worst[2]:.2e} "
              f"mean {worst[3]:.2e}", flush=True)
        if c == PERIOD - 1:
            for layer in range(LAYERS):
                assert_cache_matches(cache, layer, states[layer])
