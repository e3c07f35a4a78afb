"""Benchmark of the write-time FP8 ring KV hot path on one MI355X.

One step is the per-call cache work of a block forward in the pages'
workload (Runway Characters paper, §2 "The step budget", §4, Appendix G):
write the 757 new tokens of the chunk into the 5,788-slot ring (RoPE + FP8
quantization fused), then attend the chunk's 757 queries over every slot,
12 heads x 128 (one GPU's head share) -- one cache_write_attend call, which
prepares the queries in the write's launch.  Every 42nd step is preceded by the
position reset: a delta rotation of every cached key by -42 * 757.  The
cache starts full with its ring head at slot 3,100 (8,888 tokens written).

Prints one JSON line.  `value` is microseconds per step (one write of 757
tokens plus one attention call of 757 queries; the position reset, once per
42 steps, is timed on its own and reported as `components.rotate_1layer_us`
and its 42-step share `components.reset_share_us_per_step`).  The warm-up
steps (2,000 by default, ~100 ms) bring the GPU to its sustained clock: the
first tens of milliseconds of work after idle run up to 15% slower.  The
steps then run with eager launches (`components.eager_us_per_step`); the
same number of steps is captured as one HIP graph (the device-side write
position makes every call capturable), replayed 10 times untimed (the GPU
idles for ~20 ms while the graph is captured, and takes ~7 replays to return
to its clock) and once timed, and `value` is the replayed time (`launch`
says which; --no-graph reports the eager one).  Per-operation times come from separate HIP-event-timed loops
on the launch stream; `roofline` is the attention call (the dominant cost)
against the dense FP8 matrix peak.  `cpu_baseline` times the NumPy float64
oracle on the same work, median of 5.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H, D, N, CHUNK, RESET_EVERY = 12, 128, 5788, 757, 42
ATTN_FLOP = 4.0 * CHUNK * N * H * D  # QK^T and PV, 2 flops per multiply-add
STRESS_FLOP = 4.0 * CHUNK * 11576 * 48 * D  # the stress shape: 48 heads, 11,576 slots
STRESS_WRITE_BYTES = (6 * 48 * D + 8 * 48 + 4) * CHUNK  # one 757-token write at 48 heads
FULL_WRITE_BYTES = (6 * H * D + 8 * H + 4) * N  # one write of 5,788 tokens at 12 heads
WRITE_BYTES = (6 * H * D + 8 * H + 4) * CHUNK  # bf16 K,V in; e4m3 K,V + 2 scales + pos out
ROTATE_BYTES = (2 * H * D + 8 * H + 8) * N  # codes r/w, scale r/w, position r/w
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=84)
    ap.add_argument("--warmup", type=int, default=2000,
                    help="untimed steps first (the GPU's clock ramps up over the first tens of ms of work)")
    ap.add_argument("--precision", choices=["precise", "fast"], default="precise")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--attend-components-only", action="store_true",
                    help="of the per-operation loops, run only the attention call's (counter runs)")
    ap.add_argument("--reps", type=int, default=200, help="launches per component loop")
    ap.add_argument("--workgroups", type=int, default=0,
                    help="persistent workgroups per attention call (0 = one per compute unit)")
    ap.add_argument("--no-graph", action="store_true",
                    help="report the eager launches as value (no HIP-graph capture and replay)")
    ap.add_argument("--upkeep-only", action="store_true",
                    help="run only a few launches of the cache-upkeep kernels at their bandwidth shapes "
                         "(60-layer rotation, a whole-ring write, the 48-head write) and exit: "
                         "the command that the byte counters of those kernels are taken on")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the steps, run one plain copy kernel over this many MiB "
                         "(fp32 negation, read + write): the reference for HBM byte counters")
    return ap.parse_args()


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attend_757x5788_h12_hbm_traffic.md")
COUNTER_RECORD = os.path.join(ROOT, "profiles", "attend_757x5788_h12_counters.md")
ATTEND_SOURCES = ["k_attend.hip", "rkv_device.h", "rkv_launch.h"]


def attend_source_digest():
    import hashlib
    h = hashlib.sha256()
    for name in ATTEND_SOURCES:
        with open(os.path.join(ROOT, "fp8_ring_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_value(path, key):
    """A per-call figure from a committed counter record (profiles/), or None when
    the record is absent or was taken on different attention sources."""
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip().strip("`")
        if line.startswith("sources_sha256:") or line.startswith(key + ":"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if fields.get("sources_sha256") != attend_source_digest() or key not in fields:
        return None
    return float(fields[key])


def recorded_traffic():
    """HBM bytes per attention call (both kernels), from the byte-counter record."""
    return recorded_value(TRAFFIC_RECORD, "hbm_bytes_per_call")


def to_dev(x):
    """bf16 bit patterns (workloads.Bf16) -> device bf16 tensor."""
    import torch
    return torch.from_numpy(x.bits.view(np.int16).copy()).view(torch.bfloat16).to("cuda:0")


def timed(fn, reps, stream):
    """Average milliseconds of fn() over `reps` launches, bracketed by events on `stream`."""
    import torch
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / reps


def cpu_baseline(runs=5):
    """The oracle on the host cores, on the work of one step: one 757-token
    write (12 heads), the attention of the 757 queries over the full
    5,788-slot cache on all 12 heads, and one full-cache rotation (the reset,
    once per 42 steps, reported apart).  Median of `runs` runs after one
    warm-up, on the cache the bench's own writes produce."""
    import statistics
    import numpy
    from threadpoolctl import threadpool_info
    from oracle import attend as oatt, ring as oring
    from workloads import ATTEND, Stream, positions
    st = oring.RingState(N, H, D)
    s = Stream(ATTEND)
    p0 = 0
    while p0 < 8888:
        n = min(CHUNK, 8888 - p0)
        _, k, v = s.chunk(n)
        oring.write(st, k.f64, v.f64, positions(p0, n))
        p0 += n
    q, k, v = s.chunk()
    pos = positions(8888, CHUNK)
    parts = {"write": [], "attend": [], "rotate": []}
    for r in range(runs + 1):
        w = st.copy()
        t0 = time.perf_counter()
        oring.write(w, k.f64, v.f64, pos)
        t1 = time.perf_counter()
        oatt.attend_exact(w, q.f64, pos)
        t2 = time.perf_counter()
        oring.rotate(w, -RESET_EVERY * CHUNK)
        t3 = time.perf_counter()
        if r:  # the first run warms up
            parts["write"].append(t1 - t0)
            parts["attend"].append(t2 - t1)
            parts["rotate"].append(t3 - t2)
    med = {k2: statistics.median(v2) for k2, v2 in parts.items()}
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": (med["write"] + med["attend"]) * 1e6,
        "unit": "us per step",
        "cores": int(threads),
        "kind": "oracle",
        "sample": ("NumPy float64 oracle on the host, the work of one step: one 757-token write (12 heads) "
                   "and attend_exact of 757 queries over the full 5,788-slot cache, all 12 heads; "
                   f"median of {runs} runs after a warm-up (the full-cache rotation, once per 42 steps, "
                   "in parts_s)"),
        "parts_s": {k2: round(v2, 5) for k2, v2 in med.items()},
        "host_cpus": os.cpu_count(),
        "numpy": numpy.__version__,
    }


def measured_peaks(stream):
    """The two ceilings measured on this device with the library's probes
    (librkv_probe.so), reported beside the published peaks: dense FP8
    matrix throughput of the attention's instruction, and the HBM bandwidth
    of an in-place streaming read-modify-write (the rotation's pattern) over
    1 GiB, far beyond the 256 MB last-level cache (best of three timings)."""
    import torch
    from fp8_ring_kv_amd import probe as rkv
    s = stream.cuda_stream
    wg, iters = 2048, 2000
    sink = torch.empty(wg, dtype=torch.float32, device="cuda:0")
    rkv.rkv_probe_fp8_mfma(wg, 10, sink.data_ptr(), s)  # warm-up (code load)
    ms = timed(lambda: rkv.rkv_probe_fp8_mfma(wg, iters, sink.data_ptr(), s), 5, stream)
    mfma_tflops = wg * 4 * iters * 4 * 131072 / ms / 1e9
    nbytes = 1 << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")
    rkv.rkv_probe_stream(buf.data_ptr(), nbytes, s)  # warm-up
    ms = min(timed(lambda: rkv.rkv_probe_stream(buf.data_ptr(), nbytes, s), 4, stream) for _ in range(3))
    del buf, sink
    return {"fp8_mfma_TFLOPs": round(mfma_tflops, 1), "hbm_stream_GBps": round(2 * nbytes / ms / 1e6, 1),
            "probes": "rkv_probe_fp8_mfma (2048 x 4 waves x 2000 x 4 instructions 32x32x64 e4m3), "
                      "rkv_probe_stream (in-place read-modify-write of 1 GiB, 2 GiB moved)"}


def capture_steps(cache, pool, pos_pool, out, first, steps):
    """`steps` consecutive steps (from step index `first`) captured as ONE HIP
    graph: the same calls as the eager steps, one graph launch for all of
    them.  The device-side write position is what makes the calls
    capturable; each replay advances the ring as the eager calls would."""
    import torch
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(first, first + steps):
                j = i % RESET_EVERY
                q, k, v = pool[j]
                cache.write_attend(0, k, v, pos_pool[j], q, pos_pool[j], out)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    return g


def upkeep_only(args, rkv, pool, pos_pool, prec, dev):
    """A few launches of each cache-upkeep kernel at its bandwidth shape: the
    60-layer rotation (2 launches), a whole-ring write of 5,788 tokens x 12
    heads (3 launches) and the 48-head 757-token write (3 launches)."""
    import torch
    big = rkv.RingCache(60, N, H, D, CHUNK, prec, device=dev)
    for layer in range(60):
        for c in range(8):
            q, k, v = pool[(layer + c) % RESET_EVERY]
            big.write(layer, k, v, pos_pool[c])
    torch.cuda.synchronize()
    for d in (1, -1):
        big.rotate(-1, d)
    torch.cuda.synchronize()
    del big
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    fr = rkv.RingCache(1, N, H, D, CHUNK, prec, device=dev)
    kf = torch.randn(N, H, D, generator=gen, device=dev).to(torch.bfloat16)
    vf = torch.randn(N, H, D, generator=gen, device=dev).to(torch.bfloat16)
    pf = torch.arange(N, dtype=torch.int32, device=dev)
    for _ in range(3):
        fr.write(0, kf, vf, pf)
    torch.cuda.synchronize()
    del fr, kf, vf, pf
    st = rkv.RingCache(1, 11576, 48, D, CHUNK, prec, device=dev)
    ks = torch.randn(CHUNK, 48, D, generator=gen, device=dev).to(torch.bfloat16)
    for c in range(3):
        st.write(0, ks, ks, pos_pool[0] + CHUNK * c)
    torch.cuda.synchronize()
    if args.copy_mib:  # the byte counters' reference kernel, as in the full run
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps({"upkeep_only": True, "rotate_60layer_launches": 2, "write_full_ring_launches": 3,
                      "write_48head_launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    import fp8_ring_kv_amd as rkv
    from workloads import ATTEND, Stream, positions

    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    prec = rkv.RKV_PRECISE if args.precision == "precise" else rkv.RKV_FAST
    cache = rkv.RingCache(1, N, H, D, CHUNK, prec, device=dev, attn_workgroups=args.workgroups)

    # starting state: 8,888 tokens written in 757-token chunks -> ring head at slot 3,100
    s = Stream(ATTEND)
    p0 = 0
    fill = []
    while p0 < 8888:
        n = min(CHUNK, 8888 - p0)
        _, k, v = s.chunk(n)
        fill.append((to_dev(k), to_dev(v), torch.from_numpy(positions(p0, n)).to(dev)))
        cache.write(0, *fill[-1])
        p0 += n
    torch.cuda.synchronize()
    assert int(cache.state(0)[0]) == 3100 and int(cache.state(0)[1]) == N

    # input pool resident in HBM before timing: RESET_EVERY chunks of q, k, v
    pool = []
    for _ in range(RESET_EVERY):
        q, k, v = s.chunk()
        pool.append((to_dev(q), to_dev(k), to_dev(v)))
    pos_base = torch.arange(CHUNK, dtype=torch.int32, device=dev)
    out = torch.empty(CHUNK, H, D, dtype=torch.bfloat16, device=dev)
    # positions of the 42 chunks of a reset period (after each reset the cached
    # positions move back by 42 * 757, so new chunks reuse the same ones)
    pos_pool = [pos_base + (8888 + CHUNK * j) for j in range(RESET_EVERY)]

    if args.upkeep_only:
        upkeep_only(args, rkv, pool, pos_pool, prec, dev)
        return

    def step(i):
        j = i % RESET_EVERY
        q, k, v = pool[j]
        cache.write_attend(0, k, v, pos_pool[j], q, pos_pool[j], out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    # eager launches (one HIP launch per kernel)
    t_host0 = time.perf_counter()
    a.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    b.record(stream)
    b.synchronize()
    torch.cuda.synchronize()
    host_s = time.perf_counter() - t_host0
    eager_ms = a.elapsed_time(b) / args.steps
    assert torch.isfinite(out.float()).all()
    ms_per_step, launch = eager_ms, "eager (one HIP launch per kernel)"
    if not args.no_graph:
        # The same number of steps captured as one graph, replayed 10 times
        # untimed (back to the sustained clock after the capture's idle
        # time) and then once timed: exactly args.steps steps.
        first = args.warmup + args.steps
        g = capture_steps(cache, pool, pos_pool, out, first, args.steps)
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
        a.record(stream)
        g.replay()
        b.record(stream)
        b.synchronize()
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        ms_per_step = a.elapsed_time(b) / args.steps
        launch = f"hip_graph ({args.steps} steps captured as one graph, replayed)"
        del g

    if args.copy_mib:
        # reference kernel for the byte counters: reads and writes copy_mib MiB once
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    comp = {}
    peaks = None
    comp["eager_us_per_step"] = 1e3 * eager_ms
    if not args.no_components:
        r = args.reps
        q0, k0, v0 = pool[0]
        comp["attend_us"] = 1e3 * timed(lambda: cache.attend(0, q0, pos_pool[0], out), r, stream)
        # the other precision on a cache holding the same tokens
        other = rkv.RKV_FAST if prec == rkv.RKV_PRECISE else rkv.RKV_PRECISE
        twin = rkv.RingCache(1, N, H, D, CHUNK, other, device=dev, attn_workgroups=args.workgroups)
        for kvp in fill:
            twin.write(0, *kvp)
        key = "attend_fast_us" if other == rkv.RKV_FAST else "attend_precise_us"
        comp[key] = 1e3 * timed(lambda: twin.attend(0, q0, pos_pool[0], out), r, stream)
        del twin
        comp["write_us"] = 1e3 * timed(lambda: cache.write(0, k0, v0, pos_pool[0]), r, stream)
        comp["attend_TFLOPs"] = ATTN_FLOP / comp["attend_us"] / 1e6
        comp["write_GBps"] = WRITE_BYTES / comp["write_us"] / 1e3
    if not args.no_components and not args.attend_components_only:
        flip = [1]

        def rot():
            cache.rotate(0, flip[0])
            flip[0] = -flip[0]
        comp["rotate_1layer_us"] = 1e3 * timed(rot, max(20, r // 4), stream)
        comp["rotate_1layer_GBps"] = ROTATE_BYTES / comp["rotate_1layer_us"] / 1e3
        comp["reset_share_us_per_step"] = comp["rotate_1layer_us"] / RESET_EVERY
        # 60 stacked layer caches (1.1 GB): rotation of every layer in one launch,
        # and writes cycling over the layers -- both far beyond the 256 MB cache
        big = rkv.RingCache(60, N, H, D, CHUNK, prec, device=dev)
        for layer in range(60):
            for c in range(8):
                q, k, v = pool[(layer + c) % RESET_EVERY]
                big.write(layer, k, v, pos_pool[c])
        torch.cuda.synchronize()
        flip60 = [1]

        def rot60():
            big.rotate(-1, flip60[0])
            flip60[0] = -flip60[0]
        comp["rotate_60layer_us"] = 1e3 * timed(rot60, 6, stream)
        comp["rotate_60layer_GBps"] = 60 * ROTATE_BYTES / comp["rotate_60layer_us"] / 1e3
        lay = [0]

        def wr60():
            q, k, v = pool[lay[0] % RESET_EVERY]
            big.write(lay[0] % 60, k, v, pos_pool[0])
            lay[0] += 1
        comp["write_60layer_cycling_us"] = 1e3 * timed(wr60, 240, stream)
        comp["write_60layer_cycling_GBps"] = WRITE_BYTES / comp["write_60layer_cycling_us"] / 1e3
        # per-chunk sequence on the 60 layer caches: 4 denoising passes x 60
        # layers = 240 attention calls of 757 queries, each layer's cache
        # written once (the first pass writes and attends in one call); the
        # reset every 42 chunks is amortized from the 60-layer rotation above
        ch = [0]

        def chunk60():
            c = ch[0]
            for pas in range(4):
                for layer in range(60):
                    q, k, v = pool[(c + 4 * layer + pas) % RESET_EVERY]
                    if pas == 0:
                        big.write_attend(layer, k, v, pos_pool[c % RESET_EVERY], q, pos_pool[c % RESET_EVERY], out)
                    else:
                        big.attend(layer, q, pos_pool[c % RESET_EVERY], out)
            ch[0] += 1
        chunk60()
        comp["per_chunk_ms"] = timed(chunk60, 3, stream) + comp["rotate_60layer_us"] / 1e3 / RESET_EVERY
        del big
        torch.cuda.synchronize()
        # stress shape: 48 heads x 128 (the full width on one GPU), 11,576
        # slots filled by 16 writes of 757 tokens, one attention call of 757
        # queries over all of it (timing only: seeded N(0,1) device tensors)
        gen = torch.Generator(device=dev)
        gen.manual_seed(4)
        HS, NS = 48, 11576
        st = rkv.RingCache(1, NS, HS, D, CHUNK, prec, device=dev)
        ks = torch.randn(CHUNK, HS, D, generator=gen, device=dev).to(torch.bfloat16)
        vs = torch.randn(CHUNK, HS, D, generator=gen, device=dev).to(torch.bfloat16)
        qs = torch.randn(CHUNK, HS, D, generator=gen, device=dev).to(torch.bfloat16)
        for c in range(16):
            st.write(0, ks, vs, pos_base + CHUNK * c)
        wc = [16]

        def wst():
            st.write(0, ks, vs, pos_base + CHUNK * wc[0])
            wc[0] += 1
        comp["stress_write_us"] = 1e3 * timed(wst, 50, stream)
        comp["stress_write_GBps"] = STRESS_WRITE_BYTES / comp["stress_write_us"] / 1e3
        outs = torch.empty(CHUNK, HS, D, dtype=torch.bfloat16, device=dev)
        qpos = pos_base + CHUNK * 15
        st.attend(0, qs, qpos, outs)
        comp["stress_attend_us"] = 1e3 * timed(lambda: st.attend(0, qs, qpos, outs), 20, stream)
        comp["stress_attend_TFLOPs"] = STRESS_FLOP / comp["stress_attend_us"] / 1e6
        assert torch.isfinite(outs.float()).all()
        del st, ks, vs, qs, outs
        # the pages' layout: 1,246 global slots + a 4,542-slot ring of six
        # 757-token latents with 3-D RoPE (22/21/21 pairs); one attention call
        # of 757 queries over all 5,788 slots (the same work as the ring-only
        # workload) and one latent write
        from workloads import PAGES_LAYOUT, frame_positions
        pg = rkv.RingCache(1, PAGES_LAYOUT.n_slots, H, D, CHUNK, prec, device=dev,
                           n_global=PAGES_LAYOUT.n_global, rope_bands=PAGES_LAYOUT.bands)
        kg = torch.randn(PAGES_LAYOUT.n_global, H, D, generator=gen, device=dev).to(torch.bfloat16)
        pg.write_global(0, 0, kg, kg, torch.from_numpy(frame_positions(-1, PAGES_LAYOUT.n_global, 36)).to(dev))
        fpos = [torch.from_numpy(frame_positions(t, CHUNK, 28)).to(dev) for t in range(8)]
        for t in range(8):
            q, k, v = pool[t]
            pg.write(0, k, v, fpos[t])
        comp["pages_layout_attend_us"] = 1e3 * timed(lambda: pg.attend(0, q0, fpos[7], out), r, stream)
        comp["pages_layout_write_us"] = 1e3 * timed(lambda: pg.write(0, k0, v0, fpos[7]), r, stream)
        del pg, kg
        # one write of a whole ring's worth of tokens (5,788 x 12 heads, 54 MB
        # moved): the write kernel with enough work to approach bandwidth
        fr = rkv.RingCache(1, N, H, D, CHUNK, prec, device=dev)
        kf = torch.randn(N, H, D, generator=gen, device=dev).to(torch.bfloat16)
        vf = torch.randn(N, H, D, generator=gen, device=dev).to(torch.bfloat16)
        pf = torch.arange(N, dtype=torch.int32, device=dev)
        fr.write(0, kf, vf, pf)
        comp["write_full_ring_us"] = 1e3 * timed(lambda: fr.write(0, kf, vf, pf), 50, stream)
        comp["write_full_ring_GBps"] = FULL_WRITE_BYTES / comp["write_full_ring_us"] / 1e3
        del fr, kf, vf, pf
        torch.cuda.synchronize()
        # fused pre-attention RMS norm of Q and K (the same calls with the norm on)
        q0, k0, v0 = pool[0]
        wa = lambda: cache.write_attend(0, k0, v0, pos_pool[0], q0, pos_pool[0], out)
        comp["write_attend_us"] = 1e3 * timed(wa, r, stream)
        gen_w = torch.Generator(device=dev)
        gen_w.manual_seed(5)
        wq = (1 + 0.25 * torch.randn(D, generator=gen_w, device=dev)).to(torch.bfloat16)
        wk = (1 + 0.25 * torch.randn(D, generator=gen_w, device=dev)).to(torch.bfloat16)
        cache.set_qk_norm(0, wq, wk, 1e-6)
        comp["write_qk_norm_us"] = 1e3 * timed(lambda: cache.write(0, k0, v0, pos_pool[0]), r, stream)
        comp["write_attend_qk_norm_us"] = 1e3 * timed(wa, r, stream)
        cache.set_qk_norm(0, None, None)
        # the pages' static per-(layer, head) scales: calibrate from the cache
        # (amax x 1.5), then the same write and rotation with fixed scales
        cache.calibrate_static(0, 1.5)
        comp["write_static_us"] = 1e3 * timed(lambda: cache.write(0, k0, v0, pos_pool[0]), r, stream)
        # attention with the static scales (s_k folded into the queries, s_v
        # after the product, no per-slot scale reads)
        comp["attend_static_us"] = 1e3 * timed(lambda: cache.attend(0, q0, pos_pool[0], out), r, stream)
        comp["attend_static_TFLOPs"] = ATTN_FLOP / comp["attend_static_us"] / 1e6
        comp["rotate_static_1layer_us"] = 1e3 * timed(rot, max(20, r // 4), stream)
        cache.reset(0)
        torch.cuda.synchronize()
        peaks = measured_peaks(stream)

    res = {
        "metric": "µs per attention call (757q×5788 FP8 KV) + cache-write GB/s; % of roofline",
        "value": round(ms_per_step * 1e3, 3),
        "unit": "us per step (write 757 tokens + attend 757 queries)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 matmul, fp32 softmax/accumulate",
        "data": "synthetic",
        "config": {"workload": "attend_757x5788_h12", "heads": H, "head_dim": D, "slots": N,
                   "new_tokens": CHUNK, "queries": CHUNK, "reset_every": RESET_EVERY,
                   "ring_head_start": 3100, "precision": args.precision,
                   "outliers": "2% of channels x8"},
        "launch": launch,
        "host_wall_s": round(host_s, 4),
    }
    if comp:
        res["components"] = {k: round(v, 4) for k, v in comp.items()}
    if "attend_us" in comp:
        res["write_GBps"] = round(comp["write_GBps"], 2)
        achieved = comp["attend_TFLOPs"]
        res["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2),
                           "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": recorded_traffic(),
                           "kernel": "cache_attend call = q_prep_kernel + attend_kernel",
                           "per_launch_flop": ATTN_FLOP,
                           "per_launch_us": round(comp["attend_us"], 3)}
        busy = recorded_value(COUNTER_RECORD, "mfma_busy_cycles_per_call")
        if busy is not None:
            # matrix-core busy cycles (counter record) over the SIMD-cycles of the timed call
            simds = 4 * torch.cuda.get_device_properties(0).multi_processor_count
            res["roofline"]["mfma_busy_frac"] = round(busy / (simds * 2.4e9 * comp["attend_us"] * 1e-6), 4)
        if peaks:
            res["roofline"]["frac_of_measured_peak"] = round(achieved / peaks["fp8_mfma_TFLOPs"], 4)
    if "attend_static_us" in comp:
        a2 = comp["attend_static_TFLOPs"]
        res["roofline_static"] = {"workload": "attend_757x5788_h12, static per-head scales (calibrated x1.5)",
                                  "bound": "mfma", "achieved": round(a2, 2), "peak": PEAK_FP8_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(a2 / PEAK_FP8_TFLOPS, 4),
                                  "per_launch_flop": ATTN_FLOP, "per_launch_us": round(comp["attend_static_us"], 3)}
    if "rotate_60layer_GBps" in comp:
        res["roofline_hbm"] = {
            "write": {"achieved": round(comp["write_GBps"], 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                      "frac": round(comp["write_GBps"] / PEAK_HBM_GBPS, 4), "bytes": WRITE_BYTES},
            "rotate_60layer": {"achieved": round(comp["rotate_60layer_GBps"], 1), "peak": PEAK_HBM_GBPS,
                               "unit": "GB/s", "frac": round(comp["rotate_60layer_GBps"] / PEAK_HBM_GBPS, 4),
                               "bytes": 60 * ROTATE_BYTES},
        }
        for key, nbytes in [("stress_write", STRESS_WRITE_BYTES), ("write_full_ring", FULL_WRITE_BYTES)]:
            if key + "_GBps" in comp:
                a = comp[key + "_GBps"]
                res["roofline_hbm"][key] = {"achieved": round(a, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                            "frac": round(a / PEAK_HBM_GBPS, 4), "bytes": nbytes}
        if "stress_attend_TFLOPs" in comp:
            a = comp["stress_attend_TFLOPs"]
            res["roofline_stress"] = {"workload": "attend_757x11576_h48", "bound": "mfma", "achieved": round(a, 2),
                                      "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(a / PEAK_FP8_TFLOPS, 4),
                                      "per_launch_flop": STRESS_FLOP,
                                      "per_launch_us": round(comp["stress_attend_us"], 3)}
            if peaks:
                res["roofline_stress"]["frac_of_measured_peak"] = round(a / peaks["fp8_mfma_TFLOPs"], 4)
        if peaks:
            for part in res["roofline_hbm"].values():
                part["frac_of_measured_peak"] = round(part["achieved"] / peaks["hbm_stream_GBps"], 4)
    if peaks:
        res["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
