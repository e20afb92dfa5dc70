"""Benchmark of the per-frame hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--no-cpu-baseline]
    python bench.py --append-only [--workload W]

One step of a single-layer workload is one pass of the whole path over one
synthetic stream: reset the caches, then for every frame RoPE + append, paged
attention (attend_frame) and deferred eviction (kv_evict_deferred).  One step
of the full-depth workload is a quarter of its stream (64 frames through all
layers; the stream runs on across steps).  The default workload (4) is the
full-depth stack, the largest single-GPU workload of 37x37-patch frames: 4
streams of 256 frames (37x37 patches + 6 special tokens, 16 heads of 64,
bf16), 24 layers alternating frame attention (the frame's own tokens) and
global attention over the paged cache (scale_frames 8, sliding_window 32,
keyframe every 2nd frame), each layer's fused QKV projection + RoPE + append
(kv_project_append_frame, hidden 1024) and the fp32 residual included; value
counts stream-frames.  --workload 0..3 select the single-layer streams (RoPE +
append by kv_append_frame).  All inputs are generated (seeded, N(0,1), rounded
to bf16) and copied to HBM before timing.

Prints one JSON line: value = frames/s over the K timed steps; roofline of the
dominant kernel (paged attention, matrix-core bound) from HIP events recorded
around every attend_frame launch in the timed region; cpu_baseline = the CPU
oracle on a bounded sample of the same stream.

--append-only times kv_append_frame alone (RoPE + page write, HBM bound) at
the workload's geometry, all its streams in one launch, cold and warm, beside
a device copy of the same bytes, and prints its GB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix-core peak
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_tokens(wl, f, interval=None, sf=None, w=None, patches=None):
    """|T(f)|: retained tokens frame f attends to (keyframe schedule, scale
    frames, window; own frame always visible); patches: tokens per patch page
    when every frame has a grid of its own."""
    iv = wl.keyframe_interval if interval is None else interval
    sf = wl.scale_frames if sf is None else sf
    w = wl.sliding_window if w is None else w
    m = (f + iv - 1) // iv if iv > 0 else 0                   # keyframes before f
    n_patch_frames = min(m, sf) + min(max(m - sf, 0), w) + 1
    return n_patch_frames * (wl.patches if patches is None else patches) + (m + 1) * wl.n_special


def attn_flops(wl, f, queries=None, **kw):
    n_q = wl.tokens if queries is None else queries
    return 4.0 * wl.heads * wl.head_dim * n_q * visible_tokens(wl, f, **kw) * wl.streams


def append_bytes(wl):
    e = 2 if wl.dtype == "bf16" else 4
    return 6.0 * wl.tokens * wl.heads * wl.head_dim * e * wl.streams


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload, record="attend_hbm_traffic.json"):
    """HBM bytes per call of a kernel measured with rocprofv3 counters (a
    record under profiles/: attend_hbm_traffic.json for attend_frame,
    append_hbm_traffic.json for kv_append_frame), if they were taken on the
    current kernel sources for this workload; else None."""
    p = os.path.join(ROOT, "profiles", record)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("workload") != workload or d.get("source_sha256_16") != source_digest(d.get("sources", [])):
        return None
    return d.get("bytes_per_launch")


def cpu_threads():
    """Threads of the BLAS pool numpy runs its products on (the oracle's
    parallel part; its exponentials run on one thread)."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def cpu_host():
    """CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cores_available": len(os.sched_getaffinity(0))}


def cpu_baseline(wl, budget_s=20.0):
    """The oracle as it stands, timed on steady-state frames of the same stream."""
    from oracle.stream import OracleStream
    from rpkv_inputs import qkv
    ost = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t))
    start = min(wl.scale_frames + wl.sliding_window + 1, wl.frames - 1)   # window full from here
    f = start
    ost.keys(f)                                               # warm: rotate the retained past frames
    done, t0 = 0, time.perf_counter()
    while f < wl.frames:
        ost.attend(f)
        done += 1
        f += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done * wl.streams / dt, "unit": "frames/s", "cores": int(cpu_threads()),
            "kind": "oracle",
            "sample": f"frames {start}..{start + done - 1} of one stream (full window, all {wl.heads} "
                      f"heads, all {wl.tokens} query rows), float64 numpy, past frames' K/V pre-rotated",
            **cpu_host()}


def cpu_baseline_chain(wl, frames=3):
    """The full-depth oracle chain on the first frames of one stream."""
    from oracle.chain import OracleChain
    from rpkv_inputs import embeddings, projection
    ch = OracleChain(wl, lambda f: embeddings(wl, 0, f), lambda l: projection(wl, l))
    ch._weight(0)
    t0 = time.perf_counter()
    for f in range(frames):
        ch.frame(f)
    dt = time.perf_counter() - t0
    return {"value": frames / dt, "unit": "stream-frames/s", "cores": int(cpu_threads()),
            "kind": "oracle",
            "sample": f"frames 0..{frames - 1} of stream 0 through all {wl.chain_layers} layers "
                      f"(projection, RoPE, attention, residual), float64 numpy",
            **cpu_host()}


def result_line(wl, args, elapsed, frames_per_step, att_ms, att_flops, info_splits,
                unit="frames/s", extra=None, config_extra=None):
    import numpy as np
    att_avg_s = float(np.mean(att_ms)) / 1e3
    achieved = float(np.mean(att_flops)) / att_avg_s / 1e12
    config = {"workload": wl.name, "frames_per_step": frames_per_step, "streams": wl.streams,
              "grid": f"{wl.grid_h}x{wl.grid_w}", "tokens_per_frame": wl.tokens, "heads": wl.heads,
              "head_dim": wl.head_dim, "scale_frames": wl.scale_frames,
              "sliding_window": wl.sliding_window, "keyframe_interval": wl.keyframe_interval,
              "attn_splits": info_splits}
    config.update(config_extra or {})
    res = {
        "metric": "frames/s + attend_frame TFLOP/s (% bf16 MFMA peak), 1369 patches/frame, 1 GPU",
        "value": round(frames_per_step * args.steps / elapsed, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) inputs rounded to the storage dtype, resident in HBM)",
        "config": config,
        "roofline": {"bound": "mfma", "kernel": "attend_frame (k_attend_bf16 + k_attend_combine)",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": read_traffic(wl.name),
                     "avg_launch_us": round(att_avg_s * 1e6, 2),
                     "algorithmic_flops_per_launch": float(np.mean(att_flops))},
        "extra": extra or {},
    }
    return res


def bench_single_layer(wl, args, dev):
    import numpy as np
    import torch

    import rope_paged_kv_amd as rp
    from rpkv_inputs import stream_qkv

    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    log(f"[bench] workload {wl.name}: generating {wl.frames} frames of inputs")
    q_all, k_all, v_all = (torch.from_numpy(x).to(dev).to(dt)
                           for x in stream_qkv(wl, 0, threads=min(16, os.cpu_count() or 1)))
    torch.cuda.synchronize()
    spec = rp.make_spec(pairs=wl.pairs, theta=wl.theta, ntk_factor=wl.ntk_factor,
                        max_frames=wl.t_rows, max_h=wl.grid_h, max_w=wl.grid_w, layout=wl.rope_layout)
    cfg = rp.make_config(num_layers=1, num_streams=wl.streams, num_heads=wl.heads,
                         grid_h=wl.grid_h, grid_w=wl.grid_w, dtype=wl.dtype,
                         patch_page_size=wl.page_size, special_page_size=wl.special_page_size,
                         scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                         max_keyframes=wl.n_keyframes(), attn_splits=args.splits, rope=spec)
    cache = rp.PagedKVCache(cfg, device=dev)
    shape = (wl.streams, wl.tokens, wl.heads, wl.head_dim)
    q_rot = torch.empty(shape, dtype=dt, device=dev)
    out = torch.empty(shape, dtype=dt, device=dev)
    lse = torch.empty((wl.streams, wl.heads, wl.tokens), dtype=torch.float32, device=dev)
    keyf = [int(wl.is_keyframe(f)) for f in range(wl.frames)]
    F = wl.frames
    grid, npatch = None, wl.patches
    if args.grid:   # every frame of its own (smaller) grid inside the configured pages
        gh, gw = (int(v) for v in args.grid.lower().split("x"))
        if not (1 <= gh <= wl.grid_h and 1 <= gw <= wl.grid_w):
            raise SystemExit(f"--grid {args.grid}: at most {wl.grid_h}x{wl.grid_w}")
        grid, npatch = (gh, gw), gh * gw

    def one_pass(ev=None):
        cache.reset(0)
        for f in range(F):
            cache.append(0, f, keyf[f], q_all[f], k_all[f], v_all[f], q_rot, grid=grid)
            if ev is not None:
                ev[f][0].record()
            cache.attend(0, q_rot, out, lse)
            if ev is not None:
                ev[f][1].record()
            cache.evict(0)

    for _ in range(args.warmup):
        one_pass()
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(F)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_pass(events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    att_ms = np.array([[e[f][0].elapsed_time(e[f][1]) for f in range(F)] for e in events])
    flops = np.array([attn_flops(wl, f, queries=wl.n_special + npatch, patches=npatch)
                      for f in range(F)])
    steady = [f for f in range(F) if f >= wl.scale_frames + wl.sliding_window]
    extra = {}
    if steady:
        extra["attend_tflops_steady"] = round(
            float(flops[steady].mean() / (att_ms[:, steady].mean() / 1e3) / 1e12), 2)
    res = result_line(wl, args, elapsed, F * wl.streams, att_ms, np.tile(flops, (args.steps, 1)),
                      cache.info()["attn_splits"], extra=extra,
                      config_extra={"frame_grid": args.grid} if grid else None)
    if not args.no_cpu_baseline and grid is None:
        log("[bench] timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(wl)
    return res


def bench_full_depth(wl, args, dev):
    import numpy as np
    import torch
    from concurrent.futures import ThreadPoolExecutor

    from rope_paged_kv_amd.chain import FullDepthStream
    from rpkv_inputs import embeddings, projection

    log(f"[bench] workload {wl.name}: generating embeddings and weights")
    weights = [torch.from_numpy(projection(wl, l)).to(dev).to(torch.bfloat16)
               for l in range(wl.chain_layers)]
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        x0 = torch.stack([torch.from_numpy(np.stack(list(ex.map(lambda s: embeddings(wl, s, f),
                                                                range(wl.streams))))).to(dev)
                          for f in range(wl.frames)])
    fds = FullDepthStream(streams=wl.streams, layers=wl.chain_layers, heads=wl.heads,
                          grid_h=wl.grid_h, grid_w=wl.grid_w, scale_frames=wl.scale_frames,
                          sliding_window=wl.sliding_window, keyframe_interval=wl.keyframe_interval,
                          frames=wl.frames, weights=weights, attn_splits=args.splits, device=dev)
    F = wl.frames
    # A step is a quarter of the stream: 64 consecutive frames of all streams
    # through every layer.  The stream runs on across steps and starts again
    # on an emptied cache at frame 0, so 4 steps are one whole pass (warm-up
    # included: 5 warm-up and 20 timed steps time every frame exactly 5 times).
    per_step = min(F, 64)
    x = torch.empty_like(x0[0])
    cursor = [0]

    def one_step(ev=None, pev=None):
        for _ in range(per_step):
            f = cursor[0]
            if f == 0:
                fds.reset()
            x.copy_(x0[f])
            fds.frame(f, x, events=ev, proj_events=pev)
            cursor[0] = (f + 1) % F

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    evs, pevs = [], []
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_step(evs, pevs)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    att_ms, flops = [], []
    for (f, layer, e0, e1) in evs:
        att_ms.append(e0.elapsed_time(e1))
        if layer % 2 == 0:
            flops.append(4.0 * wl.heads * wl.head_dim * wl.tokens * wl.tokens * wl.streams)
        else:
            flops.append(attn_flops(wl, f))
    att_ms, flops = np.array(att_ms), np.array(flops)
    glob = np.array([layer % 2 == 1 for (_, layer, _, _) in evs])
    extra = {"attend_tflops_global_layers": round(float(flops[glob].mean() / (att_ms[glob].mean() / 1e3) / 1e12), 2),
             "attend_tflops_frame_layers": round(float(flops[~glob].mean() / (att_ms[~glob].mean() / 1e3) / 1e12), 2),
             "frame_steps_per_s": round(per_step * args.steps / elapsed, 3)}
    proj_us = float(np.mean([e0.elapsed_time(e1) for (_, _, e0, e1) in pevs])) * 1e3
    proj_flops = 2.0 * wl.streams * wl.tokens * wl.hidden * 3 * wl.heads * wl.head_dim
    extra.update({"project_append_avg_us": round(proj_us, 2),
                  "project_append_tflops": round(proj_flops / proj_us / 1e6, 1),
                  "project_append_mfma_frac": round(proj_flops / proj_us / 1e6 / BF16_PEAK_TFLOPS, 4)})
    res = result_line(wl, args, elapsed, per_step * wl.streams, att_ms, flops,
                      fds.global_cache.info()["attn_splits"], unit="stream-frames/s", extra=extra,
                      config_extra={"layers": wl.chain_layers, "hidden": wl.hidden,
                                    "stream_frames": F,
                                    "step": f"{per_step} consecutive frames of the {F}-frame streams "
                                            "(the stream runs on across steps, from an emptied cache "
                                            "at frame 0)",
                                    "includes": "fused QKV projection + RoPE + append, residual"})
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle chain on a sample")
        res["cpu_baseline"] = cpu_baseline_chain(wl)
    return res


def _spin_cycles_per_ms(dev):
    """Rate of torch.cuda._sleep (a bounded spin kernel) on this GPU."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record()
    torch.cuda._sleep(20_000_000)
    e1.record()
    torch.cuda.synchronize()
    return 20_000_000 / e0.elapsed_time(e1)


def _batch_us(fn, count, spin_cycles):
    """Mean GPU time (us) per call of `count` back-to-back calls fn(i), from one
    pair of HIP events around the batch.  A spin queued first keeps the GPU
    busy while the host enqueues the batch, so the kernels run back to back
    and neither host launch gaps nor per-event overhead enter the figure."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(spin_cycles)
    e0.record()
    for i in range(count):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / count


def bench_append(wl, args, dev):
    """kv_append_frame alone at the workload's geometry (all streams in one
    launch), with a plain device copy of the same bytes (half read, half
    written) beside it as the achievable rate at this size.

    The cache is first run through the stream's opening frames, then the
    timed calls append one steady-state frame over and over (each call
    replaces the previous call's tentative slot, as the C API defines), back
    to back.  Two input regimes: cold (16 frames of inputs in rotation, more
    than the caches hold at four streams) and warm (one frame's inputs, read
    by the previous call: what a producer that has just written q, k, v
    gives)."""
    import dataclasses
    import time

    import torch

    import rope_paged_kv_amd as rp
    from rpkv_inputs import frame_qkv

    if args.rope_layout == "half_split":
        # the 2D module's form: half-split axis blocks, pairs (0, 16, 16), base 100
        wl = dataclasses.replace(wl, name=wl.name + "_halfsplit", pairs=(0, 16, 16), theta=100.0,
                                 rope_layout=1)
    grid = None
    ntok = wl.tokens
    if args.grid:
        gh, gw = (int(v) for v in args.grid.lower().split("x"))
        if not (1 <= gh <= wl.grid_h and 1 <= gw <= wl.grid_w):
            raise SystemExit(f"--grid {args.grid}: at most {wl.grid_h}x{wl.grid_w}")
        grid = (gh, gw)
        ntok = wl.n_special + gh * gw
    nf = 16
    qkv = [tuple(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in frame_qkv(wl, 0, f))
           for f in range(nf)]
    spec = rp.make_spec(pairs=wl.pairs, theta=wl.theta, ntk_factor=wl.ntk_factor,
                        max_frames=wl.t_rows, max_h=wl.grid_h, max_w=wl.grid_w, layout=wl.rope_layout)
    cfg = rp.make_config(num_layers=1, num_streams=wl.streams, num_heads=wl.heads,
                         grid_h=wl.grid_h, grid_w=wl.grid_w, dtype=wl.dtype,
                         patch_page_size=wl.page_size, special_page_size=wl.special_page_size,
                         scale_frames=wl.scale_frames, sliding_window=wl.sliding_window,
                         max_keyframes=wl.n_keyframes(), rope=spec)
    cache = rp.PagedKVCache(cfg, device=dev)
    q_rot = torch.empty_like(qkv[0][0])
    # bytes of the tokens a call reads and writes (a frame of its own grid: only those)
    nbytes = append_bytes(wl) * ntok / wl.tokens
    src = [torch.cat([t[:, :ntok].reshape(-1) for t in f]) for f in qkv]   # the same bytes as q, k, v
    dst = torch.empty_like(src[0])
    assert 2 * src[0].numel() * src[0].element_size() == nbytes

    # steady state: scale pages and a full window behind the timed frame
    f_pos = min(wl.frames - 1, wl.scale_frames * wl.keyframe_interval + wl.sliding_window + 2)
    cache.reset(0)
    for f in range(f_pos):
        q, k, v = qkv[f % nf]
        cache.append(0, f, int(wl.is_keyframe(f)), q, k, v, q_rot, grid=grid)
        cache.evict(0)
    commit = int(wl.is_keyframe(f_pos))

    def append_fn(rot):
        return lambda i: cache.append(0, f_pos, commit, *qkv[i % nf if rot else 0], q_rot, grid=grid)

    def copy_fn(rot):
        return lambda i: dst.copy_(src[i % nf if rot else 0])

    count = wl.frames * args.steps
    rate = _spin_cycles_per_ms(dev)
    # host enqueue time of one batch (GPU left to drain), to size the spin
    t0 = time.perf_counter()
    for _ in range(max(args.warmup, 1)):
        _batch_us(append_fn(True), count, 1000)
    host_ms = (time.perf_counter() - t0) * 1e3 / max(args.warmup, 1)
    spin = int(rate * (1.5 * host_ms + 2.0))
    res = {}
    for name, fn in (("append_cold", append_fn(True)), ("append_warm", append_fn(False)),
                     ("copy_cold", copy_fn(True)), ("copy_warm", copy_fn(False))):
        _batch_us(fn, nf, 1000)                         # warm-up
        us = _batch_us(fn, count, spin)
        res[name] = (us, nbytes / us / 1e3)
    cache.rollback(0)
    us, gbs = res["append_cold"]
    extra = {k: {"avg_us": round(v[0], 2), "gbs": round(v[1], 1),
                 "hbm_frac": round(v[1] / HBM_PEAK_GBS, 4)} for k, v in res.items()}
    extra.update({"cold_frac_of_copy": round(res["copy_cold"][0] / res["append_cold"][0], 3),
                  "warm_frac_of_copy": round(res["copy_warm"][0] / res["append_warm"][0], 3),
                  "copy": "device-to-device copy of the same byte count (torch copy_)",
                  "launches_per_regime": count, "host_enqueue_ms_per_batch": round(host_ms, 2)})
    return {"metric": "kv_append_frame GB/s (RoPE + page write, % HBM)", "value": round(gbs, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "dtype": wl.dtype, "data": "synthetic",
            "config": {"workload": wl.name, "streams": wl.streams,
                       "grid": f"{wl.grid_h}x{wl.grid_w}", "heads": wl.heads,
                       "launches_per_step": wl.frames, "inputs": "cold (16 frames in rotation)",
                       "rope_layout": "half_split" if wl.rope_layout == 1 else "interleaved",
                       "frame_grid": f"{grid[0]}x{grid[1]}" if grid else f"{wl.grid_h}x{wl.grid_w}"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": read_traffic(wl.name, "append_hbm_traffic.json"),
                         "avg_launch_us": round(us, 2), "algorithmic_bytes_per_launch": nbytes},
            "extra": extra}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--append-only", action="store_true",
                    help="time kv_append_frame alone at the workload's geometry")
    ap.add_argument("--rope-layout", choices=["interleaved", "half_split"], default="interleaved",
                    help="--append-only: rotary layout (half_split: the 2D module's half-split "
                         "axis blocks, pairs 0/16/16, base 100)")
    ap.add_argument("--grid", default=None,
                    help="single-layer workloads and --append-only: every frame of its own patch "
                         "grid HxW inside the workload's pages (kv_append_frame_grid)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times) and exit: "
                         "the reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.calibration_copy_mb:
        import torch
        n = args.calibration_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "copies": 3}))
        return
    if args.rope_layout != "interleaved" and not args.append_only:
        raise SystemExit("--rope-layout applies to --append-only (the other lines run the workload's layout)")
    if args.grid and not args.append_only and args.workload == 4:
        raise SystemExit("--grid applies to the single-layer workloads and to --append-only")
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              f"(streams and heads shard without communication: run one process per GPU)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from rpkv_inputs import WORKLOADS

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.append_only:
        res = bench_append(wl, args, dev)
    elif wl.chain_layers:
        res = bench_full_depth(wl, args, dev)
    else:
        res = bench_single_layer(wl, args, dev)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
