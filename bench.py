"""Benchmark of the per-frame hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1] [--no-cpu-baseline]

One step is one pass of the whole path over one synthetic stream: reset the
cache, then for every frame RoPE + append (kv_append_frame), paged attention
(attend_frame) and deferred eviction (kv_evict_deferred).  The default
workload is the single-layer bf16 stream of 64 frames of 37x37 patches + 6
special tokens, 16 heads of 64, scale_frames 8, sliding_window 16, every frame
a keyframe.  --workload 0/2/3 select the other single-layer streams, --workload
4 the full-depth stack (4 streams x 24 layers alternating frame and global
attention, the fused QKV projection + RoPE + append (kv_project_append_frame)
and the fp32 residual included; value counts stream-frames).  All inputs are generated (seeded, N(0,1), rounded to bf16)
and copied to HBM before timing.

Prints one JSON line: value = frames/s over the K timed steps; roofline of the
dominant kernel (paged attention, matrix-core bound) from HIP events recorded
around every attend_frame launch in the timed region; cpu_baseline = the CPU
oracle on a bounded sample of the same stream.
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


def visible_tokens(wl, f, interval=None, sf=None, w=None):
    """|T(f)|: retained tokens frame f attends to (keyframe schedule, scale
    frames, window; own frame always visible)."""
    iv = wl.keyframe_interval if interval is None else interval
    sf = wl.scale_frames if sf is None else sf
    w = wl.sliding_window if w is None else w
    m = (f + iv - 1) // iv if iv > 0 else 0                   # keyframes before f
    n_patch_frames = min(m, sf) + min(max(m - sf, 0), w) + 1
    return n_patch_frames * wl.patches + (m + 1) * wl.n_special


def attn_flops(wl, f, **kw):
    return 4.0 * wl.heads * wl.head_dim * wl.tokens * visible_tokens(wl, f, **kw) * wl.streams


def append_bytes(wl):
    e = 2 if wl.dtype == "bf16" else 4
    return 6.0 * wl.tokens * wl.heads * wl.head_dim * e * wl.streams


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per attend_frame call measured with rocprofv3 counters
    (profiles/attend_hbm_traffic.json), if they were taken on the current
    kernel sources for this workload; else None."""
    p = os.path.join(ROOT, "profiles", "attend_hbm_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("workload") != workload or d.get("source_sha256_16") != source_digest(d.get("sources", [])):
        return None
    return d.get("bytes_per_launch")


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


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
                      f"heads, all {wl.tokens} query rows), float64 numpy, past frames' K/V pre-rotated"}


def cpu_baseline_chain(wl, frames=2):
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
                      f"(projection, RoPE, attention, residual), float64 numpy"}


def result_line(wl, args, elapsed, frames_per_step, att_ms, att_flops, app_ms, info_splits,
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
    if app_ms is not None:
        app_gbs = append_bytes(wl) / (float(np.mean(app_ms)) / 1e3) / 1e9
        res["extra"].update({"rope_append_gbs": round(app_gbs, 1),
                             "rope_append_hbm_frac": round(app_gbs / HBM_PEAK_GBS, 4),
                             "rope_append_avg_us": round(float(np.mean(app_ms)) * 1e3, 2),
                             "rope_append_bytes_per_launch": append_bytes(wl)})
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

    def one_pass(ev=None):
        cache.reset(0)
        for f in range(F):
            if ev is not None:
                ev[f][0].record()
            cache.append(0, f, keyf[f], q_all[f], k_all[f], v_all[f], q_rot)
            if ev is not None:
                ev[f][1].record()
            cache.attend(0, q_rot, out, lse)
            if ev is not None:
                ev[f][2].record()
            cache.evict(0)

    for _ in range(args.warmup):
        one_pass()
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(F)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_pass(events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    att_ms = np.array([[e[f][1].elapsed_time(e[f][2]) for f in range(F)] for e in events])
    app_ms = np.array([[e[f][0].elapsed_time(e[f][1]) for f in range(F)] for e in events])
    flops = np.array([attn_flops(wl, f) for f in range(F)])
    steady = [f for f in range(F) if f >= wl.scale_frames + wl.sliding_window]
    extra = {}
    if steady:
        extra["attend_tflops_steady"] = round(
            float(flops[steady].mean() / (att_ms[:, steady].mean() / 1e3) / 1e12), 2)
    res = result_line(wl, args, elapsed, F * wl.streams, att_ms, np.tile(flops, (args.steps, 1)),
                      app_ms, cache.info()["attn_splits"], extra=extra)
    if not args.no_cpu_baseline:
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
    x = torch.empty_like(x0[0])

    def one_pass(ev=None, pev=None):
        fds.reset()
        for f in range(F):
            x.copy_(x0[f])
            fds.frame(f, x, events=ev, proj_events=pev)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    evs, pevs = [], []
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_pass(evs, pevs)
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
             "frame_steps_per_s": round(F * args.steps / elapsed, 3)}
    proj_us = float(np.mean([e0.elapsed_time(e1) for (_, _, e0, e1) in pevs])) * 1e3
    proj_flops = 2.0 * wl.streams * wl.tokens * wl.hidden * 3 * wl.heads * wl.head_dim
    extra.update({"project_append_avg_us": round(proj_us, 2),
                  "project_append_tflops": round(proj_flops / proj_us / 1e6, 1),
                  "project_append_mfma_frac": round(proj_flops / proj_us / 1e6 / BF16_PEAK_TFLOPS, 4)})
    res = result_line(wl, args, elapsed, F * wl.streams, att_ms, flops, None,
                      fds.global_cache.info()["attn_splits"], unit="stream-frames/s", extra=extra,
                      config_extra={"layers": wl.chain_layers, "hidden": wl.hidden,
                                    "includes": "fused QKV projection + RoPE + append, residual"})
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle chain on a sample")
        res["cpu_baseline"] = cpu_baseline_chain(wl)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3, 4])
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
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              f"(streams and heads shard without communication: run one process per GPU)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from rpkv_inputs import WORKLOADS

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if wl.chain_layers:
        res = bench_full_depth(wl, args, dev)
    else:
        res = bench_single_layer(wl, args, dev)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
