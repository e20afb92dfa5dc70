"""Benchmark of the per-frame hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1] [--no-cpu-baseline]

One step is one pass of the whole path over one synthetic stream: reset the
cache, then for every frame RoPE + append (kv_append_frame), paged attention
(attend_frame) and deferred eviction (kv_evict_deferred).  The default
workload is the single-layer bf16 stream of 64 frames of 37x37 patches + 6
special tokens, 16 heads of 64, scale_frames 8, sliding_window 16, every frame
a keyframe.  All inputs are generated (seeded, N(0,1), rounded to bf16) and
copied to HBM before timing.

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


def visible_tokens(wl, f):
    """|T(f)|: retained tokens frame f attends to (keyframe schedule, scale
    frames, window; own frame always visible)."""
    m = (f + wl.keyframe_interval - 1) // wl.keyframe_interval   # keyframes before f
    n_patch_frames = min(m, wl.scale_frames) + min(max(m - wl.scale_frames, 0), wl.sliding_window) + 1
    return n_patch_frames * wl.patches + (m + 1) * wl.n_special


def attn_flops(wl, f):
    return 4.0 * wl.heads * wl.head_dim * wl.tokens * visible_tokens(wl, f) * wl.streams


def append_bytes(wl):
    e = 2 if wl.dtype == "bf16" else 4
    return 6.0 * wl.tokens * wl.heads * wl.head_dim * e * wl.streams


def source_digest(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def read_traffic(kernel_src):
    """HBM traffic per launch measured with rocprofv3 counters, if the summary
    was taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", "attend_hbm_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_sha256_16") != source_digest(kernel_src):
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(wl, budget_s=20.0):
    """The oracle as it stands, timed on steady-state frames of the same stream."""
    from oracle.stream import OracleStream
    from rpkv_inputs import qkv
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    ost = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t))
    start = wl.scale_frames + wl.sliding_window + 1          # window full from here
    f0 = min(start, wl.frames - 1)
    ost.keys(f0)                                               # warm: rotate the retained past frames
    done, t0 = 0, time.perf_counter()
    f = f0
    while f < wl.frames:
        ost.attend(f)
        done += 1
        f += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done * wl.streams / dt, "unit": "frames/s", "cores": int(cores), "kind": "oracle",
            "sample": f"frames {f0}..{f0 + done - 1} of the stream (full window, all {wl.heads} heads, "
                      f"all {wl.tokens} query rows), float64 numpy, past frames' K/V pre-rotated"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3])
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

    import numpy as np
    import torch

    import rope_paged_kv_amd as rp
    from rpkv_inputs import WORKLOADS, stream_qkv

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    log(f"[bench] workload {wl.name}: generating {wl.frames} frames of inputs")
    q_all, k_all, v_all = (torch.from_numpy(x).to(dev).to(dt)
                           for x in stream_qkv(wl, 0, threads=min(16, os.cpu_count() or 1)))
    torch.cuda.synchronize()
    spec = rp.make_spec(pairs=wl.pairs, theta=wl.theta, ntk_factor=wl.ntk_factor,
                        max_frames=wl.t_rows, max_h=wl.grid_h, max_w=wl.grid_w)
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
    torch.cuda.synchronize()

    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(F)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_pass(events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    att_ms = np.array([[events[k][f][1].elapsed_time(events[k][f][2]) for f in range(F)]
                       for k in range(args.steps)])
    app_ms = np.array([[events[k][f][0].elapsed_time(events[k][f][1]) for f in range(F)]
                       for k in range(args.steps)])
    flops = np.array([attn_flops(wl, f) for f in range(F)])
    att_avg_s = att_ms.mean() / 1e3
    achieved_tflops = flops.mean() / att_avg_s / 1e12
    steady = [f for f in range(F) if f >= wl.scale_frames + wl.sliding_window]
    steady_tflops = (flops[steady].mean() / (att_ms[:, steady].mean() / 1e3) / 1e12) if steady else None
    app_gbs = append_bytes(wl) / (app_ms.mean() / 1e3) / 1e9
    frames_per_s = F * args.steps * wl.streams / elapsed
    traffic = read_traffic(os.path.join(ROOT, "rope_paged_kv_amd", "csrc", "k_attend.hip"))

    info = cache.info()
    res = {
        "metric": "frames/s + attend_frame TFLOP/s (% bf16 MFMA peak), 1369 patches/frame, 1 GPU",
        "value": round(frames_per_s, 3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V rounded to bf16, resident in HBM)",
        "config": {"workload": wl.name, "frames_per_step": F, "streams": wl.streams,
                   "grid": f"{wl.grid_h}x{wl.grid_w}", "tokens_per_frame": wl.tokens,
                   "heads": wl.heads, "head_dim": wl.head_dim, "scale_frames": wl.scale_frames,
                   "sliding_window": wl.sliding_window, "keyframe_interval": wl.keyframe_interval,
                   "attn_splits": info["attn_splits"]},
        "roofline": {"bound": "mfma", "kernel": "attend_frame",
                     "achieved": round(achieved_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "avg_launch_us": round(att_avg_s * 1e6, 2),
                     "algorithmic_flops_per_launch": flops.mean()},
        "extra": {
            "attend_tflops_steady": round(steady_tflops, 2) if steady_tflops else None,
            "rope_append_gbs": round(app_gbs, 1),
            "rope_append_hbm_frac": round(app_gbs / HBM_PEAK_GBS, 4),
            "rope_append_avg_us": round(app_ms.mean() * 1e3, 2),
            "rope_append_bytes_per_launch": append_bytes(wl),
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
