"""GPU parity at the full workload sizes, on sampled outputs the oracle
computes one by one: the long keyframe-interval stream, the 64x64 grid, the
four-stream cache geometry of the full-depth stack, and the full-depth chain
(projection, alternating frame/global layers, residual): at full size on its
first frames, and at a reduced size through eviction and page recycling.

Bars as in test_gpu_parity: bf16 outputs within 2e-2 max-abs of the float64
oracle, LSE within 1e-2, page tables bit-exact."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import rope_paged_kv_amd as rp
from gpu_harness import Runner, make_cache, to_dev
from oracle import pages
from oracle.chain import OracleChain
from oracle.stream import OracleStream
from rpkv_inputs import WORKLOADS, embeddings, projection, qkv, qkv_layer, stream_qkv

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
LSE_TOL = 1e-2


def sampled_rows(wl, f, n_patch=24):
    rng = np.random.default_rng(1000 + f)
    pr = rng.choice(np.arange(wl.n_special + 1, wl.tokens - 1), n_patch, replace=False)
    return np.unique(np.r_[np.arange(wl.n_special), wl.n_special, wl.tokens - 1, pr])


def compare(run, ost, wl, f, s=0, rows=None):
    torch.cuda.synchronize()
    r = sampled_rows(wl, f) if rows is None else rows
    o, lse = ost.attend(f, rows=r)
    got = run.out[s].float().cpu().numpy()[r]
    got_lse = run.lse[s].cpu().numpy()[:, r]
    err, lerr = np.abs(got - o).max(), np.abs(got_lse - lse).max()
    assert err <= BF16_TOL and lerr <= LSE_TOL, (f, s, err, lerr)
    return err, lerr


def stream_frames(wl, layer_fn, chunk=64):
    """Yields (f, q, k, v) device tensors [S][N][H][D], generated chunk by chunk."""
    for c0 in range(0, wl.frames, chunk):
        fr = range(c0, min(wl.frames, c0 + chunk))
        if layer_fn is None:
            q, k, v = stream_qkv(wl, 0, frames=fr, threads=16)
        else:
            q, k, v = (np.stack([np.stack([layer_fn(f, s, t) for s in range(wl.streams)]) for f in fr])
                       for t in range(3))
        qd, kd, vd = (to_dev(x, torch.bfloat16) for x in (q, k, v))
        for i, f in enumerate(fr):
            yield f, qd[i], kd[i], vd[i]


def test_long_stream_1024_frames_keyframe_every_5th():
    wl = WORKLOADS[2]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    ost = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t))
    sim = pages.PageSim(wl.scale_frames, wl.sliding_window, wl.special_page_size, wl.n_special)
    check = {0, 35, 36, 40, 360, 361, 364, 365, 366, 1020, 1023}
    worst = [0.0, 0.0]
    for f, q, k, v in stream_frames(wl, None):
        kf = wl.is_keyframe(f)
        sim.append(f, kf)
        run.frame(f, q, k, v, kf, evict=False)
        if f in check:
            st = cache.state()
            assert st["visible_pages"] == sim.visible.patch_pages, f
            assert st["visible_special_pages"] == sim.visible.special_pages, f
            e, l = compare(run, ost, wl, f)
            worst = [max(worst[0], e), max(worst[1], l)]
        sim.evict()
        cache.evict(0)
    st = cache.state()
    assert st["n_special_tokens"] == 1230 and st["free_list"] == [10] and st["fresh"] == 73
    print(f"long stream: max|out-oracle| {worst[0]:.3e}  max|lse-oracle| {worst[1]:.3e}")


def test_long_stream_every_frame_on_fixed_rows():
    """The 1024-frame stream (keyframe every 5th), every frame: the output and
    LSE of a fixed row sample -- the 6 special tokens and the first and last
    patch token -- against the float64 oracle, on 2 heads per frame (head
    h at frames f with f % 8 == h % 8, so every head every 8th frame).

    The retained set of each frame is the oracle's enumeration
    (OracleStream.visible); the K/V of the retained frames (OracleStream.kv,
    computed a few frames ahead in threads) sit in a CPU mirror, one slot per retained frame (a frame that leaves the
    set frees its slot for the next stored one), and the oracle's attention
    runs on each checked head's keys: stored patches, the frame's own patches,
    stored specials, its own specials.  Softmax does not depend on the order
    of the keys, so this is the oracle stream's computation without
    re-gathering ~1.6 GB of keys per frame."""
    from oracle import attention as att
    wl = WORKLOADS[2]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    ost = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t))
    ns, P, H, D = wl.n_special, wl.patches, wl.heads, wl.head_dim
    rows = np.r_[np.arange(ns), ns, wl.tokens - 1]
    n_slots = wl.scale_frames + wl.sliding_window
    Kp, Vp = np.zeros((H, n_slots * P, D)), np.zeros((H, n_slots * P, D))
    Ks, Vs = np.zeros((H, wl.n_keyframes() * ns, D)), np.zeros((H, wl.n_keyframes() * ns, D))
    slot_of, free, n_sp = {}, [], 0
    last = None   # (frame, K, V) of the previous frame, stored if it was a keyframe
    worst = [0.0, 0.0]

    def oracle_frame(f):
        # the oracle's rotated K, V and Q rows of frame f (independent of the
        # mirror: computed ahead, several frames at a time)
        o = OracleStream(wl, lambda f_, t: qkv(wl, 0, 0, f_, t))
        kf, vf = o.kv(f)
        return kf, vf, o.q_rot(f)[rows]

    pool = ThreadPoolExecutor(8)
    ahead = {}
    for f, q, k, v in stream_frames(wl, None):
        if f not in ahead:
            ahead = {g: pool.submit(oracle_frame, g) for g in range(f, min(wl.frames, f + 32))}
        kf, vf, qr = ahead.pop(f).result()
        run.frame(f, q, k, v, wl.is_keyframe(f))
        pf, sf = ost.visible(f)
        stored_p, stored_s = [g for g in pf if g != f], [g for g in sf if g != f]
        for g in [g for g in slot_of if g not in stored_p]:
            free.append(slot_of.pop(g))
        if last is not None and last[0] in stored_s:       # the previous frame was stored
            g, kg, vg = last
            if g in stored_p:
                slot = free.pop() if free else len(slot_of)
                slot_of[g] = slot
                Kp[:, slot * P:(slot + 1) * P] = kg[ns:].transpose(1, 0, 2)
                Vp[:, slot * P:(slot + 1) * P] = vg[ns:].transpose(1, 0, 2)
            Ks[:, n_sp:n_sp + ns] = kg[:ns].transpose(1, 0, 2)
            Vs[:, n_sp:n_sp + ns] = vg[:ns].transpose(1, 0, 2)
            n_sp += ns
        assert sorted(slot_of) == sorted(stored_p) and n_sp == ns * len(stored_s), f
        last = (f, kf, vf)
        n_used = len(slot_of)
        assert sorted(slot_of.values()) == list(range(n_used)), f   # the slots in use are a prefix
        torch.cuda.synchronize()
        got = run.out[0].float().cpu().numpy()[rows]
        got_lse = run.lse[0].cpu().numpy()[:, rows]
        for h in range(f % 8, H, 8):
            kk = np.concatenate([Kp[h][:n_used * P], kf[ns:, h], Ks[h][:n_sp], kf[:ns, h]])
            vv = np.concatenate([Vp[h][:n_used * P], vf[ns:, h], Vs[h][:n_sp], vf[:ns, h]])
            o, lse = att.attention(qr[:, h], kk, vv)
            e, le = np.abs(got[:, h] - o).max(), np.abs(got_lse[h] - lse).max()
            worst = [max(worst[0], e), max(worst[1], le)]
            assert e <= BF16_TOL and le <= LSE_TOL, (f, h, e, le)
    pool.shutdown()
    print(f"long stream, every frame: max|out-oracle| {worst[0]:.3e}  max|lse-oracle| {worst[1]:.3e}")


def test_large_grid_64x64():
    wl = WORKLOADS[3]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    ost = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t))
    check = {0, 3, 4, 5, 19, 20, 21, 31}
    worst = [0.0, 0.0]
    for f, q, k, v in stream_frames(wl, None, chunk=16):
        run.frame(f, q, k, v, wl.is_keyframe(f))
        if f in check:
            e, l = compare(run, ost, wl, f)
            worst = [max(worst[0], e), max(worst[1], l)]
    print(f"64x64 grid: max|out-oracle| {worst[0]:.3e}  max|lse-oracle| {worst[1]:.3e}")


def test_large_grid_64x64_all_rows_at_recycle_and_last_frame():
    """The 64x64 stream in full on two frames: every query row (6 specials and
    4096 patches) of every head at the first recycled page (frame 21: 4
    scale pages, the window of 16 after its first eviction, the frame's own
    page) and the last frame (31), against the float64 oracle."""
    wl = WORKLOADS[3]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    ost = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t))
    worst = [0.0, 0.0]
    for f, q, k, v in stream_frames(wl, None, chunk=16):
        run.frame(f, q, k, v, wl.is_keyframe(f))
        if f in (21, 31):
            e, l = compare(run, ost, wl, f, rows=np.arange(wl.tokens))
            worst = [max(worst[0], e), max(worst[1], l)]
            print(f"64x64 frame {f}, all rows: max|out-oracle| {e:.3e}  max|lse-oracle| {l:.3e}", flush=True)
    st = cache.state(0, 0)
    assert st["fresh"] == wl.scale_frames + wl.sliding_window + 1, st["fresh"]


def test_full_depth_cache_geometry_four_streams():
    """The cached layers of the full-depth stack at full geometry (4 streams,
    sf 8, window 32, keyframe every 2nd frame), fed seeded Q/K/V: two cached
    layers of one handle, checked on two streams at the eviction and recycle
    transitions (every row of one stream and layer at the first recycled page,
    frame 82); plus a frame (no-cache) layer on the same frames."""
    wl = WORKLOADS[4]
    layers = (3, 17)                       # input keys of handle layers 0 and 1
    cache = make_cache(wl, layers=2)
    runs = [Runner(wl, cache, layer=i) for i in range(2)]
    fwl = wl.replace(scale_frames=0, sliding_window=0)
    fcache = make_cache(fwl, max_keyframes=0, splits=1)
    frun = Runner(fwl, fcache)
    orc = {(i, s): OracleStream(wl, (lambda key, s_: (lambda f, t: qkv_layer(wl, key, s_, f, t)))(layers[i], s))
           for i in range(2) for s in (0, 3)}
    forc = OracleStream(fwl, lambda f, t: qkv_layer(wl, 0, 1, f, t), keyframe_interval=0)
    check = {1, 81, 82, 255}
    for f, q, k, v in stream_frames(wl, None):
        kf = wl.is_keyframe(f)
        for i, run in enumerate(runs):
            sh = layers[i]
            run.frame(f, torch.roll(q, sh, 2), torch.roll(k, sh, 2), torch.roll(v, sh, 2), kf)
            if f in check:
                for s in (0, 3):
                    # the first recycled page (frame 82): every row of stream 0, layer 0
                    full = f == 82 and i == 0 and s == 0
                    compare(run, orc[(i, s)], wl, f, s=s,
                            rows=np.arange(wl.tokens) if full else sampled_rows(wl, f, 12))
        frun.frame(f, q, k, v, False, evict=False)
        if f in check:
            compare(frun, forc, fwl, f, s=1, rows=sampled_rows(wl, f, 12))
    for s in range(4):
        st = cache.state(1, s)
        assert st["n_special_tokens"] == 6 * 128 and st["fresh"] == 41, s


def _chain(wl, frames=None):
    from rope_paged_kv_amd.chain import FullDepthStream
    weights = [to_dev(projection(wl, l), torch.bfloat16) for l in range(wl.chain_layers)]
    return FullDepthStream(streams=wl.streams, layers=wl.chain_layers, heads=wl.heads,
                           grid_h=wl.grid_h, grid_w=wl.grid_w, scale_frames=wl.scale_frames,
                           sliding_window=wl.sliding_window, keyframe_interval=wl.keyframe_interval,
                           frames=wl.frames if frames is None else frames, weights=weights)


def _chain_oracles(wl, streams):
    return {s: OracleChain(wl, (lambda s_: (lambda f: embeddings(wl, s_, f)))(s),
                           lambda l: projection(wl, l)) for s in streams}


def _check_chain_frame(wl, fds, oracles, f, streams):
    """Runs frame f on the GPU chain and compares every stored layer output of
    the given streams with the float64 chain (each side feeds its own outputs
    forward: nothing is teacher-forced).  Returns the worst error."""
    x = torch.from_numpy(np.stack([embeddings(wl, s, f) for s in range(wl.streams)])).cuda()
    keep = []
    fds.frame(f, x, keep)
    torch.cuda.synchronize()
    worst = 0.0
    for s in streams:
        outs, xl = oracles[s].frame(f)
        errs = [float(np.abs(keep[layer][s].float().cpu().numpy() - outs[layer]).max())
                for layer in range(wl.chain_layers)]
        mags = [float(np.abs(outs[layer]).max()) for layer in range(wl.chain_layers)]
        dx = float(np.abs(x[s].cpu().numpy() - xl).max())
        print(f"frame {f} stream {s}: per-layer max err {np.round(errs, 4).tolist()}")
        print(f"   per-layer max|O| {np.round(mags, 2).tolist()}  max|x_L - oracle| {dx:.4f}")
        # every stored layer output (bf16) within the bf16 bar; x_L is the fp32
        # sum of x_0 and these outputs, so the per-layer outputs are the gate
        assert max(errs) <= BF16_TOL, (f, s, errs)
        worst = max(worst, max(errs))
    return worst


def test_full_depth_chain_first_frames():
    """The 24-layer, 4-stream chain (hidden 1024, weights N(0, 0.02)) on its
    first frames, every output of streams 0 and 3 against the float64 chain."""
    wl = WORKLOADS[4]
    fds = _chain(wl)
    oracles = _chain_oracles(wl, (0, 3))
    worst = 0.0
    for f in range(3):
        worst = max(worst, _check_chain_frame(wl, fds, oracles, f, (0, 3) if f < 2 else (0,)))
    print(f"full-depth chain, frames 0-2: max|O_l - oracle| {worst:.3e}")


def test_full_depth_structure_through_eviction_and_recycle():
    """The full-depth stack's structure at a reduced size (4 streams, 24
    alternating frame / global layers, fused projection + RoPE + append,
    keyframe every 2nd frame, scale_frames 2, window 3; 6x6 grid, 4 heads,
    hidden 256): all 16 frames, every layer's output of every stream against
    the float64 chain -- past the first eviction (frame 10) and the first
    recycled page (frame 12).  The global caches' bookkeeping then matches the
    page simulator."""
    from rpkv_inputs import small_variants
    wl = small_variants()["small_depth"]
    fds = _chain(wl)
    oracles = _chain_oracles(wl, range(wl.streams))
    sim = pages.PageSim(wl.scale_frames, wl.sliding_window, wl.special_page_size, wl.n_special)
    worst = 0.0
    for f in range(wl.frames):
        sim.append(f, wl.is_keyframe(f))
        worst = max(worst, _check_chain_frame(wl, fds, oracles, f, range(wl.streams)))
        sim.evict()
        if f in (10, 12):
            for layer in (0, wl.chain_layers // 2 - 1):
                for s in range(wl.streams):
                    st = fds.global_cache.state(layer, s)
                    assert st["free_list"] == sim.free and st["window_pages"] == list(sim.window), (f, layer, s)
    assert sim.fresh == wl.scale_frames + wl.sliding_window + 1 and len(sim.free) == 1
    print(f"reduced full-depth chain, 16 frames: max|O_l - oracle| {worst:.3e}")
