"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bars: page tables, indices and V pages bit-exact; fp32 outputs within 1e-5;
bf16 outputs (q_rot, cached K, attention output) within 2e-2 max-abs of the
float64 oracle; the fp32 log-sum-exp of bf16 runs within 1e-2 (a frame more or
less in the visible set moves it by ~0.04 at these sizes)."""
import math

import numpy as np
import pytest
import torch

import rope_paged_kv_amd as rp
from gpu_harness import Runner, make_cache, to_dev, torch_dtype
from oracle import pages, rope3d
from oracle.stream import OracleStream
from rpkv_inputs import WORKLOADS, frame_qkv, qkv, round_to_bf16, small_variants

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-5
LSE_TOL = 1e-2


def tol(wl):
    return F32_TOL if wl.dtype == "f32" else BF16_TOL


def sim_for(wl):
    return pages.PageSim(wl.scale_frames, wl.sliding_window, wl.special_page_size, wl.n_special)


def check_state(st, sim, f):
    vis = sim.visible
    assert st["status"] == 0, f
    assert st["target_page"] == sim.target, f
    assert st["special_offset"] == sim.sp_offset, f
    assert st["visible_pages"] == vis.patch_pages, f
    assert st["visible_special_pages"] == vis.special_pages, f
    assert st["last_page_len"] == vis.last_page_len, f
    assert st["visible_special_tokens"] == vis.special_tokens, f


def check_after_evict(st, sim, f):
    assert st["free_list"] == sim.free, f
    assert st["scale_pages"] == sim.scale, f
    assert st["window_pages"] == list(sim.window), f
    assert st["fresh"] == sim.fresh and st["n_special_tokens"] == sim.n_sp, f


# ---------------------------------------------------------------- bookkeeping

BOOK_CASES = [("wl", i) for i in range(5)] + [("small", k) for k in small_variants()]


@pytest.mark.parametrize("kind,key", BOOK_CASES, ids=[f"{a}-{b}" for a, b in BOOK_CASES])
def test_bookkeeping_bit_exact(kind, key):
    wl = WORKLOADS[key] if kind == "wl" else small_variants()[key]
    layers = 2 if wl.cached_layers > 1 else 1
    cache = make_cache(wl, layers=layers)
    run = Runner(wl, cache, layer=layers - 1)
    z = torch.zeros((wl.streams, wl.tokens, wl.heads, wl.head_dim), dtype=run.dt, device="cuda")
    sim = sim_for(wl)
    for f in range(wl.frames):
        commit = wl.is_keyframe(f)
        sim.append(f, commit)
        cache.append(run.layer, f, int(commit), z, z, z, run.q_rot)
        for s in range(wl.streams):
            check_state(cache.state(run.layer, s), sim, f)
        sim.evict()
        cache.evict(run.layer)
        if f % 7 == 0 or f == wl.frames - 1:
            check_after_evict(cache.state(run.layer, wl.streams - 1), sim, f)
    # layer 0 of a two-layer handle was never touched
    if layers == 2:
        st = cache.state(0, 0)
        assert st["n_visible_pages"] == 0 and st["fresh"] == 0
    info = cache.info()
    assert info["pool_pages"] == wl.scale_frames + wl.sliding_window + 1


def test_random_keyframe_masks_bit_exact():
    rnd = np.random.default_rng(5)
    for trial in range(4):
        sf, w = int(rnd.integers(0, 4)), int(rnd.integers(0, 5))
        spp = int(rnd.choice([6, 7, 16]))
        wl = small_variants()["small_tall"].replace(scale_frames=sf, sliding_window=w,
                                                   special_page_size=spp, frames=30)
        commits = rnd.random(30) < 0.5
        cache = make_cache(wl, max_keyframes=30)
        run = Runner(wl, cache)
        z = torch.zeros((1, wl.tokens, wl.heads, wl.head_dim), dtype=run.dt, device="cuda")
        sim = sim_for(wl)
        for f in range(30):
            sim.append(f, bool(commits[f]))
            cache.append(0, f, int(commits[f]), z, z, z, run.q_rot)
            check_state(cache.state(), sim, f)
            sim.evict()
            cache.evict(0)
            check_after_evict(cache.state(), sim, f)


def test_append_without_eviction_and_rollback():
    """Appends not followed by kv_evict_deferred replace each other in the
    tentative slot; kv_rollback drops a frame; both agree with the simulator."""
    wl = small_variants()["small_bf16"]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    z = torch.zeros((1, wl.tokens, wl.heads, wl.head_dim), dtype=run.dt, device="cuda")
    sim = sim_for(wl)
    script = [(0, 1, "evict"), (1, 1, "none"), (2, 1, "none"), (3, 1, "evict"), (4, 1, "rollback"),
              (5, 0, "evict"), (6, 1, "rollback"), (7, 1, "evict"), (8, 1, "evict"), (9, 1, "evict"),
              (10, 1, "rollback"), (11, 1, "evict")]
    for f, c, act in script:
        sim.append(f, bool(c))
        cache.append(0, f, c, z, z, z, run.q_rot)
        st = cache.state()
        check_state(st, sim, f)
        assert st["pending_commit"] == int(sim.pending is not None), f
        if act == "evict":
            sim.evict()
            cache.evict(0)
        elif act == "rollback":
            sim.rollback()
            cache.rollback(0)
        check_after_evict(cache.state(), sim, f)
        assert cache.state()["pending_commit"] == int(sim.pending is not None), f


def test_info_counts_appended_and_kept_frames():
    """kv_get_info's host counters across a skip-append, a rollback, an append
    replaced by a second one, and a reset; the device's committed special
    tokens agree (6 per kept frame)."""
    wl = small_variants()["small_bf16"]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    z = torch.zeros((1, wl.tokens, wl.heads, wl.head_dim), dtype=run.dt, device="cuda")
    script = [  # (frame, commit, action, appended, kept)
        (0, 1, "evict", 1, 1),
        (1, 0, "evict", 2, 1),        # skip-append: not kept
        (2, 1, "rollback", 3, 1),     # dropped
        (2, 1, "none", 4, 1),         # pending ...
        (3, 1, "evict", 5, 2),        # ... replaced by this one: one frame kept
        (4, 0, "rollback", 6, 2),
        (5, 1, "evict", 7, 3),
    ]
    for f, c, act, n_app, n_kept in script:
        cache.append(0, f, c, z, z, z, run.q_rot)
        if act == "evict":
            cache.evict(0)
        elif act == "rollback":
            cache.rollback(0)
            cache.evict(0)                 # a no-op after a rollback
        info = cache.info()
        assert (info["frames_appended"], info["frames_committed"]) == (n_app, n_kept), (f, act, info)
        assert cache.state()["n_special_tokens"] == wl.n_special * n_kept, (f, act)
    cache.reset(-1)
    info = cache.info()
    assert (info["frames_appended"], info["frames_committed"]) == (0, 0)


def test_special_stream_overflow_is_sticky_and_reset_recovers():
    wl = small_variants()["small_bf16"]
    cache = make_cache(wl, max_keyframes=3)
    run = Runner(wl, cache)
    z = torch.zeros((1, wl.tokens, wl.heads, wl.head_dim), dtype=run.dt, device="cuda")
    for f in range(3):
        cache.append(0, f, 1, z, z, z, run.q_rot)
        cache.evict(0)
    cache.append(0, 3, 0, z, z, z, run.q_rot)          # tentative: always fits
    cache.evict(0)
    assert cache.state()["status"] == 0
    cache.append(0, 4, 1, z, z, z, run.q_rot)
    cache.evict(0)                                       # a 4th keyframe does not fit
    st = cache.state()
    assert st["status"] == rp.RPKV_ENOSPACE and st["n_special_tokens"] == 18
    cache.append(0, 5, 1, z, z, z, run.q_rot)          # sticky: nothing written, nothing visible
    st = cache.state()
    assert st["status"] == rp.RPKV_ENOSPACE and st["n_visible_pages"] == 0
    cache.attend(0, run.q_rot, run.out, run.lse)       # empty visible set: zeros, lse -inf
    assert torch.all(run.out == 0) and torch.all(torch.isneginf(run.lse))
    cache.reset(0)
    cache.append(0, 0, 1, z, z, z, run.q_rot)
    st = cache.state()
    assert st["status"] == 0 and st["target_page"] == 0 and st["visible_pages"] == [0]


# ---------------------------------------------------------------- RoPE + pages

def _pages_for(cache, layer, s):
    kp, vp, ks, vs = cache.pool_views()
    return kp[layer, s], vp[layer, s], ks[layer, s], vs[layer, s]


@pytest.mark.parametrize("name", ["small_bf16", "small_f32", "small_partial_sp", "tiny", "small_rope2d",
                                  "small_rope2d_f32", "small_ntk", "small_cam"])
def test_rope_append_matches_oracle(name):
    wl = WORKLOADS[0] if name == "tiny" else small_variants()[name]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    ost = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t), storage_round=False)
    sim = sim_for(wl)
    perm = np.array([rp.vslot_perm(p) for p in range(64)])
    P, ns = wl.patches, wl.n_special
    for f in range(wl.frames):
        commit = wl.is_keyframe(f)
        q, k, v = run.inputs(f)
        sim.append(f, commit)
        cache.append(0, f, int(commit), q, k, v, run.q_rot)
        torch.cuda.synchronize()
        # q_rot against the fp64 rotation
        want_q = ost.rotate(qkv(wl, 0, 0, f, 0), f)
        got_q = run.q_rot[0].float().cpu().numpy()
        assert np.abs(got_q - want_q).max() <= tol(wl), f
        # K in the target page and the special stream
        kp, vp, ks, vs = _pages_for(cache, 0, 0)
        want_k = ost.rotate(qkv(wl, 0, 0, f, 1), f)
        t = sim.target
        got_kp = kp[:, t, :P].float().cpu().numpy().transpose(1, 0, 2)
        assert np.abs(got_kp - want_k[ns:]).max() <= tol(wl), f
        o = sim.sp_offset
        got_ks = ks[:, o:o + ns].float().cpu().numpy().transpose(1, 0, 2)
        assert np.abs(got_ks - want_k[:ns]).max() <= tol(wl), f
        # V bit-exact, transposed with the 16-slot storage order
        vin = v[0].cpu()
        vt = vp[:, t].cpu()                       # [H][D][cap]
        cap = vt.shape[-1]
        key_of_pos = (np.arange(cap) // 64) * 64 + perm[np.arange(cap) % 64]
        got_v = vt[:, :, np.argsort(key_of_pos)][:, :, :P].permute(2, 0, 1)
        assert torch.equal(got_v, vin[ns:]), f
        assert torch.all(vt[:, :, np.argsort(key_of_pos)][:, :, P:] == 0)   # padding stays zero
        spos = [(j // 64) * 64 + perm[j % 64] for j in range(o, o + ns)]
        got_vs = vs[:, :, spos].permute(2, 0, 1).cpu()
        assert torch.equal(got_vs, vin[:ns]), f
        cache.attend(0, run.q_rot, run.out, run.lse)
        sim.evict()
        cache.evict(0)


# ---------------------------------------------------------------- attention

def run_and_compare(wl, frames_to_check, rows=None, splits=0, heads=None, stream_ids=None):
    cache = make_cache(wl, splits=splits)
    run = Runner(wl, cache)
    ss = list(range(wl.streams)) if stream_ids is None else stream_ids
    orc = {s: OracleStream(wl, (lambda s_: (lambda f, t: qkv(wl, 0, s_, f, t)))(s)) for s in ss}
    worst = 0.0
    worst_lse = 0.0
    for f in range(wl.frames):
        commit = wl.is_keyframe(f)
        q, k, v = run.inputs(f)
        run.frame(f, q, k, v, commit)
        if f not in frames_to_check:
            continue
        torch.cuda.synchronize()
        r = np.arange(wl.frame_tokens(f)) if rows is None else np.asarray(rows(f))
        hs = np.arange(wl.heads) if heads is None else np.asarray(heads)
        got = run.out.float().cpu().numpy()
        got_lse = run.lse.cpu().numpy()
        for s in ss:
            o, lse = orc[s].attend(f, rows=r, heads=hs)
            err = np.abs(got[s][np.ix_(r, hs)] - o).max()
            lerr = np.abs(got_lse[s][np.ix_(hs, r)] - lse).max()
            worst, worst_lse = max(worst, err), max(worst_lse, lerr)
            assert err <= tol(wl), (f, s, err)
            assert lerr <= (F32_TOL if wl.dtype == "f32" else LSE_TOL), (f, s, lerr)
    return worst, worst_lse


@pytest.mark.parametrize("name", list(small_variants()))
def test_attention_small_all_rows(name):
    wl = small_variants()[name]
    if wl.chain_layers:
        wl = wl.replace(chain_layers=0)
    worst, wl_ = run_and_compare(wl, set(range(wl.frames)))
    print(f"{name}: max|out-oracle| {worst:.3e}  max|lse-oracle| {wl_:.3e}")


@pytest.mark.parametrize("splits", [1, 3, 64])
def test_attention_split_counts_agree(splits):
    """64 splits (the largest) over 3 to 9 key tiles: most splits get no tile,
    end empty (lse -inf) and must weigh nothing in the merge."""
    wl = small_variants()["small_skip"]
    run_and_compare(wl, {0, 5, 9, 19}, splits=splits)


@pytest.mark.parametrize("log2_scale", [17, -20])
def test_attention_is_linear_in_v_at_every_split_count(log2_scale):
    """V scaled by 2^k, k = 17 (|V| up to ~7e5, past fp16's largest value) and
    k = -20 (|V| ~ 1e-6, below fp16's normal range), at split counts 1, 3 and
    the automatic one.  Attention is linear in V and a power of two scales
    every product, partial and rounding exactly, so each output equals 2^k
    times the unscaled run of the same split count bit for bit, the LSE is
    unchanged, and the output is within 2^k * 2e-2 of the oracle fed the
    scaled V (the usual bar, relative to the scale of V)."""
    wl = small_variants()["small_skip"]
    k = float(2.0 ** log2_scale)

    def gen(scale):
        return lambda f, t: qkv(wl, 0, 0, f, t) * (scale if t == 2 else 1.0)

    orc = OracleStream(wl, gen(k))
    check = {0, 3, 9, 19}
    for splits in (1, 3, 0):
        outs = {}
        for scale in (1.0, k):
            cache = make_cache(wl, splits=splits)
            run = Runner(wl, cache)
            g = gen(scale)
            got = {}
            for f in range(wl.frames):
                q, kk, v = (to_dev(g(f, t)[None], run.dt) for t in range(3))
                run.frame(f, q, kk, v, wl.is_keyframe(f))
                if f in check:
                    got[f] = (run.out.clone(), run.lse.clone())
            outs[scale] = got
            if splits == 0:
                assert cache.info()["attn_splits"] > 1
        for f in check:
            o1, l1 = outs[1.0][f]
            ok, lk = outs[k][f]
            assert torch.isfinite(ok.float()).all(), (splits, f)
            assert torch.equal(ok, (o1.float() * k).to(ok.dtype)), (splits, f)
            assert torch.equal(lk, l1), (splits, f)
            o, lse = orc.attend(f)
            err = np.abs(ok[0].float().cpu().numpy() - o).max()
            assert err <= BF16_TOL * k, (splits, f, err / k)
            assert np.abs(lk[0].cpu().numpy() - lse).max() <= LSE_TOL, (splits, f)


def test_tiny_f32_full():
    wl = WORKLOADS[0]
    worst, worst_lse = run_and_compare(wl, set(range(wl.frames)))
    print(f"tiny f32: max|out-oracle| {worst:.3e}  max|lse-oracle| {worst_lse:.3e}")


def sampled_rows(wl, n_patch=40, seed=0):
    def rows(f):
        rng = np.random.default_rng(seed + f)
        pr = rng.choice(np.arange(wl.n_special + 1, wl.tokens - 1), n_patch, replace=False)
        return np.unique(np.r_[np.arange(wl.n_special), wl.n_special, wl.tokens - 1, pr])
    return rows


def test_single_layer_37x37_sampled():
    wl = WORKLOADS[1]
    frames = {0, 1, 7, 8, 23, 24, 25, 40, 63}
    worst, worst_lse = run_and_compare(wl, frames, rows=sampled_rows(wl))
    print(f"37x37 single layer: max|out-oracle| {worst:.3e}  max|lse-oracle| {worst_lse:.3e}")


def test_single_layer_37x37_all_rows_at_transitions():
    """The 37x37 stream in full on three frames: every query row of every head
    at the first eviction (frame 24), the first recycled page (frame 25) and
    the last frame (63), against the float64 oracle."""
    wl = WORKLOADS[1]
    worst, worst_lse = run_and_compare(wl, {24, 25, 63})
    print(f"37x37 all rows at frames 24, 25, 63: max|out-oracle| {worst:.3e}  max|lse-oracle| {worst_lse:.3e}")


@pytest.mark.parametrize("splits", [0, 3, 7])
def test_variable_patch_grids(splits):
    """Frames of their own grids (9x11, 7x11, 5x6, 1x1, 9x7 in a 9x11 page):
    pages record their token counts, q_rot and K follow each frame's grid,
    attention reads the valid tokens of every page and answers the frame's
    own tokens only (the rows past them keep what they held).  Pages of one
    and of two key tiles mix, so splits start inside pages of either kind."""
    wl = small_variants()["small_vargrid"]
    cache = make_cache(wl, splits=splits)
    run = Runner(wl, cache)
    sim = sim_for(wl)
    orc = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t))
    ns = wl.n_special
    for f in range(wl.frames):
        gh, gw = wl.grid_of(f)
        n = ns + gh * gw
        commit = wl.is_keyframe(f)
        q, k, v = run.inputs(f)
        run.out.fill_(7.0)
        run.lse.fill_(7.0)
        run.frame(f, q, k, v, commit, evict=False)
        sim.append(f, commit)
        st = cache.state(0, 0)
        assert st["query_tokens"] == n, f
        want_pt = {p: wl.grid_of(g)[0] * wl.grid_of(g)[1] for p, g in sim.page_frame.items()}
        want_pt[sim.target] = gh * gw
        for p, cnt in want_pt.items():
            assert st["page_tokens"][p] == cnt, (f, p)
        torch.cuda.synchronize()
        got_q = run.q_rot[0, :n].float().cpu().numpy()
        assert np.abs(got_q - orc.q_rot(f)).max() <= BF16_TOL, f
        kp = _pages_for(cache, 0, 0)[0]
        got_k = kp[:, sim.target, :gh * gw].float().cpu().numpy().transpose(1, 0, 2)
        assert np.abs(got_k - orc.kv(f)[0][ns:]).max() <= BF16_TOL, f
        o, lse = orc.attend(f)
        assert np.abs(run.out[0, :n].float().cpu().numpy() - o).max() <= BF16_TOL, f
        assert np.abs(run.lse[0, :, :n].cpu().numpy() - lse).max() <= LSE_TOL, f
        assert torch.all(run.out[0, n:] == 7.0) and torch.all(run.lse[0, :, n:] == 7.0), f
        sim.evict()
        cache.evict(0)


@pytest.mark.parametrize("splits", [0, 5])
def test_variable_grids_37x37_through_eviction(splits):
    """37x37 pages holding frames of five grids (whole, 33x33, 20x30, 37x36,
    1x1: 22, 18, 10, 21 and 1 key tiles) through the first eviction (frame
    24) and recycled pages: the attention walks each page's own tiles and
    the splits cut across pages of different lengths.  Sampled rows of each
    frame's own tokens (specials, first and last patch, 40 others) against
    the float64 oracle."""
    wl = WORKLOADS[1].replace(name="vargrid_37x37", frames=30,
                              grids=((37, 37), (33, 33), (20, 30), (37, 36), (1, 1)))

    def rows(f):
        n = wl.frame_tokens(f)
        rng = np.random.default_rng(f)
        inner = np.arange(wl.n_special + 1, max(n - 1, wl.n_special + 1))
        pr = rng.choice(inner, min(40, len(inner)), replace=False) if len(inner) else []
        return np.unique(np.r_[np.arange(min(n, wl.n_special + 1)), n - 1, pr].astype(int))

    worst, worst_lse = run_and_compare(wl, {3, 4, 9, 23, 24, 25, 29}, rows=rows, splits=splits)
    print(f"variable grids 37x37, splits {splits}: max|out-oracle| {worst:.3e}  max|lse-oracle| {worst_lse:.3e}")


def test_append_grid_is_checked():
    wl = small_variants()["small_vargrid"]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    q, k, v = run.inputs(0)
    for grid in ((10, 11), (9, 12), (0, 5), (12, 9)):
        with pytest.raises(rp.RpkvError):
            cache.append(0, 0, 1, q, k, v, run.q_rot, grid=grid)


def test_attention_large_logits_move_the_reference_max():
    """Peaked softmax: Q scaled by 3 and the keys of frame f by 1 + f/2, so
    the scores span hundreds of base-2 units and later pages beat the running
    max of earlier ones by more than 2^8 thousands of times.

    The kernel rotates K in fp32 and the oracle exactly, both rounding to
    bf16, so a rotated key element can differ by one bf16 ulp (checked
    below: never more, and rarely).  Such a difference moves a score by
    |q_d| * ulp, about 3 * 2^-5 = 0.1 (0.012 in natural-log units of the
    scaled score): the LSE is therefore held to 5e-2 here, the outputs to
    the usual 2e-2."""
    wl = small_variants()["small_bf16"]

    def gen(f, t):
        x = qkv(wl, 0, 0, f, t)
        if t == 0:
            x = x * 3.0
        elif t == 1:
            x = x * (1.0 + 0.5 * f)
        return round_to_bf16(x)

    cache = make_cache(wl)
    run = Runner(wl, cache)
    orc = OracleStream(wl, lambda f, t: gen(f, t))
    sim = sim_for(wl)
    worst, worst_lse, flips, total = 0.0, 0.0, 0, 0
    for f in range(wl.frames):
        q, k, v = (to_dev(gen(f, t)[None], run.dt) for t in range(3))
        commit = wl.is_keyframe(f)
        run.cache.append(0, f, int(commit), q, k, v, run.q_rot)
        sim.append(f, commit)
        # rotated K of the frame's patches in its page: within one bf16 ulp
        kp = _pages_for(cache, 0, 0)[0]
        got_k = kp[:, sim.target, :wl.patches].float().cpu().numpy().transpose(1, 0, 2)
        want_k = rope3d.round_bf16(orc.rotate(gen(f, 1), f))[wl.n_special:]
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want_k), 1e-30))) - 7)
        d = np.abs(got_k - want_k)
        assert np.all(d <= ulp), f
        flips += int((d > 0).sum())
        total += d.size
        run.cache.attend(0, run.q_rot, run.out, run.lse)
        o, lse = orc.attend(f)
        err = np.abs(run.out[0].float().cpu().numpy() - o).max()
        lerr = np.abs(run.lse[0].cpu().numpy() - lse).max()
        worst, worst_lse = max(worst, err), max(worst_lse, lerr)
        assert err <= BF16_TOL, (f, err)
        assert lerr <= 5e-2, (f, lerr)
        sim.evict()
        run.cache.evict(0)
    assert flips <= 1e-3 * total, (flips, total)
    print(f"large logits: max|out-oracle| {worst:.3e}  max|lse-oracle| {worst_lse:.3e}  "
          f"K elements one ulp off: {flips}/{total}")


def test_visibility_probe_q_zero():
    """Q = 0, V = one-hot of (frame mod 64) in head 0 (patches) and head 1
    (specials): the output is the histogram of visible frames."""
    wl = small_variants()["small_skip"]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    sim = sim_for(wl)
    for f in range(wl.frames):
        commit = wl.is_keyframe(f)
        _, k, _ = run.inputs(f)
        q = torch.zeros_like(k)
        v = np.zeros((1, wl.tokens, wl.heads, wl.head_dim), np.float32)
        v[0, wl.n_special:, 0, f % 64] = 1
        v[0, :wl.n_special, 1, f % 64] = 1
        run.frame(f, q, k, to_dev(v, run.dt), commit, evict=False)
        sim.append(f, commit)
        pf = sim.visible_patch_frames(f)
        spf = sim.special_frames + [f]
        total = len(pf) * wl.patches + len(spf) * wl.n_special
        want0 = np.zeros(64)
        want1 = np.zeros(64)
        for g in pf:
            want0[g % 64] += wl.patches / total
        for g in spf:
            want1[g % 64] += wl.n_special / total
        out = run.out[0].float().cpu().numpy()
        assert np.abs(out[:, 0] - want0).max() <= 2.0 ** -8, f
        assert np.abs(out[:, 1] - want1).max() <= 2.0 ** -8, f
        assert np.abs(run.lse[0].cpu().numpy() - math.log(total)).max() < 1e-4
        sim.evict()
        cache.evict(0)


def test_windowed_inference_restarts_on_a_fresh_cache():
    """Windows of 7 frames (not a multiple of the keyframe interval): kv_reset at every window start, frames keep their
    global index (temporal position), and each window sees only its own
    stored frames."""
    wl = small_variants()["small_skip"]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    win = 7
    for f in range(wl.frames):
        if f % win == 0:
            cache.reset(0)
            orc = OracleStream(wl, lambda f_, t: qkv(wl, 0, 0, f_, t), window_start=f)
        q, k, v = run.inputs(f)
        run.frame(f, q, k, v, wl.is_keyframe(f))
        torch.cuda.synchronize()
        o, lse = orc.attend(f)
        assert np.abs(run.out[0].float().cpu().numpy() - o).max() <= BF16_TOL, f
        assert np.abs(run.lse[0].cpu().numpy() - lse).max() <= LSE_TOL, f


def test_hip_graph_replays_follow_the_device_bookkeeping():
    """attend_frame captured once in a HIP graph (main kernel and split
    merge), then replayed after each eager append as the cache fills, evicts
    and recycles: every replay equals an eager call on the same state.  A
    whole frame step (append, attend, evict) captured and replayed equals the
    eager step too.  Nothing on the path synchronises with the host."""
    wl = small_variants()["small_skip"]
    cache = make_cache(wl, splits=3)
    run = Runner(wl, cache)
    out_g = torch.empty_like(run.out)
    lse_g = torch.empty_like(run.lse)
    q, k, v = run.inputs(0)
    cache.append(0, 0, 1, q, k, v, run.q_rot)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cache.attend(0, run.q_rot, out_g, lse_g)
    cache.evict(0)
    for f in range(1, wl.frames):
        q, k, v = run.inputs(f)
        cache.append(0, f, int(wl.is_keyframe(f)), q, k, v, run.q_rot)
        g.replay()
        cache.attend(0, run.q_rot, run.out, run.lse)
        torch.cuda.synchronize()
        assert torch.equal(out_g, run.out) and torch.equal(lse_g, run.lse), f
        cache.evict(0)

    # a whole step captured for frame F, replayed after eager frames 0..F-1
    F = 7
    eager = make_cache(wl, splits=3)
    graphed = make_cache(wl, splits=3)
    re, rg = Runner(wl, eager), Runner(wl, graphed)
    for f in range(F):
        q, k, v = re.inputs(f)
        re.frame(f, q, k, v, wl.is_keyframe(f))
        rg.frame(f, q, k, v, wl.is_keyframe(f))
    q, k, v = re.inputs(F)
    torch.cuda.synchronize()
    gs = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gs):
        rg.frame(F, q, k, v, wl.is_keyframe(F))
    gs.replay()
    re.frame(F, q, k, v, wl.is_keyframe(F))
    torch.cuda.synchronize()
    assert torch.equal(rg.out, re.out) and torch.equal(rg.lse, re.lse)
    assert graphed.state(0, 0) == eager.state(0, 0)


def test_replay_is_bitwise_deterministic():
    wl = small_variants()["small_skip"]
    outs = []
    for rep in range(2):
        cache = make_cache(wl)
        run = Runner(wl, cache)
        acc = []
        for f in range(wl.frames):
            q, k, v = run.inputs(f)
            run.frame(f, q, k, v, wl.is_keyframe(f))
            acc.append(run.out.clone())
        outs.append(torch.stack(acc))
    assert torch.equal(outs[0], outs[1])


def test_binding_checks_tensor_shapes_before_launch():
    """The C ABI takes bare pointers; the torch convenience layer refuses a
    tensor of the wrong shape, dtype or layout before anything is launched."""
    wl = small_variants()["small_bf16"]
    cache = make_cache(wl)
    run = Runner(wl, cache)
    q, k, v = run.inputs(0)
    with pytest.raises(ValueError):
        cache.append(0, 0, 1, q[:, :-1], k, v, run.q_rot)
    with pytest.raises(ValueError):
        cache.append(0, 0, 1, q.float(), k, v, run.q_rot)
    with pytest.raises(ValueError):
        cache.append(0, 0, 1, q.transpose(1, 2).contiguous().transpose(1, 2), k, v, run.q_rot)
    with pytest.raises(ValueError):
        cache.attend(0, run.q_rot, run.out, run.lse[:, :, :-1])
    st = cache.state(0, 0)
    assert st["query_tokens"] == 0 and st["n_visible_pages"] == 0   # nothing ran
    cache.append(0, 0, 1, q, k, v, run.q_rot)
    cache.attend(0, run.q_rot, run.out, run.lse)
    torch.cuda.synchronize()
    assert cache.state(0, 0)["query_tokens"] == wl.tokens


def test_maximum_pool_of_512_pages():
    """The largest pool a cache takes (scale_frames + sliding_window + 1 = 512
    pages): the window fills to 509 pages, the visible table reaches 512
    entries (two passes of the frame record's 256 threads, 512 one-tile pages
    of 6 keys each in the attention walk) and pages recycle; bookkeeping
    bit-exact against the page simulator, attention against the oracle.  A
    513-page pool is refused."""
    from rpkv_inputs import Workload
    wl = Workload("max_pool_2x3", "bf16", frames=530, grid_h=2, grid_w=3, heads=2,
                  scale_frames=2, sliding_window=509, keyframe_interval=1)
    cache = make_cache(wl)
    run = Runner(wl, cache)
    sim = sim_for(wl)
    orc = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t))
    check = {0, 255, 256, 300, 510, 511, 512, 529}
    for f in range(wl.frames):
        q, k, v = run.inputs(f)
        sim.append(f, True)
        run.frame(f, q, k, v, True, evict=False)
        if f in check:
            st = cache.state(0, 0)
            check_state(st, sim, f)
            assert len(st["visible_pages"]) == min(f + 1, 512), f
            torch.cuda.synchronize()
            o, lse = orc.attend(f)
            assert np.abs(run.out[0].float().cpu().numpy() - o).max() <= BF16_TOL, f
            assert np.abs(run.lse[0].cpu().numpy() - lse).max() <= LSE_TOL, f
        sim.evict()
        cache.evict(0)
    check_after_evict(cache.state(0, 0), sim, wl.frames)
    with pytest.raises(rp.RpkvError):
        make_cache(wl.replace(sliding_window=510))
