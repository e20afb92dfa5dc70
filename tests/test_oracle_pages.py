"""Pins of the page simulator and the retained-set enumeration: hand-traced
fixtures (tests/golden), the closed form of the page id of a stored frame,
structural invariants, and the cross-check between the two independent
descriptions (pages vs. direct enumeration)."""
import collections
import os
import random

import pytest

from oracle import pages, retained
from rpkv_inputs import WORKLOADS, small_variants

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append([c.strip() for c in line.split("|")])
    return out


def _ints(s):
    return [] if s == "-" else [int(t) for t in s.split()]


def run_sim(wl, frames=None, interval=None, commits=None):
    sim = pages.PageSim(wl.scale_frames, wl.sliding_window, wl.special_page_size, wl.n_special)
    iv = wl.keyframe_interval if interval is None else interval
    n = wl.frames if frames is None else frames
    for f in range(n):
        c = (f % iv == 0) if commits is None else commits[f]
        assert sim.append(f, c) == pages.OK
        yield f, c, sim
        sim.evict()


def test_tiny_trace_matches_hand_trace():
    wl = WORKLOADS[0]
    rows = _rows("evict_trace_tiny.txt")
    sim = pages.PageSim(wl.scale_frames, wl.sliding_window, wl.special_page_size, wl.n_special)
    for f, row in enumerate(rows):
        assert int(row[0]) == f
        sim.append(f, True)
        assert sim.target == int(row[1])
        assert sim.visible.patch_pages == _ints(row[2])
        assert sim.visible.special_pages == f + 1 and sim.visible.last_page_len == 6
        assert sim.evict() == _ints(row[3])
        assert sim.free == _ints(row[4])
    assert list(sim.window) == [2, 3, 4, 5]
    assert [sim.page_frame[p] for p in [0, 2, 3, 4, 5]] == [0, 12, 13, 14, 15]


def test_partial_special_pages_trace():
    wl = small_variants()["small_partial_sp"].replace(grid_h=1, grid_w=3)
    rows = _rows("partial_special_pages.txt")
    sim = pages.PageSim(1, 4, 16, 6)
    for row in rows:
        f, key = int(row[0]), bool(int(row[1]))
        sim.append(f, key)
        assert (sim.visible.special_pages, sim.visible.last_page_len) == (int(row[2]), int(row[3]))
        assert sim.target == int(row[4])
        assert sim.visible.patch_pages == _ints(row[5])
        sim.evict()
    assert wl.special_page_size == 16


def test_long_stream_transitions():
    wl = WORKLOADS[2]
    want = {int(r[0]): r for r in _rows("long_stream_transitions.txt")}
    sim = pages.PageSim(wl.scale_frames, wl.sliding_window, wl.special_page_size, wl.n_special)
    for f in range(wl.frames):
        c = wl.is_keyframe(f)
        sim.append(f, c)
        vis = sim.visible
        freed = sim.evict()
        if f in want:
            r = want[f]
            assert sim.target == int(r[1]) and c == bool(int(r[2]))
            assert len(vis.patch_pages) == int(r[3])
            assert vis.special_pages == int(r[5]) and vis.last_page_len == 6
            assert freed == _ints(r[4])
    assert vis.special_tokens == 1236 and sim.n_sp == 1230
    assert sim.fresh == 73 and sim.free == [10]


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4])
def test_closed_form_page_ids(cid):
    wl = WORKLOADS[cid]
    sf, w = wl.scale_frames, wl.sliding_window
    j = 0
    for f, c, sim in run_sim(wl):
        if c:
            want = j if j < sf else sf + ((j - sf) % (w + 1))
            assert sim.target == want
            j += 1
    assert j == wl.n_keyframes() and sim.n_sp == 6 * j


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4])
def test_pages_agree_with_enumeration(cid):
    wl = WORKLOADS[cid]
    for f, c, sim in run_sim(wl):
        pf, spf = retained.visible_for_schedule(f, wl.keyframe_interval, wl.scale_frames,
                                                wl.sliding_window)
        assert sim.visible_patch_frames(f) == pf
        want_sp = len(spf) * wl.n_special
        assert sim.visible.special_tokens == want_sp
        assert sim.special_frames + [f] == spf


def test_random_keyframe_masks_agree_and_invariants():
    rnd = random.Random(11)
    for trial in range(60):
        sf, w = rnd.randint(0, 4), rnd.randint(0, 6)
        spp = rnd.choice([6, 7, 16])
        n = rnd.randint(1, 60)
        commits = [rnd.random() < 0.5 for _ in range(n)]
        sim = pages.PageSim(sf, w, spp, 6)
        stored = []
        pool = set(range(sf + w + 1))
        for f in range(n):
            assert sim.append(f, commits[f]) == pages.OK
            pf, spf = retained.visible_frames(f, stored, sf, w)
            assert sim.visible_patch_frames(f) == pf
            vis = sim.visible
            assert len(set(vis.patch_pages)) == len(vis.patch_pages)
            assert vis.special_tokens == 6 * len(spf)
            assert vis.special_pages == -(-vis.special_tokens // spp)
            assert 1 <= vis.last_page_len <= spp
            assert (vis.special_pages - 1) * spp + vis.last_page_len == vis.special_tokens
            scale_before = list(sim.scale)
            sim.evict()
            assert len(sim.window) <= w and sim.scale[:len(scale_before)] == scale_before
            used = set(sim.scale) | set(sim.window)
            assert not (used & set(sim.free))
            assert used | set(sim.free) | set(range(sim.fresh, sf + w + 1)) == pool
            if commits[f]:
                stored.append(f)


def test_append_without_eviction_replaces_the_pending_frame():
    sim = pages.PageSim(1, 2, 6, 6)       # pool of 4 pages
    for f in range(6):                    # never evicted: nothing is kept
        assert sim.append(f, True) == pages.OK
        assert sim.target == 0 and sim.visible.patch_pages == [0]
    sim.evict()                           # keeps frame 5 only
    assert sim.scale == [0] and sim.page_frame == {0: 5} and sim.special_frames == [5]


def test_rollback_drops_the_frame():
    sim = pages.PageSim(1, 2, 6, 6)
    sim.append(0, True)
    sim.evict()
    sim.append(1, True)
    sim.rollback()
    sim.evict()
    assert sim.window == collections.deque() and sim.n_sp == 6
    sim.append(2, True)
    assert sim.target == 1
    sim.evict()
    assert list(sim.window) == [1] and sim.page_frame[1] == 2


def test_special_capacity_overflow():
    sim = pages.PageSim(1, 2, 6, 6, special_capacity=12)
    for f in range(2):
        assert sim.append(f, True) == pages.OK
        sim.evict()
    assert sim.append(2, False) == pages.OK        # the tentative slot always fits
    sim.evict()
    assert sim.append(3, True) == pages.OK
    sim.evict()                                    # keeping it would exceed 12 tokens
    assert sim.status == pages.ENOSPACE
    assert sim.append(4, True) == pages.ENOSPACE   # sticky
    sim.reset()
    assert sim.append(0, True) == pages.OK and sim.target == 0


def test_keyframe_storage_reduction():
    # a keyframe every 5th frame stores 1/5 of the frames (the pages' 80% figure)
    wl = WORKLOADS[2]
    assert wl.n_keyframes() == 205
    assert 1 - wl.n_keyframes() / wl.frames == pytest.approx(0.8, abs=0.001)


@pytest.mark.parametrize("start", [0, 6, 7])
def test_window_start_matches_a_fresh_simulator(start):
    """Windowed inference restarts on a fresh cache: the oracle stream's
    visible frames from `window_start` on equal those of a page simulator
    that is created at the window's first frame and fed only the window's
    frames (keyframe schedule and frame indices unchanged)."""
    from oracle.stream import OracleStream
    wl = small_variants()["small_skip"]          # keyframe every 3rd frame
    orc = OracleStream(wl, lambda f, t: None, window_start=start)
    sim = pages.PageSim(wl.scale_frames, wl.sliding_window, wl.special_page_size, wl.n_special)
    for f in range(start, wl.frames):
        assert sim.append(f, wl.is_keyframe(f)) == pages.OK
        pf, sf = orc.visible(f)
        assert list(pf) == sim.visible_patch_frames(f), (start, f)
        assert list(sf) == sim.special_frames + [f], (start, f)   # stored specials, then the frame's own
        assert all(g >= start for g in pf) and all(g >= start for g in sf), (start, f)
        sim.evict()
