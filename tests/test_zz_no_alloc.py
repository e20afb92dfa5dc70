"""attend_frame_noalloc (split scratch in the library's static array, no
allocation) against attend_frame on the same cache state: bit for bit, on two
calls in a row, the second with a smaller input; and its size limit."""
import pytest
import torch

import rope_paged_kv_amd as rp
from gpu_harness import Runner, make_cache
from rpkv_inputs import WORKLOADS, small_variants

pytestmark = pytest.mark.gpu


def _frames_then_both(wl, frames, splits=0):
    """Runs frames 0..frames-1 through append -> attend -> evict, then appends
    the next frame and answers it with both entry points."""
    cache = make_cache(wl, splits=splits)
    run = Runner(wl, cache)
    for f in range(frames):
        q, k, v = run.inputs(f)
        run.frame(f, q, k, v, wl.is_keyframe(f))
    q, k, v = run.inputs(frames)
    cache.append(0, frames, int(wl.is_keyframe(frames)), q, k, v, run.q_rot)
    out_n = torch.full_like(run.out, 3.0)
    lse_n = torch.full_like(run.lse, 3.0)
    cache.attend_noalloc(0, run.q_rot, out_n, lse_n)
    cache.attend(0, run.q_rot, run.out, run.lse)
    torch.cuda.synchronize()
    return cache, run, out_n, lse_n


def test_noalloc_matches_attend_frame_on_two_calls_second_smaller():
    # first call: 37x37 frames, 16 heads, 7 splits (~21 MB of scratch)
    wl = WORKLOADS[1].replace(frames=4)
    cache, run, out_n, lse_n = _frames_then_both(wl, 3)
    assert cache.info()["attn_splits"] > 1
    assert torch.equal(out_n, run.out) and torch.equal(lse_n, run.lse)
    # second call, smaller: 7x13 frames, 3 heads, 3 splits; the scratch still
    # holds the first call's rows and must not leak into this one
    wl2 = small_variants()["small_skip"]
    cache2, run2, out2, lse2 = _frames_then_both(wl2, 9, splits=3)
    assert torch.equal(out2, run2.out) and torch.equal(lse2, run2.lse)
    # one split: the scratch is not used
    cache3, run3, out3, lse3 = _frames_then_both(wl2, 5, splits=1)
    assert torch.equal(out3, run3.out) and torch.equal(lse3, run3.lse)


def test_noalloc_refuses_a_split_scratch_past_its_limit():
    wl = WORKLOADS[1].replace(frames=2)
    cache = make_cache(wl, splits=64)          # 16 * 64 * 1375 * 136 B > 128 MiB
    run = Runner(wl, cache)
    q, k, v = run.inputs(0)
    cache.append(0, 0, 1, q, k, v, run.q_rot)
    with pytest.raises(rp.RpkvError) as e:
        cache.attend_noalloc(0, run.q_rot, run.out, run.lse)
    assert e.value.code == rp.RPKV_ETOOBIG
    cache.attend(0, run.q_rot, run.out, run.lse)   # the workspace entry point still runs
    torch.cuda.synchronize()
