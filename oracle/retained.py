"""The set of tokens one frame attends to, enumerated directly from the cache
policy (no pages involved).

Policy, as the pages state it:

* patch stream: the first ``scale_frames`` stored frames stay for good; later
  stored frames form a sliding window of the ``sliding_window`` most recent
  ones, the oldest leaving first (page "How 3D RoPE Positional Encoding Works
  with the Paged KV Cache in LingBot-Map", section "Dual-Stream Memory Layout";
  page "How LingBot-Map Achieves Real-Time 3D Reconstruction", section "Cache
  Eviction and Output Generation");
* special stream: the 6 special tokens of every stored frame are kept forever
  (same page, section "Dual-Stream Memory Layout");
* only keyframes are stored; a non-keyframe is processed and attends, but its
  K/V are not kept (page "KV Caching Benefits in Ling Bot-Map", section
  "Reduced KV Growth via Keyframe Streaming"); eviction is deferred until after
  the frame is processed (same page, "Memory-Efficient Sliding Window
  Management");
* the frame being processed attends to all its own tokens and to the retained
  tokens of past frames, never to later frames (page "How LingBot-Map Achieves
  Real-Time 3D Reconstruction", section "Per-Frame Processing and Causal
  Attention").

Readings: a frame is a keyframe iff ``f % interval == 0``; the window counts
stored frames after the scale frames (scale frames are not part of it); the
frame's own patches and specials are visible to itself whether or not it is
stored; eviction runs after the frame's attention, so a stored frame sees
``scale_frames`` + up to ``sliding_window`` earlier window frames + itself.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


def keyframes_before(frame: int, interval: int) -> List[int]:
    """Stored frames before ``frame`` under the fixed-interval schedule."""
    if interval <= 0:
        return []
    return [k for k in range(frame) if k % interval == 0]


def visible_frames(frame: int, stored_before: Sequence[int], scale_frames: int,
                   sliding_window: int) -> Tuple[List[int], List[int]]:
    """(patch frames, special frames) visible to ``frame``.

    ``stored_before`` lists the stored frames before ``frame`` in order.
    Patch frames come in the order scale -> window (oldest first) -> frame."""
    ks = list(stored_before)
    m = len(ks)
    scale = ks[:min(m, scale_frames)]
    window = ks[max(scale_frames, m - sliding_window):m]
    patch = scale + window + [frame]
    special = ks + [frame]
    return patch, special


def visible_for_schedule(frame: int, interval: int, scale_frames: int, sliding_window: int):
    """``visible_frames`` under the fixed-interval keyframe schedule (interval 0: nothing stored)."""
    return visible_frames(frame, keyframes_before(frame, interval), scale_frames, sliding_window)


def token_list(patch_frames: Sequence[int], special_frames: Sequence[int], n_special: int,
               n_patches: int) -> List[Tuple[int, int]]:
    """Explicit (frame, token index) list of the retained set: the patch tokens
    of the patch frames, then the special tokens of the special frames."""
    out = []
    for f in patch_frames:
        out.extend((f, n_special + p) for p in range(n_patches))
    for f in special_frames:
        out.extend((f, s) for s in range(n_special))
    return out
