"""Page-level simulator of the dual-stream paged KV cache (one layer, one stream).

Written from page "How 3D RoPE Positional Encoding Works with the Paged KV
Cache in LingBot-Map", sections "Dual-Stream Memory Layout", "Frame Appending
and Position Encoding Integration" and "Attention Computation with Cached
RoPE", and page "KV Caching Benefits in Ling Bot-Map", sections
"Memory-Efficient Sliding Window Management" and "Reduced KV Growth via
Keyframe Streaming":

* patch stream: one page holds one frame's patch tokens; pages come from a
  free list when it has any, otherwise from the never-used pages in ascending
  id order; the first ``scale_frames`` stored pages are permanent, the later
  ones form the window, and a deferred eviction moves the oldest window pages
  back to the free list while the window holds more than ``sliding_window``;
* special stream: append-only, 6 tokens per stored frame, pages of
  ``special_page_size`` tokens filled in order and never evicted;
* visible page table: scale pages, then window pages oldest first, then all
  special pages; the number of valid tokens in the last special page is the
  last-page length.

Every appended frame first goes to the *tentative slot* -- the page the next
stored frame would take and the special tokens right after the stored ones --
where its own attention sees it; the deferred-eviction call keeps it if it is
a keyframe, a rollback (or skip-append) drops it (page "KV Caching Benefits in
Ling Bot-Map", section "Dynamic Keyframe Selection": the deferred-eviction
call is what keeps a keyframe's KV, and a rollback discards the temporary
entry).

Readings (the pages are silent): the free list is a stack (last in, first
out); the frame being processed is listed after the window.  The free
list never holds more than one page in the workloads, so the stack order does
not change any page id there.
"""
from __future__ import annotations

import collections
from dataclasses import dataclass, field
from typing import Dict, List, Optional

OK = 0
ENOSPACE = -3


@dataclass
class Visible:
    patch_pages: List[int]
    special_pages: int          # special pages 0 .. special_pages-1
    last_page_len: int
    special_tokens: int         # total special tokens visible


@dataclass
class PageSim:
    scale_frames: int
    sliding_window: int
    special_page_size: int = 6
    n_special: int = 6
    pool_pages: Optional[int] = None        # default scale_frames + sliding_window + 1
    special_capacity: Optional[int] = None  # in tokens; default unlimited

    fresh: int = 0
    free: List[int] = field(default_factory=list)
    scale: List[int] = field(default_factory=list)
    window: collections.deque = field(default_factory=collections.deque)
    n_sp: int = 0
    status: int = OK
    visible: Optional[Visible] = None
    target: int = -1                # page written by the last append
    sp_offset: int = 0              # first special token written by the last append
    page_frame: Dict[int, int] = field(default_factory=dict)   # committed page -> frame
    special_frames: List[int] = field(default_factory=list)    # stored frames, append order
    pending: Optional[tuple] = None         # (frame, page) of an appended keyframe not yet kept

    def __post_init__(self):
        if self.pool_pages is None:
            self.pool_pages = self.scale_frames + self.sliding_window + 1

    def next_page(self) -> Optional[int]:
        if self.free:
            return self.free[-1]
        if self.fresh < self.pool_pages:
            return self.fresh
        return None

    def _special_visible(self, tokens: int) -> Visible:
        sp = self.special_page_size
        pages = (tokens + sp - 1) // sp
        last = tokens - (pages - 1) * sp if pages else 0
        return Visible([], pages, last, tokens)

    def append(self, frame: int, commit: bool) -> int:
        """Append one frame to the tentative slot (``commit`` False: skip-append).

        The frame sees its own tokens; whether it is kept is decided by the
        deferred eviction (``evict``), which retains a keyframe, or by
        ``rollback``, which drops it.  Returns the status."""
        if self.status != OK:
            return self.status
        t = self.next_page()
        if t is None:
            self.status = ENOSPACE
            self.visible = Visible([], 0, 0, 0)
            self.pending = None
            return self.status
        self.target, self.sp_offset = t, self.n_sp
        vis = self._special_visible(self.n_sp + self.n_special)
        vis.patch_pages = self.scale + list(self.window) + [t]
        self.visible = vis
        self.pending = (frame, t) if commit else None
        return OK

    def rollback(self):
        """Drop the last appended frame (it is not kept)."""
        self.pending = None

    def evict(self) -> List[int]:
        """Deferred eviction: keep the pending keyframe, then move the oldest
        window pages to the free list while the window holds more than
        ``sliding_window``.  Returns the pages freed."""
        out = []
        if self.status != OK:
            return out
        if self.pending is not None:
            frame, t = self.pending
            self.pending = None
            cap = self.special_capacity
            if cap is not None and self.n_sp + self.n_special > cap:
                self.status = ENOSPACE
                return out
            if self.free:
                self.free.pop()
            else:
                self.fresh += 1
            if len(self.scale) < self.scale_frames:
                self.scale.append(t)
            else:
                self.window.append(t)
            self.page_frame[t] = frame
            self.special_frames.append(frame)
            self.n_sp += self.n_special
        while len(self.window) > self.sliding_window:
            p = self.window.popleft()
            self.page_frame.pop(p, None)
            self.free.append(p)
            out.append(p)
        return out

    def reset(self):
        self.fresh, self.n_sp, self.status = 0, 0, OK
        self.free, self.scale, self.window = [], [], collections.deque()
        self.visible, self.target, self.sp_offset = None, -1, 0
        self.page_frame, self.special_frames = {}, []
        self.pending = None

    def visible_patch_frames(self, frame: int) -> List[int]:
        """Frames whose patches the current visible table shows (``frame`` for
        the tentative page)."""
        # The tentative page is never in ``page_frame``: it comes from the free
        # list (emptied of its frame at eviction) or is a never-used page.
        return [self.page_frame.get(p, frame) for p in self.visible.patch_pages]
