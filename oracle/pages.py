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

Readings (the pages are silent): the free list is a stack (last in, first
out); a non-keyframe (skip-append) writes its K/V to the *tentative slot* --
the page the next stored frame would take and the special tokens right after
the stored ones -- which is visible to that frame's own attention and is not
committed; the frame being processed is listed after the window.  The free
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
        """Append one frame (``commit`` False: skip-append). Returns the status."""
        if self.status != OK:
            return self.status
        t = self.next_page()
        cap = self.special_capacity
        if t is None or (cap is not None and self.n_sp + self.n_special > cap):
            self.status = ENOSPACE
            self.visible = Visible([], 0, 0, 0)
            return self.status
        self.target, self.sp_offset = t, self.n_sp
        if commit:
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
            vis = self._special_visible(self.n_sp)
            vis.patch_pages = self.scale + list(self.window)
        else:
            vis = self._special_visible(self.n_sp + self.n_special)
            vis.patch_pages = self.scale + list(self.window) + [t]
        self.visible = vis
        return OK

    def evict(self) -> List[int]:
        """Deferred eviction; returns the pages moved to the free list."""
        out = []
        if self.status != OK:
            return out
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

    def visible_patch_frames(self, frame: int) -> List[int]:
        """Frames whose patches the current visible table shows (``frame`` for
        the tentative page)."""
        # The tentative page is never in ``page_frame``: it comes from the free
        # list (emptied of its frame at eviction) or is a never-used page.
        return [self.page_frame.get(p, frame) for p in self.visible.patch_pages]
