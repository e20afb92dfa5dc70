"""Frame-by-frame oracle of one (layer, stream) cache over a workload.

For frame f it rotates the frame's Q and K (``rope3d``), enumerates the
retained token set (``retained``, not the page simulator), assembles those
tokens' K and V from their own frames, and runs dense attention
(``attention``).  K/V of past frames are recomputed from the seeded inputs of
those frames, exactly as they were when the frames were processed.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import numpy as np

from . import attention as att
from . import retained
from . import rope3d

Source = Callable[[int, int], np.ndarray]   # (frame, tensor 0/1/2) -> [N, H, D]


class OracleStream:
    def __init__(self, wl, source: Source, keyframe_interval: Optional[int] = None,
                 storage_round: Optional[bool] = None, window_start: int = 0):
        """window_start: first frame of the cache's life.  Windowed inference
        starts every window on a fresh cache (page "KV Caching Benefits in
        Ling Bot-Map", section "Cross-Window Alignment for Long Videos"), so
        only frames from there on can be retained; frames keep their global
        index as the temporal position."""
        self.wl = wl
        self.window_start = window_start
        self.source = source
        self.interval = wl.keyframe_interval if keyframe_interval is None else keyframe_interval
        self.round = (wl.dtype == "bf16") if storage_round is None else storage_round
        self._kv = {}

    def _store(self, x: np.ndarray) -> np.ndarray:
        return rope3d.round_bf16(x) if self.round else x

    def rotate(self, x: np.ndarray, frame: int) -> np.ndarray:
        """Rotated tokens of the frame: its specials and its own patch grid
        (rows of x past them are not part of the frame)."""
        wl = self.wl
        gh, gw = wl.grid_of(frame)
        x = np.asarray(x)[:wl.n_special + gh * gw]
        return rope3d.rotate_frame(x, frame, gh, gw, wl.n_special, wl.pairs,
                                   wl.theta, wl.ntk_factor, layout=wl.rope_layout)

    def q_rot(self, frame: int) -> np.ndarray:
        """Rotated Q of the frame as stored for attention [N, H, D] (float64)."""
        return self._store(self.rotate(self.source(frame, 0), frame))

    def kv(self, frame: int):
        """(K rotated, V) of the frame as the cache holds them [N, H, D] (float64)."""
        if frame not in self._kv:
            k = self._store(self.rotate(self.source(frame, 1), frame))
            v = np.asarray(self.source(frame, 2), dtype=np.float64)[:k.shape[0]]
            self._kv[frame] = (k, v)
        return self._kv[frame]

    def stored_before(self, frame: int):
        return [k for k in retained.keyframes_before(frame, self.interval) if k >= self.window_start]

    def visible(self, frame: int):
        wl = self.wl
        return retained.visible_frames(frame, self.stored_before(frame), wl.scale_frames,
                                       wl.sliding_window)

    def keys(self, frame: int):
        """K, V [T, H, D] of the retained set of ``frame`` (patch tokens of the
        visible patch frames, then special tokens of the visible special frames)."""
        wl = self.wl
        pf, sf = self.visible(frame)
        keep = set(pf) | set(sf)
        for f in list(self._kv):
            if f not in keep:
                del self._kv[f]
        ns = wl.n_special
        ks = [self.kv(f)[0][ns:] for f in pf] + [self.kv(f)[0][:ns] for f in sf]
        vs = [self.kv(f)[1][ns:] for f in pf] + [self.kv(f)[1][:ns] for f in sf]
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)

    def attend(self, frame: int, rows: Optional[Sequence[int]] = None,
               heads: Optional[Sequence[int]] = None):
        """Attention output [R, H', D] and LSE [H', R] of the frame's query rows."""
        q = self.q_rot(frame)
        k, v = self.keys(frame)
        if rows is not None:
            q = q[np.asarray(rows)]
        if heads is not None:
            hs = np.asarray(heads)
            q, k, v = q[:, hs], k[:, hs], v[:, hs]
        return att.attention_heads(q, k, v)
