"""Seeded synthetic inputs and workload shapes, shared by the oracle and the GPU path.

This module holds no arithmetic of the method (no rotary embedding, no paging,
no attention).  It only describes the workloads (shapes, cache policy,
keyframe schedule) and draws their random inputs, so that the CPU oracle and
the HIP path can be fed the very same values while sharing no other code.

Every tensor is addressable on its own: the values for (workload, layer,
stream, frame, tensor) come from a PCG64 stream keyed by
``SeedSequence(base_seed, spawn_key=(workload_key, layer, stream, frame, tensor))``,
drawn as float32 N(0, 1) (or N(0, 0.02) for projection weights) and, for
bf16 workloads, rounded to the nearest bf16 (ties to even).  A value returned
here is therefore exactly representable in the workload's storage dtype.

Workload shapes follow the rotary-embedding / paged-KV pages: frames of
``gh x gw`` patch tokens preceded by 6 special tokens, 64-wide heads, a
3D rotary split of 12/10/10 complex pairs (t/h/w), theta 10000.
"""
from __future__ import annotations

import dataclasses
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_X0, TENSOR_W = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and cache policy of one synthetic streaming workload."""

    name: str
    dtype: str              # "f32" or "bf16": storage dtype of q/k/v, cache and outputs
    frames: int             # frames in the stream
    grid_h: int             # patch rows per frame
    grid_w: int             # patch columns per frame
    heads: int
    head_dim: int = 64
    n_special: int = 6      # special tokens per frame, placed before the patches
    streams: int = 1        # independent streams batched in one call
    cached_layers: int = 1  # layers that own a paged cache
    scale_frames: int = 0
    sliding_window: int = 0
    keyframe_interval: int = 1
    patch_page_size: Optional[int] = None   # default: one frame of patches per page
    special_page_size: int = 6
    pairs: tuple = (12, 10, 10)             # complex pairs on the t, h, w axes
    theta: float = 10000.0
    ntk_factor: float = 1.0
    rope_layout: int = 0                    # 0 interleaved pairs, 1 half-split axis blocks
    grids: tuple = ()                       # per-frame (gh, gw), cycled; () = the grid above
    max_frames: Optional[int] = None        # rotary t-table length (default: frames)
    # Full-depth chain (frame layers interleaved with cached layers).
    chain_layers: int = 0   # 0: single cached layer fed by seeded q/k/v
    hidden: int = 0         # model width of the chain (heads * head_dim)
    base_seed: int = 0

    @property
    def patches(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def tokens(self) -> int:
        return self.n_special + self.patches

    @property
    def page_size(self) -> int:
        return self.patch_page_size if self.patch_page_size else self.patches

    @property
    def t_rows(self) -> int:
        return self.max_frames if self.max_frames else self.frames

    @property
    def key(self) -> int:
        return zlib.crc32(self.name.encode()) & 0x7FFFFFFF

    def grid_of(self, f: int) -> tuple:
        """Patch grid of frame f (a frame may have fewer patches than the page holds)."""
        return self.grids[f % len(self.grids)] if self.grids else (self.grid_h, self.grid_w)

    def frame_tokens(self, f: int) -> int:
        gh, gw = self.grid_of(f)
        return self.n_special + gh * gw

    def is_keyframe(self, f: int) -> bool:
        return f % self.keyframe_interval == 0

    def n_keyframes(self, upto: Optional[int] = None) -> int:
        """Keyframes among frames [0, upto)."""
        n = self.frames if upto is None else upto
        return (n + self.keyframe_interval - 1) // self.keyframe_interval

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: shapes, policies and seeds of the synthetic streams.
WORKLOADS = {
    0: Workload("tiny_f32_4x4", "f32", frames=16, grid_h=4, grid_w=4, heads=2,
                scale_frames=1, sliding_window=4, keyframe_interval=1,
                patch_page_size=16, special_page_size=6),
    1: Workload("single_layer_37x37", "bf16", frames=64, grid_h=37, grid_w=37, heads=16,
                scale_frames=8, sliding_window=16, keyframe_interval=1),
    2: Workload("long_stream_37x37", "bf16", frames=1024, grid_h=37, grid_w=37, heads=16,
                scale_frames=8, sliding_window=64, keyframe_interval=5),
    3: Workload("large_grid_64x64", "bf16", frames=32, grid_h=64, grid_w=64, heads=16,
                scale_frames=4, sliding_window=16, keyframe_interval=1),
    4: Workload("full_depth_4x24_37x37", "bf16", frames=256, grid_h=37, grid_w=37, heads=16,
                streams=4, cached_layers=12, scale_frames=8, sliding_window=32,
                keyframe_interval=2, chain_layers=24, hidden=1024),
}


def small_variants() -> dict:
    """Reduced workloads the oracle finishes in seconds; they keep the
    structure (several key tiles, ragged page tails, eviction and recycling,
    skip-append frames, partial special pages)."""
    return {
        "small_bf16": Workload("small_bf16_9x11", "bf16", frames=12, grid_h=9, grid_w=11, heads=4,
                               scale_frames=2, sliding_window=3, keyframe_interval=1),
        "small_skip": Workload("small_skip_7x13", "bf16", frames=20, grid_h=7, grid_w=13, heads=3,
                               scale_frames=2, sliding_window=3, keyframe_interval=3),
        "small_partial_sp": Workload("small_partial_sp_5x5", "bf16", frames=10, grid_h=5, grid_w=5,
                                     heads=2, scale_frames=1, sliding_window=4,
                                     keyframe_interval=2, special_page_size=16),
        "small_f32": Workload("small_f32_6x10", "f32", frames=9, grid_h=6, grid_w=10, heads=3,
                              scale_frames=1, sliding_window=2, keyframe_interval=2),
        "small_tall": Workload("small_tall_3x45", "bf16", frames=8, grid_h=3, grid_w=45, heads=2,
                               scale_frames=1, sliding_window=2, keyframe_interval=1),
        "small_chain": Workload("small_chain_6x6", "bf16", frames=7, grid_h=6, grid_w=6, heads=4,
                                streams=2, cached_layers=2, scale_frames=1, sliding_window=2,
                                keyframe_interval=2, chain_layers=4, hidden=256),
        # the full-depth stack's structure (4 streams, 24 alternating layers,
        # keyframe every 2nd frame) at a size the oracle chain runs in
        # seconds, long enough for the first eviction (frame 10) and the
        # first recycled page (frame 12)
        "small_depth": Workload("small_depth_6x6", "bf16", frames=16, grid_h=6, grid_w=6, heads=4,
                                streams=4, cached_layers=12, scale_frames=2, sliding_window=3,
                                keyframe_interval=2, chain_layers=24, hidden=256),
        # the 2D module's arrangement: y and x halves, base frequency 100
        "small_rope2d": Workload("small_rope2d_10x7", "bf16", frames=8, grid_h=10, grid_w=7, heads=2,
                                 scale_frames=1, sliding_window=3, keyframe_interval=1,
                                 pairs=(0, 16, 16), theta=100.0, rope_layout=1),
        "small_rope2d_f32": Workload("small_rope2d_f32_5x6", "f32", frames=6, grid_h=5, grid_w=6,
                                     heads=2, scale_frames=1, sliding_window=2, keyframe_interval=2,
                                     pairs=(16, 8, 8), theta=100.0, rope_layout=1),
        # NTK-stretched base
        "small_ntk": Workload("small_ntk_8x8", "bf16", frames=6, grid_h=8, grid_w=8, heads=2,
                              scale_frames=1, sliding_window=2, keyframe_interval=1, ntk_factor=4.0),
        # fused projection + append: 13x17 (the specials share the last row
        # tile with the patches), hidden = H*D; 5x25 half-split (the specials
        # straddle two row tiles), hidden 192 != H*D
        "small_proj": Workload("small_proj_13x17", "bf16", frames=6, grid_h=13, grid_w=17, heads=4,
                               streams=2, scale_frames=1, sliding_window=2, keyframe_interval=2,
                               hidden=256),
        "small_proj_half": Workload("small_proj_half_5x25", "bf16", frames=5, grid_h=5, grid_w=25,
                                    heads=2, scale_frames=1, sliding_window=2, keyframe_interval=1,
                                    pairs=(0, 16, 16), theta=100.0, rope_layout=1, hidden=192),
        # frames of their own patch grids, up to 9x11 (partial patch pages)
        "small_vargrid": Workload("small_vargrid_9x11", "bf16", frames=10, grid_h=9, grid_w=11,
                                  heads=3, scale_frames=2, sliding_window=3, keyframe_interval=1,
                                  grids=((9, 11), (7, 11), (5, 6), (1, 1), (9, 7))),
        # a camera-head style grid: one patch per frame
        "small_cam": Workload("small_cam_1x1", "bf16", frames=12, grid_h=1, grid_w=1, heads=2,
                              scale_frames=2, sliding_window=3, keyframe_interval=1),
    }


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    This is the storage format of bf16 inputs, not a step of the method.
    Inputs here are finite, so NaN handling is not needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    r = (b + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of bf16-exact float32 values."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-exact")
    return (b >> np.uint32(16)).astype(np.uint16)


def _rng(wl: Workload, layer: int, stream: int, frame: int, tensor: int) -> np.random.Generator:
    ss = np.random.SeedSequence(wl.base_seed, spawn_key=(wl.key, layer, stream, frame, tensor))
    return np.random.Generator(np.random.PCG64(ss))


def _store(wl: Workload, x: np.ndarray) -> np.ndarray:
    return round_to_bf16(x) if wl.dtype == "bf16" else x


def qkv(wl: Workload, layer: int, stream: int, frame: int, tensor: int) -> np.ndarray:
    """Q (tensor 0), K (1) or V (2) of one frame: float32 [N, H, D], N(0,1)."""
    x = _rng(wl, layer, stream, frame, tensor).standard_normal(
        (wl.tokens, wl.heads, wl.head_dim), dtype=np.float32)
    return _store(wl, x)


def qkv_layer(wl: Workload, layer: int, stream: int, frame: int, tensor: int) -> np.ndarray:
    """Layer-distinct inputs without drawing new numbers: the layer-0 draw of
    the (stream, frame, tensor) rolled by `layer` positions along the head axis
    (used where many layers would make fresh draws too slow)."""
    return np.roll(qkv(wl, 0, stream, frame, tensor), layer, axis=1)


def frame_qkv(wl: Workload, layer: int, frame: int, streams: Optional[Sequence[int]] = None):
    """(q, k, v) for one frame and all streams: each float32 [S, N, H, D]."""
    ss = range(wl.streams) if streams is None else streams
    return tuple(np.stack([qkv(wl, layer, s, frame, t) for s in ss]) for t in (0, 1, 2))


def embeddings(wl: Workload, stream: int, frame: int) -> np.ndarray:
    """Chain input x_0 of one frame: float32 [N, hidden], N(0,1) (kept in fp32)."""
    return _rng(wl, 0, stream, frame, TENSOR_X0).standard_normal(
        (wl.tokens, wl.hidden), dtype=np.float32)


def projection(wl: Workload, layer: int, n_out: Optional[int] = None) -> np.ndarray:
    """QKV projection of one chain layer: float32 [hidden, n_out] (default
    3*hidden), N(0, 0.02), rounded to the storage dtype."""
    w = _rng(wl, layer, 0, 0, TENSOR_W).standard_normal(
        (wl.hidden, n_out or 3 * wl.hidden), dtype=np.float32) * np.float32(0.02)
    return _store(wl, w)


def stream_qkv(wl: Workload, layer: int = 0, frames: Optional[Sequence[int]] = None,
               threads: int = 8):
    """q, k, v for many frames at once: float32 [F, S, N, H, D] each (threaded)."""
    fr = list(range(wl.frames)) if frames is None else list(frames)

    def one(f):
        return frame_qkv(wl, layer, f)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        parts = list(ex.map(one, fr))
    return tuple(np.stack([p[t] for p in parts]) for t in range(3))
