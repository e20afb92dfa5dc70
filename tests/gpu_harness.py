"""Drives the HIP path over a workload for the GPU tests (no oracle code here)."""
from __future__ import annotations

import numpy as np
import torch

import rope_paged_kv_amd as rp
from rpkv_inputs import Workload, frame_qkv


def torch_dtype(wl: Workload):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def make_cache(wl: Workload, layers: int = 1, splits: int = 0, **over) -> rp.PagedKVCache:
    spec = rp.make_spec(pairs=wl.pairs, theta=wl.theta, ntk_factor=wl.ntk_factor,
                        max_frames=over.pop("max_frames", wl.t_rows),
                        max_h=wl.grid_h, max_w=wl.grid_w, layout=wl.rope_layout)
    kw = dict(num_layers=layers, num_streams=wl.streams, num_heads=wl.heads, grid_h=wl.grid_h,
              grid_w=wl.grid_w, dtype=wl.dtype, head_dim=wl.head_dim,
              special_tokens=wl.n_special, patch_page_size=wl.page_size,
              special_page_size=wl.special_page_size, scale_frames=wl.scale_frames,
              sliding_window=wl.sliding_window, max_keyframes=wl.n_keyframes(),
              attn_splits=splits, rope=spec)
    kw.update(over)
    return rp.PagedKVCache(rp.make_config(**kw))


def to_dev(x: np.ndarray, dt) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(dt)


class Runner:
    """Runs frames of one layer through append -> attend -> evict."""

    def __init__(self, wl: Workload, cache: rp.PagedKVCache, layer: int = 0):
        self.wl, self.cache, self.layer = wl, cache, layer
        self.dt = torch_dtype(wl)
        shape = (wl.streams, wl.tokens, wl.heads, wl.head_dim)
        self.q_rot = torch.empty(shape, dtype=self.dt, device="cuda")
        self.out = torch.empty(shape, dtype=self.dt, device="cuda")
        self.lse = torch.empty((wl.streams, wl.heads, wl.tokens), dtype=torch.float32, device="cuda")

    def frame(self, f: int, q, k, v, commit: bool, evict: bool = True):
        c = self.cache
        grid = self.wl.grid_of(f) if self.wl.grids else None
        c.append(self.layer, f, int(commit), q, k, v, self.q_rot, grid=grid)
        c.attend(self.layer, self.q_rot, self.out, self.lse)
        if evict:
            c.evict(self.layer)

    def inputs(self, f: int, layer_key: int = 0):
        q, k, v = frame_qkv(self.wl, layer_key, f)
        return to_dev(q, self.dt), to_dev(k, self.dt), to_dev(v, self.dt)
