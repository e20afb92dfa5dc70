"""Full-depth streaming driver: a stack of attention layers alternating frame
layers (attention over the frame's own tokens, nothing retained) and global
layers (attention over the dual-stream paged cache), for several independent
streams batched in every call.

Per layer: the library's fused projection + RoPE + append
(kv_project_append_frame: [Q | K | V] = bf16(x) W_l^T on the matrix cores,
rotated and written straight to q_rot and the pages), attention and (global
layers) deferred eviction, then the residual x <- x + O in fp32, fused with
the cast to bf16 that feeds the next layer's projection (residual_add_bf16).
Frame and global blocks are named on page "How LingBot-Map Achieves Real-Time
3D Reconstruction", section "AggregatorStream with FlashInfer Paged KV Cache";
the block internals need trained weights, so this driver keeps only the
projection, the attention and the residual.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import PagedKVCache, make_config, make_spec, residual_add


class FullDepthStream:
    def __init__(self, *, streams: int, layers: int, heads: int, grid_h: int, grid_w: int,
                 scale_frames: int, sliding_window: int, keyframe_interval: int, frames: int,
                 weights: List[torch.Tensor], head_dim: int = 64, special_tokens: int = 6,
                 pairs=(12, 10, 10), theta: float = 10000.0, ntk_factor: float = 1.0,
                 attn_splits: int = 0, frame_splits: int = 1, device="cuda"):
        if layers % 2:
            raise ValueError("layers alternate frame/global: an even count is expected")
        self.S, self.L, self.H, self.D = streams, layers, heads, head_dim
        self.N = special_tokens + grid_h * grid_w
        self.hidden = heads * head_dim
        self.interval = keyframe_interval
        self.device = torch.device(device)
        spec = make_spec(head_dim=head_dim, pairs=pairs, theta=theta, ntk_factor=ntk_factor,
                         max_frames=frames, max_h=grid_h, max_w=grid_w)
        common = dict(num_streams=streams, num_heads=heads, grid_h=grid_h, grid_w=grid_w,
                      dtype="bf16", head_dim=head_dim, special_tokens=special_tokens, rope=spec)
        # Frame layers keep nothing: every append is a skip-append on a cache
        # with no scale pages and no window, so one handle serves all of them.
        self.frame_cache = PagedKVCache(make_config(num_layers=1, scale_frames=0, sliding_window=0,
                                                    max_keyframes=0, attn_splits=frame_splits,
                                                    **common),
                                        device=self.device)
        n_kf = (frames + keyframe_interval - 1) // keyframe_interval
        self.global_cache = PagedKVCache(make_config(num_layers=layers // 2,
                                                     scale_frames=scale_frames,
                                                     sliding_window=sliding_window,
                                                     max_keyframes=n_kf, attn_splits=attn_splits,
                                                     **common), device=self.device)
        # W_l [hidden, 3*hidden] (x @ W_l) stored transposed, output channel
        # major as a linear layer keeps it: the fused kernel's layout.
        self.w = [wl.t().contiguous() for wl in weights]
        self.xb = torch.empty((streams, self.N, self.hidden), dtype=torch.bfloat16, device=self.device)
        shape = (streams, self.N, heads, head_dim)
        mk = lambda: torch.empty(shape, dtype=torch.bfloat16, device=self.device)
        self.q_rot, self.out = mk(), mk()

    def reset(self):
        self.global_cache.reset(-1)
        self.frame_cache.reset(-1)

    def frame(self, f: int, x: torch.Tensor, keep: Optional[List[torch.Tensor]] = None,
              events: Optional[list] = None, proj_events: Optional[list] = None) -> torch.Tensor:
        """Runs frame f (x: fp32 [S][N][hidden], updated in place) through all
        layers; appends each layer's attention output to `keep` if given, and
        (frame, layer, start event, end event) around each attention launch to
        `events` (around each fused projection + append to `proj_events`) if
        given."""
        commit = int(f % self.interval == 0)
        self.xb.copy_(x)   # later layers get their bf16 input from the residual kernel
        for layer in range(self.L):
            c, g, cm = (self.frame_cache, 0, 0) if layer % 2 == 0 else (self.global_cache, layer // 2, commit)
            if proj_events is not None:
                p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                p0.record()
            c.project_append(g, f, cm, self.xb, self.w[layer], self.q_rot)
            if proj_events is not None:
                p1.record()
                proj_events.append((f, layer, p0, p1))
            if events is not None:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
            c.attend(g, self.q_rot, self.out)
            if events is not None:
                e1.record()
                events.append((f, layer, e0, e1))
            if layer % 2 == 1:
                c.evict(g)
            if keep is not None:
                keep.append(self.out.clone())
            # x += O in fp32 and the next layer's bf16 input, in one pass
            residual_add(x, self.out, self.xb if layer + 1 < self.L else None)
        return x
