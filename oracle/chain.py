"""Full-depth chain of one stream: QKV projection, 3D rotary embedding, then
alternately frame attention (the frame's own tokens only) and global attention
over the paged cache, with a residual connection.

The pages name frame blocks and global blocks (page "How LingBot-Map Achieves
Real-Time 3D Reconstruction", section "AggregatorStream with FlashInfer Paged
KV Cache") and place the rotary embedding right after the Q/K projection and
before the cache write (page "How 3D RoPE Positional Encoding Works with the
Paged KV Cache in LingBot-Map", FAQ on where RoPE is applied).  The block
internals need trained weights and are not on the pages; the chain here is the
plainest one those statements support (reading):

* layer l has its own projection W_l [hidden, 3*hidden], no bias:
  [Q | K | V] = bf16(x_l) @ W_l, rounded to the storage dtype; head h takes
  columns h*D .. h*D+D-1 of each third;
* even layers are frame layers, odd layers are global (cached) layers;
* x_{l+1} = x_l + concat_h(O_h), where O is the stored attention output.
"""
from __future__ import annotations

from typing import Callable, Dict, List

import numpy as np

from . import attention as att
from . import retained
from . import rope3d


def project_qkv(x, w, heads: int, head_dim: int, round_store: bool = True):
    """The chain's projection of one frame: [Q | K | V] = store(store(x) @ w)
    with x [N, C] and w [C, 3*H*D] (no bias), split into three [N, H, D]
    arrays (head h at columns h*D .. h*D+D-1 of each third).  store() rounds
    to bf16 when round_store is set (the stored projection output)."""
    st = rope3d.round_bf16 if round_store else (lambda a: np.asarray(a, dtype=np.float64))
    x = st(np.asarray(x, dtype=np.float64))
    qkv = st(x @ np.asarray(w, dtype=np.float64))
    n, hd = x.shape[0], heads * head_dim
    return tuple(qkv[:, i * hd:(i + 1) * hd].reshape(n, heads, head_dim) for i in range(3))


class OracleChain:
    def __init__(self, wl, x0: Callable[[int], np.ndarray], weight: Callable[[int], np.ndarray]):
        self.wl = wl
        self.x0 = x0
        self.weight = weight
        self.round = wl.dtype == "bf16"
        self._w: Dict[int, np.ndarray] = {}
        # cached layer index -> frame -> (K rotated, V) [N, H, D]
        self.cache: Dict[int, Dict[int, tuple]] = {}

    def _store(self, x):
        return rope3d.round_bf16(x) if self.round else np.asarray(x, dtype=np.float64)

    def _weight(self, layer):
        if layer not in self._w:
            self._w[layer] = np.asarray(self.weight(layer), dtype=np.float64)
        return self._w[layer]

    def _rotate(self, x, frame):
        wl = self.wl
        return rope3d.rotate_frame(x, frame, wl.grid_h, wl.grid_w, wl.n_special, wl.pairs,
                                   wl.theta, wl.ntk_factor, layout=wl.rope_layout)

    def frame(self, f: int):
        """Run frame f through every layer. Returns (list of O_l [N, H, D], x_L [N, hidden])."""
        wl = self.wl
        n, h, d = wl.tokens, wl.heads, wl.head_dim
        hid = h * d
        x = np.asarray(self.x0(f), dtype=np.float64)
        outs: List[np.ndarray] = []
        for layer in range(wl.chain_layers):
            q, k, v = project_qkv(x, self._weight(layer), h, d, self.round)
            q = self._store(self._rotate(q, f))
            k = self._store(self._rotate(k, f))
            if layer % 2 == 0:
                kk, vv = k, v
            else:
                c = layer // 2
                store = self.cache.setdefault(c, {})
                pf, sf = retained.visible_for_schedule(f, wl.keyframe_interval, wl.scale_frames,
                                                       wl.sliding_window)
                store[f] = (k, v)
                ns = wl.n_special
                kk = np.concatenate([store[g][0][ns:] for g in pf] + [store[g][0][:ns] for g in sf])
                vv = np.concatenate([store[g][1][ns:] for g in pf] + [store[g][1][:ns] for g in sf])
                if not wl.is_keyframe(f):
                    del store[f]
            o, _ = att.attention_heads(q, kk, vv)
            o = self._store(o)
            outs.append(o)
            x = x + o.reshape(n, hid)
        return outs, x
