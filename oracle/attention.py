"""Dense softmax attention over an explicit key set, float64.

The pages hand the visible page table and the query to a paged prefill
attention routine (page "How 3D RoPE Positional Encoding Works with the Paged
KV Cache in LingBot-Map", section "Attention Computation with Cached RoPE").
What that routine computes is ordinary scaled dot-product attention of every
query token over every visible key token, with no mask inside the visible set
(reading: the frame's tokens see each other in both directions; causality
comes from the cache never holding later frames).  Scale 1/sqrt(head_dim)
(reading: the pages do not state it; it is the standard one).

Returns the output and the natural-log log-sum-exp of the scaled scores.
"""
from __future__ import annotations

import math

import numpy as np


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None,
              row_chunk: int = 256):
    """q [Nq, D], k [Nk, D], v [Nk, Dv] -> (out [Nq, Dv], lse [Nq]), float64.

    Max-subtracted softmax; rows are processed in chunks to bound memory."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    nq = q.shape[0]
    out = np.empty((nq, v.shape[1]), dtype=np.float64)
    lse = np.empty(nq, dtype=np.float64)
    if k.shape[0] == 0:
        out[:] = 0.0
        lse[:] = -np.inf
        return out, lse
    for r0 in range(0, nq, row_chunk):
        s = (q[r0:r0 + row_chunk] @ k.T) * scale
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        out[r0:r0 + row_chunk] = (p @ v) / l
        lse[r0:r0 + row_chunk] = (m + np.log(l))[:, 0]
    return out, lse


def attention_heads(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None):
    """Per-head attention: q [Nq, H, D], k/v [Nk, H, D] -> (out [Nq, H, D], lse [H, Nq])."""
    nq, h, d = q.shape
    out = np.empty((nq, h, v.shape[2]), dtype=np.float64)
    lse = np.empty((h, nq), dtype=np.float64)
    for hh in range(h):
        out[:, hh], lse[hh] = attention(q[:, hh], k[:, hh], v[:, hh], scale)
    return out, lse
