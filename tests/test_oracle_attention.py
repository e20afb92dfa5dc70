"""Pins of the oracle's attention and of the frame-by-frame assembly of the
retained keys: explicit loops, PyTorch's scaled_dot_product_attention (a
library routine) on the CPU, scipy's logsumexp, closed forms (Q = 0 gives the
mean of the visible V; one key gives its V), and the visibility probe whose
expected value comes from the page simulator, not from the enumeration."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention as att
from oracle import pages, rope3d
from oracle.stream import OracleStream
from rpkv_inputs import WORKLOADS, qkv, small_variants


def loop_attention(q, k, v):
    """Row by row, key by key, with math.exp and no max subtraction."""
    d = q.shape[1]
    out = np.zeros((q.shape[0], v.shape[1]))
    lse = np.zeros(q.shape[0])
    for i in range(q.shape[0]):
        w = [math.exp(sum(q[i, c] * k[j, c] for c in range(d)) / math.sqrt(d))
             for j in range(k.shape[0])]
        tot = sum(w)
        for j in range(k.shape[0]):
            out[i] += w[j] / tot * v[j]
        lse[i] = math.log(tot)
    return out, lse


def test_matches_explicit_loops():
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((5, 8)), rng.standard_normal((7, 8)), rng.standard_normal((7, 3))
    o, l = att.attention(q, k, v, row_chunk=2)
    o2, l2 = loop_attention(q, k, v)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(l, l2, atol=1e-13)


def test_matches_torch_sdpa_and_logsumexp():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((33, 64)) * 3, rng.standard_normal((517, 64)) * 3,
               rng.standard_normal((517, 64)))
    o, l = att.attention(q, k, v, row_chunk=16)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)
    np.testing.assert_allclose(l, logsumexp(q @ k.T / 8.0, axis=1), atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(2)
    k, v = rng.standard_normal((9, 64)), rng.standard_normal((9, 5))
    o, l = att.attention(np.zeros((3, 64)), k, v)
    np.testing.assert_allclose(o, np.tile(v.mean(0), (3, 1)), atol=1e-15)
    np.testing.assert_allclose(l, math.log(9), atol=1e-15)
    o, l = att.attention(rng.standard_normal((2, 64)), k[:1], v[:1])
    np.testing.assert_allclose(o, np.tile(v[0], (2, 1)), atol=1e-15)
    o, l = att.attention(np.zeros((2, 64)), k[:0], v[:0])
    assert np.all(o == 0) and np.all(np.isneginf(l))


def _probe_source(wl):
    """Q = 0; V of every token = one-hot of (frame mod D) in head 0 for patch
    tokens and in head 1 for special tokens; K random."""
    def src(frame, t):
        n, h, d = wl.tokens, wl.heads, wl.head_dim
        if t == 0:
            return np.zeros((n, h, d))
        if t == 1:
            return qkv(wl, 0, 0, frame, 1)
        v = np.zeros((n, h, d))
        v[wl.n_special:, 0, frame % d] = 1.0
        v[:wl.n_special, 1, frame % d] = 1.0
        return v
    return src


@pytest.mark.parametrize("name", ["small_skip", "small_bf16", "small_partial_sp"])
def test_visibility_probe_against_page_simulator(name):
    """With Q = 0 attention is the plain mean of the visible V, so the output
    is the histogram of visible frames; the expected histogram is read from the
    page simulator's page -> frame map, an independent description."""
    wl = small_variants()[name]
    ost = OracleStream(wl, _probe_source(wl))
    sim = pages.PageSim(wl.scale_frames, wl.sliding_window, wl.special_page_size, wl.n_special)
    for f in range(wl.frames):
        sim.append(f, wl.is_keyframe(f))
        pf = sim.visible_patch_frames(f)
        spf = sim.special_frames + [f]
        total = len(pf) * wl.patches + len(spf) * wl.n_special
        want0 = np.zeros(wl.head_dim)
        want1 = np.zeros(wl.head_dim)
        for g in pf:
            want0[g % wl.head_dim] += wl.patches / total
        for g in spf:
            want1[g % wl.head_dim] += wl.n_special / total
        o, lse = ost.attend(f)
        np.testing.assert_allclose(o[:, 0], np.tile(want0, (wl.tokens, 1)), atol=1e-14)
        np.testing.assert_allclose(o[:, 1], np.tile(want1, (wl.tokens, 1)), atol=1e-14)
        np.testing.assert_allclose(lse, math.log(total), atol=1e-12)
        sim.evict()


def test_frame_only_cache_is_dense_attention_within_frame():
    """scale_frames = window = 0 and nothing stored: plain attention of the
    frame over its own tokens (library SDPA on the rotated tensors)."""
    wl = small_variants()["small_bf16"].replace(scale_frames=0, sliding_window=0)
    ost = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t), keyframe_interval=0)
    for f in (0, 3):
        o, lse = ost.attend(f)
        q = rope3d.round_bf16(ost.rotate(qkv(wl, 0, 0, f, 0), f))
        k = rope3d.round_bf16(ost.rotate(qkv(wl, 0, 0, f, 1), f))
        v = qkv(wl, 0, 0, f, 2).astype(np.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).transpose(0, 1), torch.from_numpy(k).transpose(0, 1),
            torch.from_numpy(v).transpose(0, 1)).transpose(0, 1).numpy()
        np.testing.assert_allclose(o, ref, atol=1e-12)


def test_unbounded_window_is_block_causal_attention():
    """A window larger than the stream keeps everything: each frame attends to
    all tokens of all earlier keyframes and its own (block-causal mask built
    by hand over the concatenated stream, library SDPA)."""
    wl = small_variants()["small_skip"].replace(sliding_window=100, scale_frames=0)
    ost = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t))
    qs, ks, vs, owner = [], [], [], []
    for f in range(wl.frames):
        qs.append(rope3d.round_bf16(ost.rotate(qkv(wl, 0, 0, f, 0), f)))
        ks.append(rope3d.round_bf16(ost.rotate(qkv(wl, 0, 0, f, 1), f)))
        vs.append(qkv(wl, 0, 0, f, 2).astype(np.float64))
        owner += [f] * wl.tokens
    q, k, v = (torch.from_numpy(np.concatenate(a)).transpose(0, 1) for a in (qs, ks, vs))
    owner = np.array(owner)
    keyf = np.array([wl.is_keyframe(g) for g in owner])
    allow = (owner[None, :] == owner[:, None]) | ((owner[None, :] < owner[:, None]) & keyf[None, :])
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.from_numpy(allow)).transpose(0, 1).numpy()
    for f in (0, 1, 4, 7, wl.frames - 1):
        o, _ = ost.attend(f)
        np.testing.assert_allclose(o, ref[owner == f], atol=1e-12)


def test_sampled_rows_and_heads_match_full():
    wl = small_variants()["small_tall"]
    ost = OracleStream(wl, lambda f, t: qkv(wl, 0, 0, f, t))
    o, l = ost.attend(5)
    o2, l2 = ost.attend(5, rows=[0, 5, 6, 100, wl.tokens - 1], heads=[1])
    np.testing.assert_allclose(o2[:, 0], o[[0, 5, 6, 100, wl.tokens - 1], 1], atol=1e-14)
    np.testing.assert_allclose(l2[0], l[1, [0, 5, 6, 100, wl.tokens - 1]], atol=1e-13)
