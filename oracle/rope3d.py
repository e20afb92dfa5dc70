"""3D (t/h/w) rotary position embedding in float64.

Follows page "How 3D RoPE Positional Encoding Works with the Paged KV Cache in
LingBot-Map" (sections "Multi-Axis Frequency Generation", "Complex-Valued
Tensor Application") and page "Video RoPE Positional Encoding: 3D Rotary
Embeddings for Long-Sequence Video in Ling-Bot-Map" (sections "The Three
Rotary Dimensions", "NTK-Aware Frequency Scaling", "Temporal Consistency in
KV-Cache Streaming"):

* each axis a in (t, h, w) owns d_a = 2 * pairs_a of the head's channels and a
  1D table of angles pos * omega_{a,j}; the three tables are concatenated
  along the pair axis in t, h, w order into one complex table of head_dim/2
  entries per token;
* the frequencies are the textbook rotary ones, omega_{a,j} =
  (theta * ntk)^(-2j / d_a), j < d_a/2 (the pages name theta and the NTK factor
  that multiplies it, not the formula: reading, textbook RoPE);
* the complex table multiplies the feature vector viewed as head_dim/2 complex
  numbers x_{2j} + i x_{2j+1} (adjacent pairs: the plainest reading of a
  complex table of head_dim/2 entries per token applied with real arithmetic);
* the temporal coordinate of a frame is its global frame index; the 6 special
  tokens that precede the patches sit at (t, 0, 0) (reading: only the temporal
  rotation, as for the camera head's 1x1 grid); patch token p sits at
  (t, p // gw, p % gw), 0-based.

Only Q and K are rotated; V is stored as is (page "How 3D RoPE ...", FAQ "Where
does the RoPE application occur relative to the KV cache write?").

Second channel layout, half-split (page "How to Handle Sequences Exceeding the
RoPE Training Range in LingBot-Map", sections "Understanding the 2D RoPE
Architecture" and "Spatial Position Encoding"): the 2D module gives the
vertical and the horizontal axis one half of the features each and rotates
each half on its own; reading: axis a owns a block of 2*pairs_a consecutive
channels (t, h, w in that order) and pair i of the block is (block[i],
block[i + pairs_a]), turned by the same angle pos * omega_{a,i} as above; the
module's base frequency is 100 (the example's `frequency=100.0`).
"""
from __future__ import annotations

import numpy as np


def axis_frequencies(pairs: int, theta: float = 10000.0, ntk_factor: float = 1.0) -> np.ndarray:
    """omega_j = (theta*ntk)^(-2j/d) for j < pairs, with d = 2*pairs real channels."""
    base = float(theta) * float(ntk_factor)
    d = 2 * pairs
    return np.array([base ** (-2.0 * j / d) for j in range(pairs)], dtype=np.float64)


def axis_table(length: int, pairs: int, theta: float = 10000.0, ntk_factor: float = 1.0) -> np.ndarray:
    """Complex 1D table exp(i * pos * omega_j) for pos < length: [length, pairs]."""
    ang = np.outer(np.arange(length, dtype=np.float64), axis_frequencies(pairs, theta, ntk_factor))
    return np.exp(1j * ang)


def token_positions(frame: int, grid_h: int, grid_w: int, n_special: int = 6):
    """(t, h, w) integer coordinates of the frame's tokens, specials first."""
    n = n_special + grid_h * grid_w
    t = np.full(n, frame, dtype=np.int64)
    h = np.zeros(n, dtype=np.int64)
    w = np.zeros(n, dtype=np.int64)
    p = np.arange(grid_h * grid_w)
    h[n_special:] = p // grid_w
    w[n_special:] = p % grid_w
    return t, h, w


def rotation_table(positions, pairs=(12, 10, 10), theta: float = 10000.0,
                   ntk_factor: float = 1.0) -> np.ndarray:
    """Concatenated complex table [N, sum(pairs)] for explicit (t, h, w) positions."""
    cols = []
    for pos, n_pairs in zip(positions, pairs):
        pos = np.asarray(pos, dtype=np.int64)
        tab = axis_table(int(pos.max()) + 1 if pos.size else 1, n_pairs, theta, ntk_factor)
        cols.append(tab[pos])
    return np.concatenate(cols, axis=1)


def apply_rotary(x: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Rotate x [N, H, D] (real) by the complex table [N, D/2]; returns float64."""
    x = np.asarray(x, dtype=np.float64)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * table[:, None, :]
    out = np.empty(x.shape, dtype=np.float64)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def apply_half_split(x: np.ndarray, table: np.ndarray, pairs=(12, 10, 10)) -> np.ndarray:
    """Rotate x [N, H, D] (real) by the complex table [N, D/2] with the
    half-split pairing: in the block of axis a, channel i and channel
    i + pairs_a form the complex number block[i] + i*block[i + pairs_a]."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    ch = 0   # first channel of the axis block
    col = 0  # first table column of the axis
    for n_pairs in pairs:
        re = x[..., ch:ch + n_pairs]
        im = x[..., ch + n_pairs:ch + 2 * n_pairs]
        z = (re + 1j * im) * table[:, None, col:col + n_pairs]
        out[..., ch:ch + n_pairs] = z.real
        out[..., ch + n_pairs:ch + 2 * n_pairs] = z.imag
        ch += 2 * n_pairs
        col += n_pairs
    return out


INTERLEAVED, HALF_SPLIT = 0, 1


def rotate_frame(x: np.ndarray, frame: int, grid_h: int, grid_w: int, n_special: int = 6,
                 pairs=(12, 10, 10), theta: float = 10000.0, ntk_factor: float = 1.0,
                 layout: int = INTERLEAVED) -> np.ndarray:
    """Rotate one frame's Q or K [N, H, D] at its (t, h, w) token positions."""
    tab = rotation_table(token_positions(frame, grid_h, grid_w, n_special), pairs, theta, ntk_factor)
    if layout == HALF_SPLIT:
        return apply_half_split(x, tab, pairs)
    return apply_rotary(x, tab)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of float64 input, returned as float64.

    Rounds directly from float64 (a single rounding)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    m, e = np.frexp(x[nz])            # x = m * 2^e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: scale the mantissa to [128, 256).
    out[nz] = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)   # np.round: ties to even
    return out
