"""Python binding of librpkv (include/rpkv.h): the per-frame hot path of a
streaming 3D-reconstruction transformer on MI355X -- 3D rotary embedding,
dual-stream paged KV cache with device-resident bookkeeping, and paged
attention on the matrix cores.

The functions below carry the C names and only marshal arguments: every step
runs in the HIP kernels of ``csrc/``.  PyTorch is used for device memory and
streams (``PagedKVCache`` allocates with torch and passes raw pointers).
Importing this package loads the library and raises if it is missing.

One layer over a stream of 37x37 frames (6 special tokens + 1369 patches,
16 heads of 64, bf16)::

    spec = make_spec(max_frames=1024, max_h=37, max_w=37)
    cfg = make_config(num_layers=1, num_streams=1, num_heads=16, grid_h=37, grid_w=37,
                      scale_frames=8, sliding_window=16, max_keyframes=256, rope=spec)
    cache = PagedKVCache(cfg)
    for f, (q, k, v) in enumerate(frames):        # each [1, 1375, 16, 64] bf16 on the GPU
        cache.append(0, f, is_keyframe(f), q, k, v, q_rot)   # RoPE + page write
        cache.attend(0, q_rot, out, lse)                      # paged attention
        cache.evict(0)                                        # deferred commit / eviction

``cache.project_append`` replaces ``append`` when the frame's hidden states
and the layer's QKV weight are at hand (the projection runs in the same
kernel).
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

# torch first: the library must bind to the HIP runtime torch carries.  Loaded
# before torch, it would pull in the system runtime, and torch's device
# pointers and streams would belong to another runtime instance.
import torch  # noqa: F401

from . import _abi
from ._abi import (RPKV_BF16, RPKV_EHIP, RPKV_EINVAL, RPKV_ENOSPACE, RPKV_ESTATE, RPKV_ETOOBIG,
                   RPKV_F32, RPKV_OK, RPKV_STATIC_SCRATCH_BYTES, KvConfig, Rope3dSpec)

_lib = _abi.load()


class RpkvError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_lib.rpkv_strerror(code).decode()} ({code})")
        self.code = code


def _check(rc: int, what: str) -> None:
    if rc != RPKV_OK:
        raise RpkvError(rc, what)


def _vp(x) -> Optional[int]:
    if x is None:
        return None
    return x if isinstance(x, int) else x.data_ptr()


# ---- C functions ---------------------------------------------------------

def rope3d_tables_bytes(spec: Rope3dSpec) -> int:
    return _lib.rope3d_tables_bytes(C.byref(spec))


def rope3d_build_tables(spec: Rope3dSpec, d_tables, nbytes: int, stream: int) -> None:
    _check(_lib.rope3d_build_tables(C.byref(spec), _vp(d_tables), nbytes, stream),
           "rope3d_build_tables")


def kv_required_bytes(cfg: KvConfig) -> int:
    return _lib.kv_required_bytes(C.byref(cfg))


def kv_create(cfg: KvConfig, d_mem, nbytes: int, stream: int) -> C.c_void_p:
    h = C.c_void_p()
    _check(_lib.kv_create(C.byref(cfg), _vp(d_mem), nbytes, stream, C.byref(h)), "kv_create")
    return h


def kv_destroy(h) -> None:
    _check(_lib.kv_destroy(h), "kv_destroy")


def kv_reset(h, layer: int, stream: int) -> None:
    _check(_lib.kv_reset(h, layer, stream), "kv_reset")


def kv_append_frame(h, layer: int, frame_idx: int, commit: int, q, k, v, q_rot, d_tables,
                    stream: int) -> None:
    _check(_lib.kv_append_frame(h, layer, frame_idx, int(commit), _vp(q), _vp(k), _vp(v),
                                _vp(q_rot), _vp(d_tables), stream), "kv_append_frame")


def kv_append_frame_grid(h, layer: int, frame_idx: int, commit: int, grid_h: int, grid_w: int,
                         q, k, v, q_rot, d_tables, stream: int) -> None:
    _check(_lib.kv_append_frame_grid(h, layer, frame_idx, int(commit), grid_h, grid_w, _vp(q),
                                     _vp(k), _vp(v), _vp(q_rot), _vp(d_tables), stream),
           "kv_append_frame_grid")


def kv_project_append_frame(h, layer: int, frame_idx: int, commit: int, x, hidden: int, w, q_rot,
                            d_tables, stream: int) -> None:
    _check(_lib.kv_project_append_frame(h, layer, frame_idx, int(commit), _vp(x), hidden, _vp(w),
                                        _vp(q_rot), _vp(d_tables), stream),
           "kv_project_append_frame")


def kv_project_append_frame_grid(h, layer: int, frame_idx: int, commit: int, grid_h: int,
                                 grid_w: int, x, hidden: int, w, q_rot, d_tables, stream: int) -> None:
    _check(_lib.kv_project_append_frame_grid(h, layer, frame_idx, int(commit), grid_h, grid_w,
                                             _vp(x), hidden, _vp(w), _vp(q_rot), _vp(d_tables),
                                             stream),
           "kv_project_append_frame_grid")


def attend_frame(h, layer: int, q_rot, out, lse, stream: int) -> None:
    _check(_lib.attend_frame(h, layer, _vp(q_rot), _vp(out), _vp(lse), stream), "attend_frame")


def attend_frame_noalloc(h, layer: int, q_rot, out, lse, stream: int) -> None:
    _check(_lib.attend_frame_noalloc(h, layer, _vp(q_rot), _vp(out), _vp(lse), stream),
           "attend_frame_noalloc")


def residual_add_bf16(x, o, xb, n: int, stream: int) -> None:
    _check(_lib.residual_add_bf16(_vp(x), _vp(o), _vp(xb), n, stream), "residual_add_bf16")


def residual_add(x, o, xb=None) -> None:
    """x += o (fp32 += bf16) and, if given, xb = bf16(x), on torch's current
    stream: x fp32, o and xb bf16, contiguous, on one device, o and xb with
    x's number of elements."""
    import torch
    if x.dtype != torch.float32 or o.dtype != torch.bfloat16 or not x.is_contiguous() \
            or not o.is_contiguous() or o.numel() != x.numel() or o.device != x.device:
        raise ValueError("residual_add: x fp32 and o bf16, contiguous, same size and device")
    if xb is not None and (xb.dtype != torch.bfloat16 or not xb.is_contiguous()
                           or xb.numel() != x.numel() or xb.device != x.device):
        raise ValueError("residual_add: xb bf16, contiguous, x's size and device")
    residual_add_bf16(x, o, xb, x.numel(), torch.cuda.current_stream(x.device).cuda_stream)


def kv_evict_deferred(h, layer: int, stream: int) -> None:
    _check(_lib.kv_evict_deferred(h, layer, stream), "kv_evict_deferred")


def kv_rollback(h, layer: int, stream: int) -> None:
    _check(_lib.kv_rollback(h, layer, stream), "kv_rollback")


def kv_read_state(h, layer: int, stream_idx: int, stream: int) -> dict:
    st = _abi.KvStateHost()
    _check(_lib.kv_read_state(h, layer, stream_idx, C.byref(st), stream), "kv_read_state")
    out = {name: getattr(st, name) for name, _ in _abi.KvStateHost._fields_[:13]}
    out["free_list"] = list(st.free_list[:st.n_free])
    out["scale_pages"] = list(st.scale_pages[:st.n_scale])
    out["window_pages"] = list(st.window_pages[:st.n_window])
    out["visible_pages"] = list(st.visible_pages[:st.n_visible_pages])
    out["query_tokens"] = st.query_tokens
    out["page_tokens"] = list(st.page_tokens)
    return out


def kv_get_info(h) -> dict:
    info = _abi.KvInfo()
    _check(_lib.kv_get_info(h, C.byref(info)), "kv_get_info")
    return {name: getattr(info, name) for name, _ in _abi.KvInfo._fields_}


def rpkv_strerror(code: int) -> str:
    return _lib.rpkv_strerror(code).decode()


# ---- convenience: device memory from torch --------------------------------

ROPE_INTERLEAVED = 0
ROPE_HALF_SPLIT = 1


def make_spec(head_dim=64, pairs=(12, 10, 10), theta=10000.0, ntk_factor=1.0, max_frames=1,
              max_h=1, max_w=1, layout=ROPE_INTERLEAVED) -> Rope3dSpec:
    return Rope3dSpec(head_dim, pairs[0], pairs[1], pairs[2], theta, ntk_factor, max_frames,
                      max_h, max_w, layout)


def make_config(*, num_layers, num_streams, num_heads, grid_h, grid_w, dtype="bf16", head_dim=64,
                special_tokens=6, patch_page_size=None, special_page_size=6, scale_frames=0,
                sliding_window=0, max_keyframes=1, attn_splits=0, rope: Rope3dSpec) -> KvConfig:
    dt = {"bf16": RPKV_BF16, "f32": RPKV_F32}[dtype]
    pps = patch_page_size or grid_h * grid_w
    return KvConfig(num_layers, num_streams, num_heads, head_dim, dt, grid_h, grid_w,
                    special_tokens, pps, special_page_size, scale_frames, sliding_window,
                    max_keyframes, attn_splits, rope)


class PagedKVCache:
    """A handle plus the torch-allocated device memory and rotary tables it uses.

    Methods take torch tensors (or raw pointers) and the current torch stream."""

    def __init__(self, cfg: KvConfig, device="cuda"):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        if self.device.index is None:   # "cuda" -> the current device, as tensors report it
            self.device = torch.device(self.device.type, torch.cuda.current_device())
        nbytes = kv_required_bytes(cfg)
        if nbytes == 0:
            raise RpkvError(RPKV_EINVAL, "kv_required_bytes")
        # 256-byte aligned: torch's caching allocator returns >= 512-byte aligned blocks
        self.mem = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        tb = rope3d_tables_bytes(cfg.rope)
        self.tables = torch.empty(tb, dtype=torch.uint8, device=self.device)
        rope3d_build_tables(cfg.rope, self.tables, tb, self.stream)
        self.h = kv_create(cfg, self.mem, nbytes, self.stream)

    @property
    def stream(self) -> int:
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def _expect(self, name, t, shape, dtype):
        """The C ABI takes bare pointers: check a torch tensor's shape, dtype,
        device and layout here, before anything is launched (raw integer
        pointers are passed through unchecked)."""
        if t is None or isinstance(t, int):
            return
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != self.device \
                or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous {dtype} tensor of shape {tuple(shape)} "
                             f"on {self.device}, got {t.dtype} {tuple(t.shape)} on {t.device}"
                             f"{'' if t.is_contiguous() else ' (not contiguous)'}")

    def _act(self, name, t, rows=None):
        c = self.cfg
        dt = self.torch.bfloat16 if c.dtype == RPKV_BF16 else self.torch.float32
        n = c.special_tokens + c.grid_h * c.grid_w
        self._expect(name, t, (c.num_streams, n, c.num_heads, c.head_dim), dt)

    def close(self):
        if getattr(self, "h", None) is not None:
            kv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self, layer: int = -1):
        kv_reset(self.h, layer, self.stream)

    def append(self, layer, frame_idx, commit, q, k, v, q_rot, grid=None):
        """grid: this frame's (grid_h, grid_w) if it differs from the configured one."""
        for name, t in (("q", q), ("k", k), ("v", v), ("q_rot", q_rot)):
            self._act(name, t)
        if grid is None:
            kv_append_frame(self.h, layer, frame_idx, commit, q, k, v, q_rot, self.tables,
                            self.stream)
        else:
            kv_append_frame_grid(self.h, layer, frame_idx, commit, grid[0], grid[1], q, k, v,
                                 q_rot, self.tables, self.stream)

    def project_append(self, layer, frame_idx, commit, x, w, q_rot, grid=None):
        """Fused projection + RoPE + append: x [S][N][hidden] bf16, w [3*H*D][hidden] bf16;
        grid: this frame's (grid_h, grid_w) if it differs from the configured one."""
        c, bf = self.cfg, self.torch.bfloat16
        n = c.special_tokens + c.grid_h * c.grid_w
        hidden = x.shape[-1]
        self._expect("x", x, (c.num_streams, n, hidden), bf)
        self._expect("w", w, (3 * c.num_heads * c.head_dim, hidden), bf)
        self._act("q_rot", q_rot)
        if grid is None:
            kv_project_append_frame(self.h, layer, frame_idx, commit, x, hidden, w, q_rot,
                                    self.tables, self.stream)
        else:
            kv_project_append_frame_grid(self.h, layer, frame_idx, commit, grid[0], grid[1], x,
                                         hidden, w, q_rot, self.tables, self.stream)

    def attend(self, layer, q_rot, out, lse=None):
        self._act("q_rot", q_rot)
        self._act("out", out)
        c = self.cfg
        self._expect("lse", lse, (c.num_streams, c.num_heads, c.special_tokens + c.grid_h * c.grid_w),
                     self.torch.float32)
        attend_frame(self.h, layer, q_rot, out, lse, self.stream)

    def attend_noalloc(self, layer, q_rot, out, lse=None):
        """attend_frame_noalloc: the split partials in the library's static scratch."""
        self._act("q_rot", q_rot)
        self._act("out", out)
        c = self.cfg
        self._expect("lse", lse, (c.num_streams, c.num_heads, c.special_tokens + c.grid_h * c.grid_w),
                     self.torch.float32)
        attend_frame_noalloc(self.h, layer, q_rot, out, lse, self.stream)

    def evict(self, layer):
        kv_evict_deferred(self.h, layer, self.stream)

    def rollback(self, layer):
        kv_rollback(self.h, layer, self.stream)

    def state(self, layer=0, stream_idx=0) -> dict:
        return kv_read_state(self.h, layer, stream_idx, self.stream)

    def info(self) -> dict:
        return kv_get_info(self.h)

    # Views of the pools (for tests): K [L][S][H][pool][slot_cap][D],
    # V^T [L][S][H][pool][D][slot_cap], K special [L][S][H][sp_cap][D],
    # V^T special [L][S][H][D][sp_cap].
    def pool_views(self):
        torch = self.torch
        info = self.info()
        cfg = self.cfg
        dt = torch.bfloat16 if cfg.dtype == RPKV_BF16 else torch.float32
        el = 2 if cfg.dtype == RPKV_BF16 else 4
        L, S, H, D = cfg.num_layers, cfg.num_streams, cfg.num_heads, cfg.head_dim
        pool, cap, spc = info["pool_pages"], info["slot_capacity"], info["special_capacity"]
        kpool_b = L * S * H * pool * cap * D * el
        ksp_b = L * S * H * spc * D * el
        m = self.mem
        o = info["off_kpool"]
        kp = m[o:o + kpool_b].view(dt).view(L, S, H, pool, cap, D)
        o = info["off_vpool"]
        vp = m[o:o + kpool_b].view(dt).view(L, S, H, pool, D, cap)
        o = info["off_ksp"]
        ks = m[o:o + ksp_b].view(dt).view(L, S, H, spc, D)
        o = info["off_vsp"]
        vs = m[o:o + ksp_b].view(dt).view(L, S, H, D, spc)
        return kp, vp, ks, vs


def vslot_perm(p):
    """Storage position <-> key index inside a 16-slot group of a transposed V page."""
    return (p & ~12) | (((p >> 2) & 1) << 3) | (((p >> 3) & 1) << 2)
