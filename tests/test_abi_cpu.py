"""CPU-only checks of the C ABI: the library loads, exports every function
declared in include/rpkv.h, the ctypes structures match the C layout (checked
against a gcc-compiled probe of the header), and the pure host functions
validate their arguments.  No kernel is launched."""
import ctypes as C
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rpkv.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+\*?([a-z_0-9]+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    from rope_paged_kv_amd import _abi
    lib = C.CDLL(_abi.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_abi.EXPORTS) == names


def test_struct_layout_matches_header():
    from rope_paged_kv_amd import _abi
    src = r'''
    #include <stdio.h>
    #include <stddef.h>
    #include "rpkv.h"
    int main(void) {
      printf("%zu %zu %zu %zu\n", sizeof(rope3d_spec), sizeof(kv_config), sizeof(kv_state_host), sizeof(kv_info));
      printf("%zu %zu %zu\n", offsetof(kv_config, rope), offsetof(kv_state_host, visible_pages),
             offsetof(kv_info, frames_committed));
      return 0;
    }'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "p.c")
        exe = os.path.join(d, "p")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    got = [C.sizeof(_abi.Rope3dSpec), C.sizeof(_abi.KvConfig), C.sizeof(_abi.KvStateHost),
           C.sizeof(_abi.KvInfo), _abi.KvConfig.rope.offset, _abi.KvStateHost.visible_pages.offset,
           _abi.KvInfo.frames_committed.offset]
    assert [int(x) for x in out] == got


def test_host_validation():
    import rope_paged_kv_amd as r
    spec = r.make_spec(max_frames=64, max_h=37, max_w=37)
    assert r.rope3d_tables_bytes(spec) == (64 * 12 + 37 * 10 + 37 * 10) * 8
    assert r.rope3d_tables_bytes(r.make_spec(pairs=(12, 10, 9))) == 0
    good = dict(num_layers=1, num_streams=1, num_heads=16, grid_h=37, grid_w=37, scale_frames=8,
                sliding_window=16, max_keyframes=64, rope=spec)
    n = r.kv_required_bytes(r.make_config(**good))
    # K + V pools: 25 pages x 16 heads x 1408 padded slots x 64 x 2 B each
    assert n > 2 * 25 * 16 * 1408 * 64 * 2
    for bad in (dict(head_dim=128), dict(grid_h=38), dict(patch_page_size=100),
                dict(special_tokens=65), dict(scale_frames=300, sliding_window=300),
                dict(num_heads=0)):
        assert r.kv_required_bytes(r.make_config(**{**good, **bad})) == 0, bad
    with pytest.raises(r.RpkvError):
        r.kv_create(r.make_config(**{**good, "grid_w": 40}), 0, 0, 0)
    assert r.rpkv_strerror(r.RPKV_ENOSPACE).startswith("cache pool")


def test_vslot_perm_is_an_involution_on_16_groups():
    from rope_paged_kv_amd import vslot_perm
    for p in range(64):
        assert vslot_perm(vslot_perm(p)) == p
        assert vslot_perm(p) // 16 == p // 16
    assert [vslot_perm(p) for p in range(16)] == [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]


def test_residual_add_validates_before_launching():
    import rope_paged_kv_amd as r
    for x, o, xb, n in ((256, 512, 768, -1), (0, 512, 768, 8), (256, 0, 768, 8),
                        (264, 512, 768, 8), (256, 520, 768, 8), (256, 512, 776, 8),
                        (256, 512, None, 1 << 40)):
        with pytest.raises(r.RpkvError) as e:
            r.residual_add_bf16(x, o, xb, n, 0)
        assert e.value.code == r.RPKV_EINVAL, (x, o, xb, n)
    r.residual_add_bf16(256, 512, None, 0, 0)   # n = 0 launches nothing


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback: without librpkv.so the binding raises instead of running
    anything else."""
    from rope_paged_kv_amd import _abi
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", "/nonexistent/librpkv.so")
    with pytest.raises(RuntimeError, match="missing"):
        _abi.load()
