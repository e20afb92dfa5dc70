"""Builds librpkv.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python rope_paged_kv_amd/build.py      (run by path: importing the package
                                            loads the library this builds)
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "librpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 instructions stay off: the compiler must not emit them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs (no AGPR copies around the
    # softmax that reads them)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]
# Attention only: its data holds no NaN (masked scores are -inf), so min/max
# need no NaN quieting and fold into v_max3.
EXTRA = {"k_attend_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    with tempfile.TemporaryDirectory() as tmpd:
        objs = []
        for src in sources():
            obj = os.path.join(tmpd, os.path.basename(src) + ".o")
            _run([HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), *inc, "-c", src, "-o", obj],
                 verbose)
            objs.append(obj)
        tmp = LIB + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
