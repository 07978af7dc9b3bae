"""Build libmsgl.so in-tree with hipcc for gfx950.

    python -m paged_kv_attention_loc_amd.build

Every source under csrc/ is compiled to an object in parallel, then linked
into ``paged_kv_attention_loc_amd/libmsgl.so``.  Packed-fp32 VALU forms are
turned off for all device code (they are not used by the kernels, and plain
fp32 keeps results reproducible).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmsgl.so")
ARCH = "gfx950"

SOURCES = ["abi.hip", "store_kv.hip", "decode.hip", "extend.hip", "mixed.hip", "rope.hip", "alloc.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmsgl.so)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source and link libmsgl.so; returns its path."""
    hipcc = _hipcc()
    flags = COMMON_FLAGS + list(extra_flags or [])
    tmp = tempfile.mkdtemp(prefix="msgl_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
            if verbose and res.stderr.strip():
                print(res.stderr, file=sys.stderr)
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        out_tmp = LIB + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
