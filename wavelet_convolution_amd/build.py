"""Build libwtconv.so (HIP, gfx950) in-tree with hipcc.

    python -m wavelet_convolution_amd.build

Every translation unit compiles in parallel into ``_build/`` and is linked
into ``wavelet_convolution_amd/libwtconv.so``. Packed-fp32 instructions are
switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libwtconv.so")
SOURCES = ["wtconv_fused.hip", "wtconv_tiled.hip", "wtconv_bwdw.hip", "wtconv_naive.hip", "wtconv_api.hip",
           "wtconv_peaks.hip", "wtconv_layout.hip", "wtconv_dw.hip", "wtconv_bwd1.hip",
           *(f"wtconv_fam{h}_{kind}.hip" for h in (56, 28, 14, 7) for kind in ("data", "bw"))]
ARCH = os.environ.get("WTCONV_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the WTConv HIP library cannot be built")
    return path


def _inputs_hash(src: str) -> str:
    """Hash of a translation unit's inputs: its source, every header beside
    it and the flags (headers are few, so all of them count)."""
    h = hashlib.sha256(" ".join(HIPCC_FLAGS).encode())
    for name in [src] + sorted(f for f in os.listdir(CSRC) if f.endswith(".h")) + ["../../include/wtconv.h"]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    stamp = obj + ".inputs"
    digest = _inputs_hash(src)
    if incremental and os.path.exists(obj) and os.path.exists(stamp) and open(stamp).read() == digest:
        return obj
    cmd = [_hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    with open(stamp, "w") as f:
        f.write(digest)
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every HIP source and link libwtconv.so; return its path.
    With incremental=True (a development aid, off by default), translation
    units whose inputs are unchanged since their last compile are reused."""
    os.makedirs(OUT_DIR, exist_ok=True)
    workers = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv[1:])
    sys.exit(0)
