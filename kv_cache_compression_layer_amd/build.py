"""Build libcachegen_mi355x.so from the HIP sources with hipcc for gfx950.

Usage: ``python -m kv_cache_compression_layer_amd.build`` (or call
:func:`build`). Objects are compiled in parallel, then linked into
``kv_cache_compression_layer_amd/_build/libcachegen_mi355x.so``.

Flags:
  --offload-arch=gfx950      MI355X only; no other targets.
  -ffp-contract=off          every float operation rounds on its own (the
                             quantiser and dequantiser must not fuse a*b+c).
  -Xclang -target-feature -Xclang -packed-fp32-ops
                             no packed fp32 instructions (v_pk_*_f32).
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libcachegen_mi355x.so"
LIB_PATH = os.path.join(OUT_DIR, LIB_NAME)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], check=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
