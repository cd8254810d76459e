"""Build liblcsi.so (gfx950) in-tree with hipcc.

    python -m long_context_sparse_idx_amd.build

Objects go to long_context_sparse_idx_amd/_build/, the library next to this
file.  Every HIP source is compiled with packed-fp32 VALU ops disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblcsi.so")
SOURCES = ["score.hip", "select.hip", "attn.hip", "overlap.hip", "api.hip"]
CEILING_SOURCES = ["ceiling.hip"]
CEILING_LIB = os.path.join(PKG, "libceiling.so")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


# Per-source flags.  score.hip, attn.hip: NaN inputs are outside the
# contract, so fmaxf needs no NaN-quieting instruction.
SOURCE_FLAGS = {"score.hip": ["-fno-honor-nans"], "attn.hip": ["-fno-honor-nans"]}


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *CFLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    r = subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, extra=()) -> str:
    """Build liblcsi.so (the library) and libceiling.so (the benchmark's
    matrix-core ceiling helper)."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES + CEILING_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CEILING_LIB)
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
