"""Builds the gfx950 HIP library ``libdit.so`` in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-FP32 instructions
disabled (``-packed-fp32-ops``), then linked into one shared library next
to this file. Object files go to ``_build/`` at the repository root."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdit.so")
OUT_F32 = os.path.join(PKG, "libdit_f32.so")
SOURCES = ["gemm.hip", "attention.hip", "mask.hip", "elementwise.hip", "head.hip", "peak.hip",
           "dit_api.cpp"]
# fp32 debug build: fp32 activations / cache / attention, plain FMA GEMMs
SOURCES_F32 = ["debug_f32.hip", "mask.hip", "elementwise.hip", "head.hip", "dit_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _compile(src: str, bdir: str, extra=()) -> str:
    obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _build_one(sources, out, bdir, extra=()):
    os.makedirs(bdir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(sources))) as ex:
        objs = list(ex.map(lambda s: _compile(s, bdir, extra), sources))
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Builds libdit.so (bf16) and libdit_f32.so (fp32 debug build)."""
    _build_one(SOURCES, OUT, os.path.join(ROOT, "_build"))
    _build_one(SOURCES_F32, OUT_F32, os.path.join(ROOT, "_build", "f32"), ("-DDIT_F32",))
    if verbose:
        print(f"built {OUT} and {OUT_F32}", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
