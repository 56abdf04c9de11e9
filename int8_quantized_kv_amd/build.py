"""Ahead-of-time build of libkvq.so for gfx950 (MI355X).

Compiles every ``csrc/*.hip`` translation unit with hipcc and links them into
``int8_quantized_kv_amd/libkvq.so`` (in-tree, so the built library travels
with the source tree).  Usage: ``python int8_quantized_kv_amd/build.py`` (run
as a file: importing the package would load the library being rebuilt).
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvq.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    f"-I{INCLUDE}",
    # fp32 division and sqrt stay IEEE correctly rounded (quantization codes
    # depend on it); no fast-math, no denormal flushing.
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # never emit packed-fp32 VALU ops (device pass only; the host pass warns
    # that it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(line for line in r.stderr.splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile all HIP sources and link libkvq.so; returns the library path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(SRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources found")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
