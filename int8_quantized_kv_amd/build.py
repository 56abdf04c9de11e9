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


# Host-side sanitizer build (a CPU check of the host validation layer, not a
# product library): every translation unit at -O0 with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host pass only; the device pass is left
# alone.  Loaded with the compiler's ASan runtime preloaded (see san_env).
SAN_DIR = os.path.join(PKG, "_san")
SAN_LIB = os.path.join(SAN_DIR, "libkvq.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def san_runtime() -> str:
    """Path of the compiler's shared ASan runtime (it carries UBSan's handlers)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isfile(path):
        hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        if not hits:
            raise RuntimeError("no libclang_rt.asan-x86_64.so found")
        path = hits[-1]
    return path


def san_env() -> dict:
    """Environment that loads the sanitized library under the ASan runtime."""
    env = dict(os.environ)
    env["KVQ_LIBRARY"] = SAN_LIB
    env["LD_PRELOAD"] = san_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def build_sanitized(verbose: bool = True) -> str:
    """Compile and link the sanitizer build into _san/libkvq.so (skipped when
    it is newer than every source and header)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(SRC, "*.hip")))
    deps = sources + glob.glob(os.path.join(SRC, "*.hpp")) + glob.glob(os.path.join(INCLUDE, "*.h")) + [__file__]
    if os.path.exists(SAN_LIB) and os.path.getmtime(SAN_LIB) > max(os.path.getmtime(d) for d in deps):
        return SAN_LIB
    common = [a for a in COMMON if a != "-O3"] + ["-O0", "-g"] + SAN_FLAGS

    def one(src: str) -> str:
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        r = subprocess.run([HIPCC, *common, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(one, sources))
    tmp = SAN_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libsan", "-o", tmp,
                        *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


# Debug build: the C ABI translation unit compiled with -DKVQ_DEBUG (host-side
# checks of lengths and page ids before each attention launch), linked with
# the release build's other objects.  Run build() first.
DBG_DIR = os.path.join(PKG, "_dbg")
DBG_LIB = os.path.join(DBG_DIR, "libkvq.so")


def build_debug(verbose: bool = True) -> str:
    os.makedirs(DBG_DIR, exist_ok=True)
    api = os.path.join(SRC, "kvq_api.hip")
    obj = os.path.join(DBG_DIR, "kvq_api.hip.o")
    r = subprocess.run([HIPCC, *COMMON, "-DKVQ_DEBUG", "-c", api, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"debug build failed:\n{r.stdout}\n{r.stderr}")
    others = [os.path.join(OUT_DIR, os.path.basename(src) + ".o") for src in sorted(glob.glob(os.path.join(SRC, "*.hip")))
              if os.path.basename(src) != "kvq_api.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"debug build needs the release objects first (missing {missing[0]})")
    tmp = DBG_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj, *others],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"debug link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, DBG_LIB)
    if verbose:
        print(f"built {DBG_LIB}")
    return DBG_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--sanitize":
        build_sanitized()
    elif len(sys.argv) > 1 and sys.argv[1] == "--debug":
        build_debug()
    else:
        build()
        build_debug()
