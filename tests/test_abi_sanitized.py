"""tests/test_abi.py again, against a host-sanitized build of the library
(AddressSanitizer and UndefinedBehaviorSanitizer on the host pass), in a
child process with the compiler's ASan runtime preloaded.  CPU only: what
runs is the host validation layer (argument checks, size arithmetic, error
paths); no kernel is launched.  The first run builds the sanitized library
(about a minute); later runs reuse it until a source changes."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("kvq_build", os.path.join(ROOT, "int8_quantized_kv_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_under_asan_and_ubsan():
    b = _build_module()
    lib = b.build_sanitized(verbose=False)
    env = b.san_env()
    # the child loads the sanitized library, with the sanitizer runtime live
    probe = ("import ctypes, int8_quantized_kv_amd.kvq as k; "
             "ctypes.CDLL(None).__asan_init; print(k.LIB_PATH)")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert os.path.realpath(r.stdout.strip().splitlines()[-1]) == os.path.realpath(lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
