"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The C ABI's host side (api.cpp: argument checks, planning; plan.cpp;
block_manager.cpp) is built with g++ -fsanitize=address,undefined into a
host-only library whose launchers report "no device" (sanitize/no_device.cpp),
and the oracle (pa_oracle.c) with gcc likewise.  The ABI suite (every
host-checked status), the block-manager suite (scenarios and random
operations against the independent model) and the oracle pins then run
again in a child process against those libraries, with the sanitizer
runtime preloaded; any report fails the test.  Device code is not
instrumented.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_58_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if gxx is None or gcc is None:
        pytest.skip("gcc/g++ not found")
    d = tmp_path_factory.mktemp("san")
    host = d / "libpa_host_san.so"
    srcs = [os.path.join(CSRC, f) for f in ("api.cpp", "plan.cpp", "block_manager.cpp")]
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "no_device.cpp"))
    subprocess.run([gxx, *SAN, "-std=c++17", "-shared", "-fPIC", "-fvisibility=hidden",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", str(host)],
                   check=True)
    orc = d / "liboracle_san.so"
    subprocess.run([gcc, *SAN, "-std=c11", "-fopenmp", "-shared", "-fPIC",
                    os.path.join(ROOT, "oracle", "pa_oracle.c"), "-o", str(orc), "-lm"],
                   check=True)
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("libasan.so not found")
    return str(host), str(orc), asan


def test_host_suites_clean_under_asan_ubsan(san_libs):
    host, orc, asan = san_libs
    env = dict(os.environ)
    env.update(PA_LIB=host, ORACLE_LIB=orc, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87",
               OMP_NUM_THREADS="4")
    env.pop("PA_DEBUG", None)
    suites = ["tests/test_abi.py", "tests/test_block_manager.py", "tests/test_oracle_pins.py",
              "tests/test_oracle_mxfp8.py", "tests/test_oracle_multi.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *suites],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout


def test_sanitizer_catches_a_planted_overflow(san_libs, tmp_path):
    """The same flags and preload do report a heap overflow (so a clean run
    above means something)."""
    _, _, asan = san_libs
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint bad(int n) { int *a = malloc(4 * n); "
                   "int r = a[n]; free(a); return r; }\n")
    so = tmp_path / "libbad.so"
    subprocess.run(["gcc", *SAN, "-shared", "-fPIC", str(src), "-o", str(so)], check=True)
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).bad(4)"
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
