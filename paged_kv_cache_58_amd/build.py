"""Build libpa.so for gfx950 with hipcc (in-tree, no JIT cache).

Every HIP source is compiled with ``-Xclang -target-feature -Xclang
-packed-fp32-ops`` so the compiler never emits packed fp32 arithmetic.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
DEBUG_LIB = os.path.join(PKG, "libpa_debug.so")  # PA_DEBUG: device checks of the index arrays
ARCH = "gfx950"

SOURCES = ["plan.cpp", "block_manager.cpp", "api.cpp", "append.hip", "grouped_decode.hip",
           "gqa_mfma_decode.hip", "latent_decode.hip", "mxfp8_append.hip", "block_copy.hip",
           "attention_scores.hip", "noalloc.hip"]
HOST_ONLY = {"plan.cpp", "block_manager.cpp", "api.cpp"}  # pure C++: no HIP headers
# The debug library links the release objects except api.cpp, which it
# compiles again with PA_DEBUG, plus the check kernels.
DEBUG_SOURCES = ["api.cpp", "debug_checks.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden", "-Wall",
          "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]
# Per-source extras.  The matrix-core grouped kernel keeps its accumulators in
# ordinary VGPRs (its rare rescale multiplies them on the VALU; in the
# accumulation registers every block would copy them out and back).
EXTRA = {"gqa_mfma_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, debug: bool = False) -> str:
    path = os.path.join(CSRC, src)
    out_dir = os.path.join(BUILD, "debug") if debug else BUILD
    obj = os.path.join(out_dir, src.rsplit(".", 1)[0] + ".o")
    flags = [*COMMON, "-DPA_DEBUG=1"] if debug else COMMON
    if src in HOST_ONLY:  # built by the host compiler
        cmd = ["g++", *flags, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *DEVICE, *flags, *EXTRA.get(src, []), "-x", "hip", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(lib: str, objs) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link libpa.so and libpa_debug.so.  Always
    rebuilds."""
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [(src, True) for src in DEBUG_SOURCES]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    release = objs[:len(SOURCES)]
    debug_objs = dict(zip(DEBUG_SOURCES, objs[len(SOURCES):]))
    _link(LIB, release)
    _link(DEBUG_LIB, [debug_objs.get(src, o) for src, o in zip(SOURCES, release)] +
          [o for src, o in debug_objs.items() if src not in SOURCES])
    if verbose:
        print(f"built {LIB} and {DEBUG_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
