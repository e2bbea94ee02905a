"""Build libpagedkv.so (HIP for gfx950) in-tree.

    python -m paged_kv_cache_323_amd.build          # compile every source, link the library

Every HIP source is compiled with packed-fp32 instruction selection disabled; the host-only
block manager is compiled with the system C++ compiler.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
# The same sources with bounds checks of device-resident indices (PKV_DEBUG_CHECKS).
DEBUG_LIB = os.path.join(PKG, "libpagedkv_debug.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
# Per-source extra flags. The prefill kernel's scores are never NaN (its clamped keys are written
# rows and masking selects by position), so it runs with IEEE mode off: fmax then needs no
# quieting of its operands, which would otherwise cost one extra instruction per score. Its one
# inf/NaN test (a V value beyond the f16 range) reads exponent bits as integers.
FILE_FLAGS = {"ragged.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-I", INCLUDE]


def _hip_sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip")) + [
        os.path.join(CSRC, "api.cpp")]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in p.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8, defines=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile and link; ``defines`` are extra -D macros (kernel tuning knobs)."""
    if not out.endswith(".so"):
        raise ValueError(f"output must be a .so path, got {out!r}")
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(build_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    jobs_list = []
    objs = []
    for src in _hip_sources():
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        extra = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs_list.append([HIPCC, *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *dflags, *extra, "-c", src,
                          "-o", obj])
        objs.append(obj)
    bm_src = os.path.join(CSRC, "block_manager.cpp")
    bm_obj = os.path.join(build_dir, "block_manager.cpp.o")
    cxx = shutil.which("g++") or "c++"
    jobs_list.append([cxx, *HOST_FLAGS, "-c", bm_src, "-o", bm_obj])
    objs.append(bm_obj)
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        for log in ex.map(_run, jobs_list):
            if verbose and log.strip():
                print(log)
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


PROBE_SRC = os.path.join(CSRC, "probe", "stream_read.hip")
PROBE_LIB = os.path.join(PKG, "libpkv_probe.so")


def build_probe() -> str:
    """The benchmark's streaming-read and tile-gather probes (their own small library, outside
    libpagedkv)."""
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", PROBE_SRC, "-o", tmp])
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


TOKEN_MAJOR_LIB = os.path.join(PKG, "tuning", "libpagedkv_token_major.so")


def build_token_major() -> str:
    """A tuning build that stores the pools token-major ([N][B][H][D]) in the cache write and reads
    them so in decode, used only to measure the layout choice (bench.py --layout-study token). Its
    prefill kernel and pool-layout contract are the head-major ones: not a product library."""
    os.makedirs(os.path.dirname(TOKEN_MAJOR_LIB), exist_ok=True)
    return build(defines=("PKV_TOKEN_MAJOR",), out=TOKEN_MAJOR_LIB, build_dir=os.path.join(BUILD, "token_major"))


def build_all(verbose: bool = False):
    """The release library, the debug (bounds-checked) library and the benchmark's probe."""
    return [build(verbose=verbose),
            build(verbose=verbose, defines=("PKV_DEBUG_CHECKS",), out=DEBUG_LIB,
                  build_dir=os.path.join(BUILD, "debug")),
            build_probe()]


if __name__ == "__main__":
    if "--token-major" in sys.argv:
        print(build_token_major())
    else:
        print("\n".join(build_all(verbose="-v" in sys.argv)))
