"""Build libw8a8.so in-tree with hipcc for gfx950.

Every HIP source is compiled with IEEE binary32 division and square root
(correctly rounded), without FP contraction, without packed-FP32
instructions and without moving per-thread arrays into LDS, then linked into
one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libw8a8.so")
# on-device reference rates for the benchmark (not part of the library's ABI)
PEAKS_LIB = os.path.join(HERE, "libpeaks.so")
# debug build: every kernel fills its LDS with a fixed pattern before use (W8A8_LDS_POISON);
# the GPU tests require its outputs to be bit-identical to the normal build's
POISON_LIB = os.path.join(HERE, "libw8a8_ldspoison.so")
POISON_FLAGS = ["-DW8A8_LDS_POISON"]
PEAKS_SOURCE = "peaks.hip"
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["quantize_rows.hip", "gemm_tiled.hip", "gemm_decode.hip", "bsr_gemm.hip", "sparse24.hip",
           "w4a16.hip", "w8a8_abi.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep per-thread address arrays in registers instead of LDS
    "-mllvm", "-disable-promote-alloca-to-lds=true",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the CPU tests: only the host
# half of each translation unit is instrumented (the gfx950 code objects are unchanged).
HOST_SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _compile(src: str, out_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build_library(jobs: int = 8) -> str:
    """Compile every source and link libw8a8.so, its LDS-poisoned debug twin
    libw8a8_ldspoison.so, and the benchmark's reference-rate kernels into libpeaks.so
    (always rebuilds)."""
    poison_dir = os.path.join(BUILD_DIR, "ldspoison")
    os.makedirs(poison_dir, exist_ok=True)
    jobs_list = [(s, BUILD_DIR, ()) for s in SOURCES + [PEAKS_SOURCE]]
    jobs_list += [(s, poison_dir, POISON_FLAGS) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs_list))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:n + 1], PEAKS_LIB)
    _link(objs[n + 1:], POISON_LIB)
    return LIB


def build_host_sanitized(lib: str, jobs: int = 8) -> str:
    """libw8a8.so with the host code under AddressSanitizer + UndefinedBehaviorSanitizer, for
    the CPU tests of the C ABI (loaded with clang's AddressSanitizer runtime preloaded)."""
    out_dir = os.path.join(os.path.dirname(lib), "objs")
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, HOST_SAN_FLAGS), SOURCES))
    _link(objs, lib)
    return lib


if __name__ == "__main__":
    print(build_library())
