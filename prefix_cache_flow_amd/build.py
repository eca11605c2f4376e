"""Compile the HIP sources of the library into prefix_cache_flow_amd/libvla.so (gfx950).

Every source is compiled with hipcc for gfx950 only, optimised, without
fast-math (the ternary quantizer relies on IEEE division and round-to-even),
and with the packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libvla.so")
ARCH = "gfx950"

SOURCES = ["gemm.hip", "attention.hip", "norm.hip", "expert.hip", "w2a8.hip", "fused.hip", "runtime.cpp"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-unused-value",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), "-O3", "-std=c++17", "-fPIC", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"  compiled {src}", flush=True)
    return obj


def build(verbose: bool = True, jobs: int = 8) -> str:
    """Compile every source and link libvla.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"  linked {LIB}", flush=True)
    return LIB


ASAN_LIB = os.path.join(BUILD, "libvla_asan.so")
# host code only: each sanitizer flag goes to the host compilation (device code is built as usual)
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def asan_runtime() -> str:
    """The compiler's AddressSanitizer runtime (it carries the UBSan handlers too), preloaded into a
    process that loads the sanitized library."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/lib/llvm")
    return hits[-1]


def build_sanitized(verbose: bool = True) -> str:
    """libvla_asan.so: the host runtime (runtime.cpp: handles, validation, planning, graph cache)
    compiled with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the regular device
    objects.  Load it with the runtime from asan_runtime() preloaded."""
    dev_objs = [os.path.join(BUILD, src + ".o") for src in SOURCES if not src.endswith(".cpp")]
    if not all(os.path.exists(o) for o in dev_objs):
        build(verbose=False)
    obj = os.path.join(BUILD, "runtime.asan.o")
    cmd = [_hipcc(), "-std=c++17", "-fPIC", *SANITIZE, "-c", os.path.join(CSRC, "runtime.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling the sanitized runtime failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    objs = dev_objs + [obj]
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", ASAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking the sanitized library failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"  linked {ASAN_LIB}", flush=True)
    return ASAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
