"""Build libhga.so (HIP C++ for gfx950) in-tree with hipcc.

Each source is compiled to an object in parallel, then linked into
long_context_fine_amd/libhga.so. Usage: python -m long_context_fine_amd.build

`--host-sanitize` also builds long_context_fine_amd/libhga_hostsan.so: the same
library with the host-side C-ABI layer (argument checks, workspace sizing,
dispatch) built with AddressSanitizer and UndefinedBehaviorSanitizer. Only host
code is instrumented; a process loading it needs the ASan runtime preloaded
(`asan_runtime()` gives its path).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libhga.so")
SAN_LIB_PATH = os.path.join(PKG, "libhga_hostsan.so")
SOURCES = ["hga_api.cpp", "summaries.hip", "route.hip", "gather.hip", "attn_fwd.hip", "attn_bwd.hip",
           "decode.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # keep the compiler from emitting packed-fp32 VALU instructions
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


# host-only instrumentation: each sanitizer flag applies to the host pass alone
_HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, verbose: bool, extra=(), suffix="") -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [_hipcc(), *_flags(), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload)."""
    clang = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(_hipcc()))), "lib", "llvm", "bin",
                         "clang++")
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError("the ASan runtime of the ROCm compiler was not found")
    return out


def _fresh(obj: str, src: str) -> bool:
    """obj exists and is newer than its source and every shared header."""
    if not os.path.exists(obj):
        return False
    deps = [os.path.join(CSRC, src), os.path.join(INCLUDE, "hga.h")] + \
        [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".hpp")]
    return os.path.getmtime(obj) >= max(os.path.getmtime(d) for d in deps)


def build_host_sanitized(verbose: bool = False) -> str:
    """libhga_hostsan.so: the C-ABI layer with ASan + UBSan on its host code,
    linked with the kernels' objects of the regular build (compiled here when
    missing or older than their sources)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    kernels = [s for s in SOURCES if s != "hga_api.cpp"]
    objs = []
    for src in kernels:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj if _fresh(obj, src) else _compile(src, verbose))
    api = _compile("hga_api.cpp", verbose, extra=["-O1", "-g", *_HOST_SAN], suffix="_hostsan")
    objs = [api] + objs
    tmp = SAN_LIB_PATH + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *_HOST_SAN[:4], "-Xarch_host",
           "-shared-libasan", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, SAN_LIB_PATH)
    return SAN_LIB_PATH


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
