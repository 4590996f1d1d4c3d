"""Build the HIP library libhyena_mi355x.so in-tree for gfx950.

Usage: python -m hyena_long_conv_amd.build   (or hyena_long_conv_amd.build.build())

Each translation unit is compiled by hipcc in parallel into _build/, then
linked into hyena_long_conv_amd/libhyena_mi355x.so.  Packed FP32 VALU
instructions are disabled for the device code (-packed-fp32-ops).
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
LIB = os.path.join(PKG, "libhyena_mi355x.so")

SOURCES = ["api.cpp", "kernels_single.hip", "kernels_fourstep.hip", "kernels_filter.hip", "kernels_proj.hip",
           "kernels_fir.hip", "kernels_nd.hip", "kernels_bwd_long.hip", "scratch.hip"]
ARCH = os.environ.get("HYENA_OFFLOAD_ARCH", "gfx950")


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # x + 0 folds to x: the zero-padded FFT legs cost no adds
            "-fno-signed-zeros",
            "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def _compile(src: str, defines=(), tag: str = "") -> str:
    obj = os.path.join(BUILD, tag + os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    cmd = [_hipcc(), *(["-x", "hip"] if src.endswith(".hip") else []), *_common_flags(),
           *[f"-D{d}" for d in defines], "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, defines=(), out: str | None = None) -> str:
    """Compile and link; ``defines`` (NAME=VALUE strings) and ``out`` serve
    tuning builds of the same sources."""
    os.makedirs(BUILD, exist_ok=True)
    out = out or LIB
    tag = "" if out == LIB else os.path.basename(out) + "."
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, defines, tag), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


HOSTCHECK_LIB = os.path.join(BUILD, "libhyena_hostcheck.so")


def build_hostcheck(out: str = HOSTCHECK_LIB) -> str:
    """Host-only build of the C ABI for the sanitizers: api.cpp (argument
    checks, planning, size queries) and stand-ins for the kernel launchers
    (csrc/hostcheck_stubs.cpp), compiled by g++ with AddressSanitizer and
    UndefinedBehaviorSanitizer.  No device code is involved.  Load it with
    the sanitizer runtimes preloaded (tests/test_hostcheck.py)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", INCLUDE, "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "hostcheck_stubs.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host-check build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


if __name__ == "__main__":
    build()
    sys.exit(0)
