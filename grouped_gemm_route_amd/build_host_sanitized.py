"""A host-sanitized build of libmoe_route.so, for checks on the CPU.

The host code (argument checks, size and workspace arithmetic, the entry
points' bookkeeping) is built with AddressSanitizer and UndefinedBehavior
Sanitizer, every report fatal; device code is built as usual.  The library
lands in ``_build/host_sanitized/`` and is loaded with the sanitizer runtime
preloaded (``runtime()``).  Run as
``python -m grouped_gemm_route_amd.build_host_sanitized``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

from .build import ARCH, BUILD, CSRC, INCLUDE, hipcc, sources

OUT = os.path.join(BUILD, "host_sanitized")
LIB = os.path.join(OUT, "libmoe_route.so")

# each host-only option follows its -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-Werror",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, *SAN]


def runtime():
    """The AddressSanitizer runtime of hipcc's clang (it carries the UBSan
    handlers too), to preload into an unsanitized Python."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm")
    found = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError(f"no AddressSanitizer runtime under {llvm}")
    return found[-1]


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    p = subprocess.run([hipcc(), *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{p.stderr}")
    return obj


def build(verbose=True):
    os.makedirs(OUT, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN[:4], "-shared-libsan",
           "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
