"""Build libpagedkv.so (gfx950) in-tree with hipcc.

    python -m paged_kv_cache_290_amd.build

Every HIP source compiles to an object under `_build/` (in parallel), then one shared
library is linked next to this file.  No GPU is needed: hipcc cross-compiles.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpagedkv.so")
SOURCES = ("api.hip", "kv_write.hip", "decode.hip", "prefill.hip", "cascade.hip", "blocks.hip",
           "planner.hip", "prefix.hip", "swap.hip", "probe.hip")
# Host-only C++ (no device code), compiled by the host compiler.
HOST_SOURCES = ("sha256_x86.cpp",)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"

# Packed fp32 VALU instructions are switched off for the device code (the host pass
# prints a harmless "not a recognized feature" warning for this flag).
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd: list[str], verbose: bool) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    if verbose and res.stdout.strip():
        print(res.stdout)


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile and link; returns the library path.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = CFLAGS + list(extra_flags or [])
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".cpp", ".host.o"))
        objs.append(obj)
        cmds.append([CXX, "-O3", "-std=c++17", "-fPIC", "-c", os.path.join(CSRC, src),
                     "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
