"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libpagedkv is rebuilt with the sanitizers on its host code only
(device code is compiled as usual), linked into `tests/sanitize/host_driver.cpp`,
and run: a random serving loop over the block allocator, prefix caching and the
chunked-prefill planner, the metadata validator, and the argument checks of the GPU
entry points (all of them return before any launch, so no GPU is needed).  Any
memory error or undefined behaviour fails the test.
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_290_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs the ROCm compilers")
def test_host_code_is_clean_under_sanitizers():
    from paged_kv_cache_290_amd import build as B

    os.makedirs(OUT, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmds, objs = [], []
    for src in B.SOURCES:
        obj = os.path.join(OUT, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, *inc,
                     "-c", os.path.join(CSRC, src), "-o", obj])
    for src in B.HOST_SOURCES:
        obj = os.path.join(OUT, src.replace(".cpp", ".host.o"))
        objs.append(obj)
        cmds.append([CLANG, "-O1", "-g", "-std=c++17", "-fPIC", "-fsanitize=address,undefined",
                     "-fno-sanitize-recover=undefined", *inc, "-c", os.path.join(CSRC, src),
                     "-o", obj])
    drv = os.path.join(OUT, "host_driver.o")
    cmds.append([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=undefined", *inc, "-c",
                 os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", drv])
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_run, cmds))
    exe = os.path.join(OUT, "host_driver")
    _run([HIPCC, f"--offload-arch={B.ARCH}", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", drv, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "host driver ok" in r.stdout, r.stdout + r.stderr
    shutil.rmtree(OUT, ignore_errors=True)
