"""Build libpkv.so in-tree: HIP kernels for gfx950 plus the host allocator.

Usage: ``python paged_kv_cache_292_amd/build.py`` (run as a file: importing the
package would load the library being rebuilt).
Host-only C++ is compiled with g++; ``.hip`` files with hipcc for gfx950;
everything is linked by hipcc into ``paged_kv_cache_292_amd/libpkv.so``.
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
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")

ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: without this the decode
    # kernel kept them in AGPRs and copied all of them to VGPRs and back on
    # every loop iteration (and ran at 2 instead of 3 waves per SIMD)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-result",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + p.stdout)
    return p.stdout


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libpkv.so``; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    hipcc = _hipcc()
    hip, cpp = sources()
    inc = ["-I", INCLUDE, "-I", CSRC]
    jobs = []
    objs = []
    for f in hip:
        o = os.path.join(OUT_DIR, f + ".o")
        jobs.append([hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    for f in cpp:
        o = os.path.join(OUT_DIR, f + ".o")
        jobs.append(["g++", *CXX_FLAGS, *inc, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    workers = max(1, min(8, len(jobs), (os.cpu_count() or 2)))
    with ThreadPoolExecutor(workers) as ex:
        logs = list(ex.map(_run, jobs))
    if verbose:
        for line in logs:
            if line.strip():
                print(line)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5", *objs,
          "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
