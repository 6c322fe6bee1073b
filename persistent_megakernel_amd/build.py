"""Build libamk.so in-tree with hipcc for gfx950.

Device sources (.hip) are compiled with packed fp32 arithmetic disabled (the hardware's
packed fp32 forms are avoided on this target) and without type-based alias analysis (the kernels
reinterpret LDS bytes between widths); host sources (.cpp) are plain C++17 built with g++.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libamk.so")
BENCH = os.path.join(HERE, "amk_bench")
ARCH = "gfx950"

HIP_SOURCES = ["megakernel.hip", "prep.hip", "prefill.hip"]
CPP_SOURCES = ["abi.cpp", "lower.cpp", "lower_prefill.cpp", "validate.cpp", "vm.cpp"]


def _hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError("compile failed: " + os.path.basename(cmd[-1]))
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libamk.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append([hipcc, "-c", "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall",
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-strict-aliasing",
                     "-Wno-unused-function", "-Wno-unused-variable", *inc, "-o", obj, os.path.join(CSRC, s)])
    for s in CPP_SOURCES:   # host-only C++ (no device code): the system C++ compiler
        obj = os.path.join(BUILD, s + ".o")
        jobs.append(["g++", "-c", "-O2", "-fPIC", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
                     "-I", "/opt/rocm/include", *inc, "-o", obj, os.path.join(CSRC, s)])
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            sys.stderr.write(o.stderr)
    objs = [j[j.index("-o") + 1] for j in jobs]
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, "-pthread"])
    os.replace(tmp, LIB)
    # the C-ABI benchmark driver (links the library, no device code of its own)
    tmp = BENCH + ".tmp%d" % os.getpid()
    _run(["g++", "-O2", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", *inc,
          "-o", tmp, os.path.join(CSRC, "amk_bench.cpp"), "-L", HERE, "-lamk", "-L", "/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,$ORIGIN", "-Wl,-rpath,/opt/rocm/lib"])
    os.replace(tmp, BENCH)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
