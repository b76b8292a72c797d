"""Build libkbit.so in-tree with hipcc for gfx950.

    python -m blockwise_bit_codebook_amd.build [-v] [-j N]

HIP translation units are compiled for gfx950 only, with IEEE binary32
division and square root, no contraction of multiply-add, denormals kept and
packed fp32 instructions disabled; host-only C++ files are compiled as plain
C++.  Objects go to ``_build/`` next to the package; the shared library
lands in the package directory.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkbit.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_SOURCES = ["quantize.hip", "dequantize.hip", "nested_encode.hip", "linear.hip", "act_fwht.hip",
               "act_block.hip"]
CXX_SOURCES = ["api.cpp", "codebook.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC]
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
CXX_FLAGS = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-ffp-contract=off", "-fno-fast-math",
             "-I", os.path.join(ROCM, "include")]


USAGE_REMARK = "-Rpass-analysis=kernel-resource-usage"


def _scratch_kernels(lines):
    """(function, bytes per lane) for every function whose resource-usage
    remark reports a nonzero ScratchSize."""
    bad, fn = [], None
    for l in lines:
        if "Function Name:" in l:
            fn = l.split("Function Name:", 1)[1].split("[-R", 1)[0].strip()
        elif "ScratchSize [bytes/lane]:" in l:
            n = int(l.split("ScratchSize [bytes/lane]:", 1)[1].split()[0])
            if n:
                bad.append((fn, n))
    return bad


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    hip = src.endswith(".hip")
    flags = HIP_FLAGS + [USAGE_REMARK] if hip else CXX_FLAGS
    cmd = [HIPCC] + COMMON + flags + ["-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    lines = (r.stdout + r.stderr).splitlines()
    out = "\n".join(l for l in lines if "packed-fp32-ops" not in l and "unused during compilation" not in l
                    and "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    # Every kernel keeps its state in registers and LDS: a spill to scratch
    # (private memory) is a build error, not a silent slowdown.
    spills = _scratch_kernels(lines) if hip else []
    if spills:
        raise RuntimeError(f"{src}: kernels use scratch memory: " +
                           ", ".join(f"{f} ({n} B/lane)" for f, n in spills))
    if out.strip() and verbose:
        print(out)
    return obj


def build(verbose=False, jobs=None):
    """Compile every source and link libkbit.so; returns the library path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = HIP_SOURCES + CXX_SOURCES
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    shutil.move(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    a = ap.parse_args(argv)
    print(build(verbose=a.verbose, jobs=a.jobs))


if __name__ == "__main__":
    sys.exit(main())
