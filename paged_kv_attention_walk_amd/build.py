"""Builds libpa_walk.so in-tree with hipcc for gfx950.

    python -m paged_kv_attention_walk_amd.build

Every call compiles from source; nothing is cached between calls.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa_walk.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

# Packed FP32 instructions are turned off for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]
MAX_QTOK = 8        # query tokens per decode call (one vector-path split-kernel object per count)
MFMA_MAX_QTOK = 5   # tokens of one matrix-core launch group (larger calls run as groups)


def _run(cmd, verbose):
    if verbose:
        print("+", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = True) -> str:
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    cxx = shutil.which("g++") or "g++"
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    hip_inc = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")]
    objs = []
    o = os.path.join(BUILD_DIR, "pa_alloc.o")
    _run([cxx, *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "pa_alloc.cpp"), "-o", o], verbose)
    objs.append(o)
    o = os.path.join(BUILD_DIR, "pa_host.o")
    _run([cxx, *HOST_FLAGS, *inc, *hip_inc, "-c", os.path.join(CSRC, "pa_host.cpp"), "-o", o], verbose)
    objs.append(o)
    # the device sources compile in parallel; the two split-kernel sources
    # are built once per query-token count (each instantiates every K x V
    # encoding pair for its count)
    cmds = []
    for name in ("pa_kernels", "pa_append", "pa_scratch"):
        o = os.path.join(BUILD_DIR, name + ".o")
        cmds.append([hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, name + ".hip"), "-o", o])
        objs.append(o)
    for name, top in (("pa_mfma", MFMA_MAX_QTOK), ("pa_valu", MAX_QTOK)):
        for t in range(1, top + 1):
            o = os.path.join(BUILD_DIR, f"{name}_t{t}.o")
            cmds.append([hipcc, *HIP_FLAGS, *inc, f"-DPA_T={t}", "-c", os.path.join(CSRC, name + ".hip"), "-o", o])
            objs.append(o)
    workers = max(1, min(len(cmds), os.cpu_count() or 8))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
    print(LIB)
