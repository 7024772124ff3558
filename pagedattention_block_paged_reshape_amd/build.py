"""Build the C-ABI shared library (host block manager + gfx950 HIP kernels).

    python pagedattention_block_paged_reshape_amd/build.py [--sanitize]

compiles every source under csrc/ with hipcc for gfx950 (the host block
manager with g++) and links ``libpagedattn.so`` next to this file.

``--sanitize`` builds ``libpagedattn_san.so`` instead, for the CPU tests: the
host sources (block manager, scheduler, work-list planner) compiled by g++
with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
ordinary HIP objects.  Python is not instrumented, so a run preloads the
sanitizer runtimes and points the binding at this file:

    LD_PRELOAD="$(g++ -print-file-name=libasan.so) $(g++ -print-file-name=libubsan.so)" \
    ASAN_OPTIONS=detect_leaks=0:halt_on_error=1 \
    UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
    PA_LIBRARY=pagedattention_block_paged_reshape_amd/libpagedattn_san.so \
    python -m pytest tests -m "not gpu"
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedattn.so")
ARCH = "gfx950"

HIP_SOURCES = ["cache_ops.hip", "decode.hip", "mixed.hip", "prefill.hip"]
HOST_SOURCES = ["block_pool.cpp", "decode_plan.cpp", "scheduler.cpp"]

# Packed-FP32 VALU ops are kept out of the generated code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]
GXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
# host code only (g++; no HIP source is compiled or linked with these)
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
             "-fsanitize=address,undefined"]
SAN_LIB = os.path.join(PKG, "libpagedattn_san.so")
ROCM_LIB = "/opt/rocm/lib"
# Per-file extras: the attention kernels keep their MFMA accumulators in
# VGPRs, which they rescale with ordinary VALU ops (no AGPR round trips); for
# the prefill kernel this also fits two wavefronts per SIMD.
EXTRA_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "mixed.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, sanitize: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    hip_objs, host_objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        hip_objs.append(obj)
        jobs.append([hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + (".san.o" if sanitize else ".o"))
        host_objs.append(obj)
        flags = [*GXX_FLAGS, *SAN_FLAGS] if sanitize else GXX_FLAGS
        jobs.append(["g++", *flags, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    if sanitize:
        tmp = SAN_LIB + ".tmp"
        link = ["g++", "-shared", "-fPIC", *SAN_FLAGS, "-o", tmp, *host_objs, *hip_objs,
                "-L", ROCM_LIB, f"-Wl,-rpath,{ROCM_LIB}", "-lamdhip64"]
        _run(link)
        os.replace(tmp, SAN_LIB)
        return SAN_LIB
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *hip_objs, *host_objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
