"""Build libpagedkv.so in-tree for gfx950.

    python -m paged_kv_cache_377_amd.build          # build (always recompiles)

The host allocator (csrc/alloc.c) is compiled with gcc as C11; each HIP source
is compiled with hipcc for gfx950 with packed FP32 instructions disabled; the
objects are linked into ``paged_kv_cache_377_amd/libpagedkv.so``.
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
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")

HIP_SOURCES = ["cache_ops.hip", "decode.hip", "prefill.hip", "measure.hip"]
C_SOURCES = ["alloc.c"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CC = os.environ.get("CC", shutil.which("gcc") or "cc")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed FP32 VALU ops stay off; hipcc -O3 would otherwise form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs: the decode rescales them with
    # VALU ops, which would otherwise copy them out of and back into AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]
C_FLAGS = ["-std=c11", "-O2", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
           "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass of hipcc warns that it does not know the packed-fp32 feature
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for src in C_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs.append([CC, *C_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HIP_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for cmd, err in zip(jobs, ex.map(_run, jobs)):
            if verbose or err.strip():
                print(" ".join(cmd), file=sys.stderr)
                if err.strip():
                    print(err, file=sys.stderr)
    objs = [os.path.join(OBJ, s + ".o") for s in C_SOURCES + HIP_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
