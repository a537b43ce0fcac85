"""Build the HIP library libmt.so in-tree for gfx950.

Every .hip and host .cpp file under csrc/ is compiled to an object in
_build/ (hipcc for HIP sources and for host files that use the HIP runtime
headers, g++ for the AVX-512 host Adam, which must not be contracted into
FMAs) and linked into host_memory_layer_amd/libmt.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmt.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result", "-Wno-unused-value"]
GXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-I" + INCLUDE, "-I" + CSRC]

HIP_SOURCES = ["gemm.hip", "attention.hip", "elementwise.hip", "engine.hip", "noalloc.hip"]
# The attention kernels feed MFMA results to vector ALU work (softmax) every
# tile: MFMAs that write the general register file avoid copies through the
# accumulation registers.
FILE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HIPCC_HOST_SOURCES = ["store.cpp", "api.cpp", "kernel_api.cpp", "dma.cpp", "linkprobe.cpp"]
GXX_SOURCES = ["adam.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        cmds.append([HIPCC] + HIP_FLAGS + FILE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIPCC_HOST_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        cmds.append([HIPCC] + HIP_FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in GXX_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        cmds.append(["g++"] + GXX_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    jobs = jobs or min(8, len(cmds))
    with ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + ["-L/opt/rocm/lib", "-lhsa-runtime64", "-lpthread"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
