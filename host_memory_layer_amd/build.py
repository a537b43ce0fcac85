"""Build the HIP library libmt.so in-tree for gfx950.

Every .hip and host .cpp file under csrc/ is compiled to an object in
_build/ (hipcc for HIP sources and for host files that use the HIP runtime
headers, g++ for the AVX-512 host Adam, which must not be contracted into
FMAs) and linked into host_memory_layer_amd/libmt.so.

A second variant, libmt_asan.so (objects in _build_asan/), instruments the
host code of every source with AddressSanitizer (device code is built as
usual; the Adam file goes through clang++, whose sanitizer runtime the
other objects use).  Its __asan_* references are resolved at load time by
the clang runtime preloaded into the process (the host-code tests run it
that way on the CPU).
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

CLANGXX = "/opt/rocm/llvm/bin/clang++"
ASAN_OUT_DIR = os.path.join(PKG, "_build_asan")
ASAN_LIB = os.path.join(PKG, "libmt_asan.so")
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime (to preload)."""
    r = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    return path


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def _commands(asan: bool):
    out_dir = ASAN_OUT_DIR if asan else OUT_DIR
    os.makedirs(out_dir, exist_ok=True)
    extra = ASAN_HOST if asan else []
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmds.append([HIPCC] + HIP_FLAGS + extra + FILE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIPCC_HOST_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmds.append([HIPCC] + HIP_FLAGS + extra + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in GXX_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmds.append(([CLANGXX] if asan else ["g++"]) + GXX_FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    return cmds, objs


def _link(objs, lib):
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + ["-L/opt/rocm/lib", "-lhsa-runtime64", "-lpthread"])
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int | None = None, asan: bool = True) -> str:
    """Builds libmt.so and, with asan, libmt_asan.so (compiled together)."""
    cmds, objs = _commands(False)
    acmds, aobjs = _commands(True) if asan else ([], [])
    jobs = jobs or 8
    with ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, cmds + acmds):
            if verbose and out.strip():
                print(out)
    _link(objs, LIB)
    if asan:
        _link(aobjs, ASAN_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
