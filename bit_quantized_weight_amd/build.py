"""Build libqgemv.so in-tree for gfx950 with hipcc.

    python -m bit_quantized_weight_amd.build

Compiles the HIP kernels (csrc/*.hip) for gfx950 and the host packer
(csrc/pack.cpp, no FMA contraction so packed bytes are reproducible), then
links them into bit_quantized_weight_amd/libqgemv.so. The library links the
HIP runtime by soname (libamdhip64.so.7); the Python binding imports torch
first so that torch's copy of the runtime is the one the library uses.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqgemv.so")

ARCH = "gfx950"
HIP_SOURCES = ["gemv.hip", "moe.hip", "mx.hip"]
# moe.hip: atomics (the routing bitmap's LDS ORs, the sticky error word) stay
# single-lane as written. Both: the kernels' leading scalar arguments are
# preloaded into SGPRs at wave launch (gfx950 kernel argument preloading), so
# a wave issues its first loads without reading the argument block.
EXTRA_FLAGS = {"moe.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None", "-mllvm",
                           "-amdgpu-kernarg-preload-count=16"],
               "gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"]}
HOST_SOURCES = ["pack.cpp"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libqgemv")


def _rocm_include() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))


# Host-sanitizer build: the same sources with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host side only (every -fsanitize goes to
# the host compilation through -Xarch_host; device code is built as usual),
# linked against the shared sanitizer runtime, which the loading process must
# preload. It serves the host-code tests (packing, argument validation).
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libqgemv_san.so")
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the HIP toolchain's
    compiler (to preload into a process that loads SAN_LIB)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build(verbose: bool = False, sanitize: bool = False) -> str:
    hipcc = _hipcc()
    out_dir = SAN_DIR if sanitize else BUILD
    lib = SAN_LIB if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    common = ["-O2" if sanitize else "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC]
    if sanitize:
        common += SAN_HOST_FLAGS
    cmds = []
    for src in HIP_SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(out_dir, src + ".o")
        cmds.append([hipcc, "--offload-arch=" + ARCH, *common,
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *EXTRA_FLAGS.get(src, []),
                     "-c", path, "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmds.append([hipcc, "-x", "c++", *common, "-I" + _rocm_include(), "-D__HIP_PLATFORM_AMD__=1",
                     "-ffp-contract=off", "-fno-fast-math",
                     "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # the translation units are independent: compile them side by side
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)) for c in cmds]
    failed = None
    for c, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0 and failed is None:
            sys.stderr.write(out)
            failed = c
    if failed:
        raise RuntimeError("build step failed: " + " ".join(failed))
    tmp = lib + ".tmp"
    link = ["-shared-libsan", *SAN_HOST_FLAGS] if sanitize else []
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *link, "-o", tmp, *objs, "-lpthread"])
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
