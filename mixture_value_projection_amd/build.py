"""Build ``libmova.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m mixture_value_projection_amd.build`` or ``build_library()``.
Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in parallel),
then linked into ``mixture_value_projection_amd/lib/libmova.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIBPATH = os.path.join(LIBDIR, "libmova.so")
BUILDDIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Device code generation flags:
# * packed-fp32 instructions are disabled for every device compile;
# * MFMA accumulators are kept in (and updated in place in) ordinary VGPRs.
#   With the default AGPR heuristics, loops whose accumulators are updated
#   under data-dependent branches were compiled into AGPR<->VGPR copies and
#   rotations at the loop head, and the copied values were read before the
#   MFMA that produced them had finished (wrong, run-to-run varying results).
#   tests/test_codegen.py checks that no AGPR copy instruction is emitted.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILDDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def device_asm(src: str) -> str:
    """gfx950 assembly of one source file, compiled with the library's flags."""
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "--cuda-device-only", "-S", src, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    return r.stdout


def build_library(verbose: bool = True) -> str:
    """Compile every kernel source and link libmova.so; returns its path."""
    os.makedirs(BUILDDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIBPATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIBPATH)
    build_example()
    if verbose:
        print(f"built {LIBPATH}")
    return LIBPATH


EXAMPLE_SRC = os.path.join(ROOT, "examples", "value_forward.c")
EXAMPLE = os.path.join(LIBDIR, "mova_value_forward_example")
CLANG = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")


def build_example() -> str:
    """Compile examples/value_forward.c (a plain C caller of the C ABI) next to
    the library, which it finds through its rpath."""
    clang = CLANG if os.path.exists(CLANG) else "/opt/rocm/llvm/bin/clang"
    rocm = os.path.realpath(os.path.join(os.path.dirname(os.path.realpath(HIPCC)), ".."))
    cmd = [clang, "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), EXAMPLE_SRC, "-o", EXAMPLE, f"-L{LIBDIR}", "-lmova",
           f"-L{os.path.join(rocm, 'lib')}", "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"example build failed:\n{r.stdout}\n{r.stderr}")
    return EXAMPLE


if __name__ == "__main__":
    build_library()
