"""AddressSanitizer run of the library's host code (CPU only, no GPU calls).

The C-ABI source (argument checks, workspace layouts, path choice, status
strings, overrides) is compiled with AddressSanitizer on its host side only
and linked with the other, uninstrumented objects into a separate library;
``tests/asan_host_driver.c``, built with the same sanitizer, calls every
entry point with arguments the host checks reject and exits 0 when each
returned the expected status.  Any heap, stack or global overflow in those
paths aborts the driver with an ASan report.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

from mixture_value_projection_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ROCM_LIB = "/opt/rocm/lib"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.fixture(scope="module")
def asan_driver():
    if not (os.path.exists(build.HIPCC) and os.path.exists(CLANG) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm compilers not found")
    os.makedirs(build.BUILDDIR, exist_ok=True)
    out = tempfile.mkdtemp(prefix="asan-", dir=build.BUILDDIR)  # one per test process
    srcs = build.sources()
    others = [os.path.join(build.BUILDDIR, os.path.basename(s) + ".o") for s in srcs
              if not s.endswith("mova_api.hip")]
    if not all(os.path.exists(o) for o in others):
        build.build_library(verbose=False)
    api = os.path.join(build.CSRC, "mova_api.hip")
    api_obj = os.path.join(out, "mova_api.asan.o")
    # The sanitizer applies to the host side of the compile only.
    _run([build.HIPCC, *build.COMMON, *build.DEVICE_FLAGS,
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
          "-c", api, "-o", api_obj])
    lib = os.path.join(out, "libmova_asan.so")
    _run([CLANGXX, "-shared", "-fPIC", "-fsanitize=address", "-o", lib, api_obj, *others,
          f"-L{ROCM_LIB}", "-lamdhip64"])
    exe = os.path.join(out, "asan_host_driver")
    _run([CLANG, "-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-I",
          os.path.join(build.ROOT, "include"), os.path.join(HERE, "asan_host_driver.c"), "-o", exe,
          f"-L{out}", "-lmova_asan", f"-Wl,-rpath,{out}", f"-Wl,-rpath,{ROCM_LIB}"])
    yield exe
    shutil.rmtree(out, ignore_errors=True)


def test_host_paths_under_asan(asan_driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([asan_driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"driver failed:\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    assert "asan host driver: ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr


def test_api_object_is_instrumented(asan_driver):
    obj = os.path.join(os.path.dirname(asan_driver), "mova_api.asan.o")
    syms = subprocess.run(["nm", "-u", obj], capture_output=True, text=True).stdout
    assert "__asan_init" in syms
