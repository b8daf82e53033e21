"""Host-side checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments before touching the GPU.

Every call here returns from the library's argument checks (or is T == 0),
so no kernel is launched and no GPU is needed.
"""
import ctypes
import os
import re

import pytest

from mixture_value_projection_amd import binding
from mixture_value_projection_amd.build import LIBPATH

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mova.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, SCRATCH = 0, -1, -2, -3, -4, -5
FAKE = 1 << 20  # an aligned non-null address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIBPATH):
        pytest.fail(f"{LIBPATH} not built (run __graft_entry__.build())")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(mova_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mova_route", "mova_value_forward", "mova_workspace_bytes", "mova_status_str",
              "mova_version", "mova_timing_enable", "mova_timing_read",
              "mova_dense_value_proj", "mova_dense_workspace_bytes",
              "mova_value_forward_paged", "mova_value_from_routing", "mova_ffn_moe_forward",
              "mova_ffn_workspace_bytes", "mova_ffn_pack_gate_up"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in mova.h but not exported"


def test_status_strings(lib):
    for rc, tag in [(OK, "MOVA_OK"), (INVALID, "INVALID_ARG"), (UNSUPPORTED, "UNSUPPORTED"),
                    (WORKSPACE, "WORKSPACE"), (HIPERR, "HIP")]:
        assert tag in binding.status_str(rc)
    assert "unknown" in binding.status_str(12345)
    assert binding.version() >= 100


def test_workspace_bytes(lib):
    assert binding.workspace_bytes(0, 2560, 64, 4, 8, 128) == 0
    prev = 0
    for T in (1, 16, 64, 65, 4096, 32768):
        n = binding.workspace_bytes(T, 2560, 64, 4, 8, 128)
        assert n > prev and n % 256 == 0
        assert n >= T * 4 * 1024 * 2   # fp16 slot partials
        prev = n
    bad = ctypes.c_size_t(-1).value
    assert lib.mova_workspace_bytes(16, 2560, 65, 4, 8, 128) == bad     # E > 64
    assert lib.mova_workspace_bytes(16, 2560, 64, 9, 8, 128) == bad     # k > 8
    assert lib.mova_workspace_bytes(16, 2500, 64, 4, 8, 128) == bad     # d % 64
    assert lib.mova_workspace_bytes(16, 2560, 64, 4, 3, 20) == bad      # N % 64
    assert lib.mova_workspace_bytes(-1, 2560, 64, 4, 8, 128) == bad


@pytest.mark.parametrize("T", [100, 4096, 5000, 8192, 20000, 40000])
def test_workspace_bytes_independent_of_kernel_choice(T):
    """The workspace size depends on the shapes alone, not on which router or
    expert kernel a call will take (the switches that force them)."""
    want = binding.workspace_bytes(T, 2560, 64, 4, 8, 128)
    for name, val in [("router", "16"), ("router", "32s4"), ("router", "32s3"), ("router", "64"),
                      ("path", "grouped"), ("path", "decode"), ("gemm_tile", "128x128")]:
        with binding.overrides(**{name: val}):
            assert binding.workspace_bytes(T, 2560, 64, 4, 8, 128) == want, (name, val)


def fwd(lib, **kw):
    a = dict(x=FAKE, rw=FAKE, rb=None, ew=FAKE, T=16, d=256, E=8, k=2, scale=2.5, H=2, D=32,
             out=FAKE, idx=None, w=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.mova_value_forward(a["x"], a["rw"], a["rb"], a["ew"], a["T"], a["d"], a["E"], a["k"],
                                  a["scale"], a["H"], a["D"], a["out"], a["idx"], a["w"], a["ws"],
                                  a["wsb"], a["stream"])


def rte(lib, **kw):
    a = dict(x=FAKE, rw=FAKE, rb=None, T=16, d=256, E=8, k=2, scale=2.5, idx=FAKE, w=FAKE,
             stream=None)
    a.update(kw)
    return lib.mova_route(a["x"], a["rw"], a["rb"], a["T"], a["d"], a["E"], a["k"], a["scale"],
                          a["idx"], a["w"], a["stream"])


@pytest.mark.parametrize("kw,rc", [
    (dict(T=-1), INVALID), (dict(d=0), INVALID), (dict(E=0), INVALID), (dict(k=0), INVALID),
    (dict(E=65), UNSUPPORTED), (dict(k=9, E=16), UNSUPPORTED), (dict(k=3, E=2), UNSUPPORTED),
    (dict(d=100), UNSUPPORTED), (dict(H=3, D=20), UNSUPPORTED), (dict(H=0), INVALID),
    (dict(scale=float("nan")), UNSUPPORTED), (dict(scale=float("inf")), UNSUPPORTED),
    (dict(T=(1 << 24) + 1), UNSUPPORTED), (dict(H=129, D=128), UNSUPPORTED),
    (dict(x=None), INVALID), (dict(rw=None), INVALID), (dict(ew=None), INVALID),
    (dict(out=None), INVALID), (dict(x=FAKE + 2), INVALID), (dict(ew=FAKE + 8), INVALID),
    (dict(rb=FAKE + 4), INVALID), (dict(idx=FAKE + 4), INVALID), (dict(out=FAKE + 2), INVALID),
    (dict(ws=None), WORKSPACE), (dict(wsb=1024), WORKSPACE), (dict(ws=FAKE + 16), INVALID),
])
def test_value_forward_rejects(lib, kw, rc):
    assert fwd(lib, **kw) == rc


def test_value_forward_empty_is_noop(lib):
    # T == 0: nothing is enqueued, even with null buffers.
    assert fwd(lib, T=0, x=None, out=None, ws=None, wsb=0) == OK


@pytest.mark.parametrize("kw,rc", [
    (dict(T=-5), INVALID), (dict(E=70), UNSUPPORTED), (dict(k=5, E=4), UNSUPPORTED),
    (dict(d=96), UNSUPPORTED), (dict(scale=float("nan")), UNSUPPORTED),
    (dict(x=None), INVALID), (dict(idx=None), INVALID), (dict(w=None), INVALID),
    (dict(w=FAKE + 4), INVALID),
])
def test_route_rejects(lib, kw, rc):
    assert rte(lib, **kw) == rc


def test_route_empty_is_noop(lib):
    assert rte(lib, T=0, x=None, idx=None, w=None) == OK


def paged(lib, **kw):
    a = dict(x=FAKE, rw=FAKE, rb=None, ew=FAKE, T=16, d=256, E=8, k=2, scale=2.5, H=2, D=32,
             cache=FAKE, nb=4, bs=16, slot=FAKE + 8, out=None, idx=None, w=None, ws=FAKE,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.mova_value_forward_paged(a["x"], a["rw"], a["rb"], a["ew"], a["T"], a["d"], a["E"],
                                        a["k"], a["scale"], a["H"], a["D"], a["cache"], a["nb"],
                                        a["bs"], a["slot"], a["out"], a["idx"], a["w"], a["ws"],
                                        a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,rc", [
    (dict(T=-1), INVALID), (dict(E=65), UNSUPPORTED), (dict(d=100), UNSUPPORTED),
    (dict(scale=float("nan")), UNSUPPORTED), (dict(nb=-1), INVALID), (dict(bs=0), INVALID),
    (dict(nb=1 << 30, bs=1 << 12), UNSUPPORTED), (dict(cache=None), INVALID),
    (dict(slot=None), INVALID), (dict(cache=FAKE + 8), INVALID), (dict(slot=FAKE + 4), INVALID),
    (dict(out=FAKE + 2), INVALID), (dict(x=None), INVALID), (dict(ws=None), WORKSPACE),
    (dict(wsb=1024), WORKSPACE),
])
def test_paged_rejects(lib, kw, rc):
    assert paged(lib, **kw) == rc


def test_paged_empty_is_noop(lib):
    assert paged(lib, T=0, x=None, cache=None, slot=None, ws=None, wsb=0) == OK


def rebuild(lib, **kw):
    a = dict(x=FAKE, idx=FAKE, w=FAKE, ew=FAKE, T=16, d=256, E=8, k=2, H=2, D=32, out=FAKE,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.mova_value_from_routing(a["x"], a["idx"], a["w"], a["ew"], a["T"], a["d"], a["E"],
                                       a["k"], a["H"], a["D"], a["out"], a["ws"], a["wsb"],
                                       a["stream"])


@pytest.mark.parametrize("kw,rc", [
    (dict(T=-1), INVALID), (dict(E=65), UNSUPPORTED), (dict(k=9, E=16), UNSUPPORTED),
    (dict(d=100), UNSUPPORTED), (dict(idx=None), INVALID), (dict(w=None), INVALID),
    (dict(idx=FAKE + 4), INVALID), (dict(w=FAKE + 8), INVALID), (dict(x=None), INVALID),
    (dict(ew=None), INVALID), (dict(out=None), INVALID), (dict(ws=None), WORKSPACE),
    (dict(wsb=1024), WORKSPACE),
])
def test_rebuild_rejects(lib, kw, rc):
    assert rebuild(lib, **kw) == rc


def test_rebuild_empty_is_noop(lib):
    assert rebuild(lib, T=0, x=None, idx=None, w=None, out=None, ws=None, wsb=0) == OK


def test_ffn_workspace_bytes(lib):
    assert binding.ffn_workspace_bytes(0, 2560, 100, 8, 768, 768) == 0
    n = binding.ffn_workspace_bytes(64, 2560, 100, 8, 768, 768)
    assert n % 256 == 0 and n >= 64 * 8 * (768 * 2 + 2560 * 2) + 64 * 2560 * 2
    bad = ctypes.c_size_t(-1).value
    assert lib.mova_ffn_workspace_bytes(16, 2560, 129, 8, 768, 0) == bad   # E > 128
    assert lib.mova_ffn_workspace_bytes(16, 2560, 100, 9, 768, 0) == bad   # k > 8
    assert lib.mova_ffn_workspace_bytes(16, 2500, 100, 8, 768, 0) == bad   # d % 64
    assert lib.mova_ffn_workspace_bytes(16, 2560, 100, 8, 700, 0) == bad   # inter % 64
    assert lib.mova_ffn_workspace_bytes(16, 2560, 100, 8, 768, 100) == bad  # shared % 64


def ffn(lib, **kw):
    a = dict(x=FAKE, rw=FAKE, rb=None, gu=FAKE, dn=FAKE, E=100, k=8, I=128, sgu=None, sdn=None,
             Is=0, T=16, d=256, scale=2.5, out=FAKE, idx=None, w=None, ws=FAKE, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return lib.mova_ffn_moe_forward(a["x"], a["rw"], a["rb"], a["gu"], a["dn"], a["E"], a["k"],
                                    a["I"], a["sgu"], a["sdn"], a["Is"], a["T"], a["d"], a["scale"],
                                    a["out"], a["idx"], a["w"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,rc", [
    (dict(T=-1), INVALID), (dict(E=0), INVALID), (dict(E=129), UNSUPPORTED),
    (dict(k=9), UNSUPPORTED), (dict(k=5, E=4), UNSUPPORTED), (dict(d=100), UNSUPPORTED),
    (dict(I=96), UNSUPPORTED), (dict(I=0), INVALID), (dict(Is=64), INVALID),
    (dict(Is=64, sgu=FAKE, sdn=FAKE + 4), INVALID), (dict(scale=float("nan")), UNSUPPORTED),
    (dict(x=None), INVALID), (dict(gu=None), INVALID), (dict(dn=None), INVALID),
    (dict(out=None), INVALID), (dict(out=FAKE + 2), INVALID), (dict(ws=None), WORKSPACE),
    (dict(wsb=1024), WORKSPACE), (dict(ws=FAKE + 16), INVALID),
])
def test_ffn_rejects(lib, kw, rc):
    assert ffn(lib, **kw) == rc


def test_ffn_empty_is_noop(lib):
    assert ffn(lib, T=0, x=None, out=None, ws=None, wsb=0) == OK


@pytest.mark.parametrize("args,rc", [
    ((FAKE, FAKE, 0, 64, 128, FAKE), INVALID), ((FAKE, FAKE, 129, 64, 128, FAKE), UNSUPPORTED),
    ((FAKE, FAKE, 4, 60, 128, FAKE), UNSUPPORTED), ((None, FAKE, 4, 64, 128, FAKE), INVALID),
    ((FAKE, FAKE, 4, 64, 128, FAKE + 8), INVALID),
])
def test_ffn_pack_rejects(lib, args, rc):
    assert lib.mova_ffn_pack_gate_up(*args, None) == rc


def test_dense_workspace_bytes(lib):
    assert binding.dense_workspace_bytes(0, 2560, 8, 128) == 0
    for T in (1, 64, 256):
        n = binding.dense_workspace_bytes(T, 2560, 8, 128)
        assert n % 256 == 0 and n >= T * 1024 * 4   # at least one fp32 partial plane
    assert binding.dense_workspace_bytes(257, 2560, 8, 128) == 0   # tiled GEMM: no workspace
    bad = ctypes.c_size_t(-1).value
    assert lib.mova_dense_workspace_bytes(16, 2500, 8, 128) == bad    # d % 64
    assert lib.mova_dense_workspace_bytes(16, 2560, 3, 20) == bad     # N % 64
    assert lib.mova_dense_workspace_bytes(-1, 2560, 8, 128) == bad


def dense(lib, **kw):
    a = dict(x=FAKE, w=FAKE, T=16, d=256, H=2, D=32, out=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.mova_dense_value_proj(a["x"], a["w"], a["T"], a["d"], a["H"], a["D"], a["out"],
                                     a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,rc", [
    (dict(T=-1), INVALID), (dict(d=0), INVALID), (dict(H=0), INVALID), (dict(d=100), UNSUPPORTED),
    (dict(H=3, D=20), UNSUPPORTED), (dict(T=(1 << 24) + 1), UNSUPPORTED),
    (dict(H=129, D=128), UNSUPPORTED), (dict(x=None), INVALID), (dict(w=None), INVALID),
    (dict(out=None), INVALID), (dict(x=FAKE + 2), INVALID), (dict(w=FAKE + 8), INVALID),
    (dict(out=FAKE + 4), INVALID), (dict(ws=None), WORKSPACE), (dict(wsb=1024), WORKSPACE),
    (dict(ws=FAKE + 16), INVALID),
])
def test_dense_rejects(lib, kw, rc):
    assert dense(lib, **kw) == rc


def test_dense_empty_is_noop(lib):
    assert dense(lib, T=0, x=None, out=None, ws=None, wsb=0) == OK


def test_timing_read_without_records(lib):
    tot = (ctypes.c_double * 5)()
    cnt = (ctypes.c_int * 5)()
    assert lib.mova_timing_read(5, tot, cnt) == OK
    assert list(cnt) == [0, 0, 0, 0, 0]
    assert lib.mova_timing_read(-1, tot, cnt) == INVALID


def test_binding_rejects_wrong_dtype_on_cpu():
    import torch
    x = torch.zeros(4, 64, dtype=torch.float32)
    with pytest.raises(ValueError):
        binding.route(x, torch.zeros(8, 64, dtype=torch.bfloat16), None, 2)


def test_kernel_choice_overrides():
    """mova_debug_override: range checks, round trip, and the binding's
    context manager restoring the automatic choice; no environment variable
    is consulted by the library."""
    lib = binding.load_library()
    for key in range(7):
        assert lib.mova_debug_override_get(key) == 0
    assert lib.mova_debug_override_get(7) == -1
    assert lib.mova_debug_override_get(-1) == -1
    assert lib.mova_debug_override(7, 1) == -1
    assert lib.mova_debug_override(0, 3) == -1      # path takes 0..2
    assert lib.mova_debug_override(2, 8) == -1      # seven tile shapes
    assert lib.mova_debug_override(0, -1) == -1
    assert lib.mova_debug_override_get(0) == 0       # a rejected value changes nothing
    with binding.overrides(path="grouped", gemm_tile="352x256"):
        assert lib.mova_debug_override_get(0) == 2
        assert lib.mova_debug_override_get(2) == 7
        assert binding.get_override("gemm_tile") == "352x256"
    assert lib.mova_debug_override_get(0) == 0 and lib.mova_debug_override_get(2) == 0
    with open(binding.LIBPATH, "rb") as fh:
        assert b"getenv" not in fh.read(), "the library must not read the environment"


def test_noalloc_rejects_before_touching_the_gpu(lib):
    """mova_value_forward_noalloc: shape errors and calls larger than the
    static scratch are refused on the host (no device lookup, no launch)."""
    def call(T, d=2560, E=64, k=4, H=8, D=128):
        return lib.mova_value_forward_noalloc(FAKE, FAKE, None, FAKE, T, d, E, k, 2.5, H, D, FAKE,
                                              None, None, None)
    assert call(0) == OK
    assert call(16, E=65) == UNSUPPORTED
    assert call(16, d=2500) == UNSUPPORTED
    assert call(-1) == INVALID
    big = 1
    while binding.workspace_bytes(big, 2560, 64, 4, 8, 128) <= binding.NOALLOC_SCRATCH_BYTES:
        big *= 2
    assert call(big) == SCRATCH
    assert "scratch" in binding.status_str(SCRATCH)
    assert 4096 < big  # the prefill chunk (T = 4096) fits


def test_record_entry_points_reject_on_the_host(lib):
    """mova_value_forward_record / mova_value_from_record: shape and pointer
    errors are refused before anything is enqueued."""
    def fwd_rec(T=16, k=2, ids=FAKE, w=FAKE):
        return lib.mova_value_forward_record(FAKE, FAKE, None, FAKE, T, 256, 8, k, 2.5, 2, 32, FAKE,
                                             ids, w, FAKE, 1 << 30, None)

    def from_rec(T=16, k=2, ids=FAKE, w=FAKE, ws=FAKE):
        return lib.mova_value_from_record(FAKE, ids, w, FAKE, T, 256, 8, k, 2, 32, FAKE, ws, 1 << 30,
                                          None)
    assert fwd_rec(T=0) == OK and from_rec(T=0) == OK
    assert fwd_rec(k=6) == UNSUPPORTED and from_rec(k=6) == UNSUPPORTED
    assert fwd_rec(ids=None) == INVALID and from_rec(w=None) == INVALID
    assert fwd_rec(ids=FAKE + 2) == INVALID and from_rec(w=FAKE + 1) == INVALID
    assert from_rec(ws=None) == WORKSPACE


def test_c_example_is_built():
    """build() compiles the plain-C example caller of the C ABI next to the
    library (it runs in the GPU tests)."""
    from mixture_value_projection_amd import build
    assert os.path.exists(build.EXAMPLE)
    with open(build.EXAMPLE, "rb") as fh:
        assert fh.read(4) == b"\x7fELF"
