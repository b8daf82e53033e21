"""Checks on the gfx950 machine code of the kernels (CPU only: compiles to
assembly, runs nothing).

* No AGPR copy instructions (v_accvgpr_read / _write / _mov): every MFMA
  accumulator lives in an ordinary VGPR and is updated in place.  Copies of
  MFMA results between register files at loop heads produced stale values on
  the GPU.
* No scratch (private segment) use: nothing spills.
* Every file whose kernels contract issues MFMA (routers, grouped GEMM,
  decode, dense projection).
* The decode kernels' stream-once weight loads carry the non-temporal hint.
"""
import concurrent.futures
import re

import pytest

from mixture_value_projection_amd import build


@pytest.fixture(scope="module")
def asm():
    srcs = build.sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        return dict(zip([s.rsplit("/", 1)[-1] for s in srcs], ex.map(build.device_asm, srcs)))


def test_no_agpr_copies(asm):
    for name, text in asm.items():
        hits = re.findall(r"\bv_accvgpr_(?:read|write|mov)_b32\b", text)
        assert not hits, f"{name}: {len(hits)} AGPR copy instructions"


def test_no_scratch(asm):
    for name, text in asm.items():
        sizes = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)]
        assert all(v == 0 for v in sizes), f"{name}: private segment {sizes}"
    assert any(re.search(r"\.private_segment_fixed_size", t) for t in asm.values())


@pytest.mark.parametrize("name", ["router.hip", "grouped_gemm.hip", "decode.hip", "dense.hip"])
def test_contractions_use_mfma(asm, name):
    assert re.search(r"\bv_mfma_f32_16x16x32_bf16\b", asm[name])


def _bodies(text, prefix):
    """Assembly bodies of the kernels whose mangled names start with prefix."""
    lines = text.splitlines()
    out = []
    for i, line in enumerate(lines):
        if re.match(rf"^{prefix}\w*:", line):
            j = i
            while j < len(lines) and ".end_amdhsa_kernel" not in lines[j]:
                j += 1
            out.append((line.split(":")[0], lines[i:j]))
    return out


@pytest.mark.parametrize("name,prefix", [("router.hip", "_ZN4mova17router_lds_kernel"),
                                         ("decode.hip", "_ZN4mova19decode_token_kernel")])
def test_direct_load_rings_stay_in_flight(asm, name, prefix):
    """Fragment reads of the direct-load rings do not wait for every
    outstanding load (a vmcnt(0) right before a ds_read would drain the ring);
    the counter waits the kernels set themselves keep later chunks in flight."""
    bodies = _bodies(asm[name], prefix)
    assert bodies, prefix
    for kname, body in bodies:
        ins = [l.strip() for l in body if l.strip() and not l.strip().startswith((";", "."))]
        for a, b in zip(ins, ins[1:]):
            assert not (re.match(r"s_waitcnt vmcnt\(0\)$", a) and b.startswith("ds_read_b128")), kname
        partial = [l for l in ins if re.match(r"s_waitcnt vmcnt\(([1-9]\d*)\)", l)]
        if "Li2ELi4EEEv" not in kname:  # the 2-stage ring keeps nothing in flight at its wait
            assert partial, f"{kname}: no partial counter wait"


def test_decode_weight_stream_is_non_temporal(asm):
    """The weight-streaming decode kernel's row-segment loads and the
    token-major kernel's direct loads (its variant with the hint) are
    non-temporal; the token rows, read by many workgroups, are not."""
    text = asm["decode.hip"]
    stream = [b for n, b in _bodies(text, "_ZN4mova13decode_kernel")]
    assert stream and any(re.search(r"global_load_dwordx4 .* nt\b", l) for b in stream for l in b)
    tok = _bodies(text, "_ZN4mova19decode_token_kernel")
    hinted = [n for n, b in tok if any(re.search(r"global_load_lds_dwordx4 .* nt\b", l) for l in b)]
    plain = [n for n, b in tok if not any(re.search(r"global_load_lds_dwordx4 .* nt\b", l) for l in b)]
    assert hinted and plain, (len(hinted), len(plain))
