"""Checks on the gfx950 machine code of the kernels (CPU only: compiles to
assembly, runs nothing).

* No AGPR copy instructions (v_accvgpr_read / _write / _mov): every MFMA
  accumulator lives in an ordinary VGPR and is updated in place.  Copies of
  MFMA results between register files at loop heads produced stale values on
  the GPU.
* No scratch (private segment) use: nothing spills.
* Every file whose kernels contract issues MFMA (router, grouped GEMM,
  decode, dense projection, FFN router).
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


@pytest.mark.parametrize("name", ["router.hip", "grouped_gemm.hip", "decode.hip", "dense.hip",
                                  "ffn.hip"])
def test_contractions_use_mfma(asm, name):
    assert re.search(r"\bv_mfma_f32_16x16x32_bf16\b", asm[name])
