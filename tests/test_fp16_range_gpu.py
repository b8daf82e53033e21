"""The fp16 slot partial's range, at its bound (exact values, no rounding).

One expert (E = k = 1, so the weight is the scale, 2.5), x = e_0 and an expert
weight column of a power of two: z = c exactly, SiLU(z) = z in fp32 for
z >= 2^10, and the slot value w * SiLU(z) = 2.5 c is exact in fp16 and bf16.
* c = 2^14: 40960 < 65504 fits fp16; the output equals the oracle exactly;
* c = 2^15: 81920 > 65504 becomes +inf (the documented domain limit), while
  the oracle's value is finite;
* k = 2 tied experts (weights 1.25 each) at c = 2^15: each slot is 40960 and
  fits, their sum 81920 exceeds the fp16 bound but is kept in fp32 and fits
  bf16 exactly; the output equals the oracle.
Both expert paths (decode kernel, grouped GEMM) are checked.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_value_projection_amd import binding

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu_only():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    binding.load_library()


def run(E, k, c, path, T=16, d=64, N=64):
    x = torch.zeros(T, d)
    x[:, 0] = 1.0
    W = torch.zeros(E, N, d)
    W[:, :, 0] = c
    Wr = torch.zeros(E, d)  # all scores tie at sigmoid(0): experts 0..k-1, weights scale / k
    g = {"x": x.to(torch.bfloat16).to(DEV), "router_w": Wr.to(torch.bfloat16).to(DEV),
         "expert_w": W.to(torch.bfloat16).to(DEV)}
    with binding.overrides(path=path):
        out = binding.value_forward(g["x"], g["router_w"], None, g["expert_w"], k, 2.5, 1, N)
    torch.cuda.synchronize()
    ref, _ = oracle.value_forward(x.double().numpy(), Wr.double().numpy(), None,
                                  W.double().numpy(), k, 2.5, 1, N)
    return out.float().cpu().numpy().reshape(T, N), ref.reshape(T, N)


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_slot_value_below_the_fp16_bound(path):
    out, ref = run(1, 1, 2.0 ** 14, path)
    assert (ref == 40960.0).all()
    np.testing.assert_array_equal(out, ref)


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_slot_value_beyond_the_fp16_bound_is_inf(path):
    out, ref = run(1, 1, 2.0 ** 15, path)
    assert np.isfinite(ref).all() and (ref == 81920.0).all()
    assert np.isposinf(out).all()


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_sum_of_slots_may_exceed_the_fp16_bound(path):
    out, ref = run(2, 2, 2.0 ** 15, path)
    assert (ref == 81920.0).all()  # two slots of 1.25 * 2^15
    np.testing.assert_array_equal(out, ref)
