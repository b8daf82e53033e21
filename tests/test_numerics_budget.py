"""Error budget of the HIP path's intermediate precisions, checked on the CPU
with the float64 oracle (no GPU).

The expert kernels keep each (token, slot) result w * SiLU(z) as fp16 before
the k-way sum (fp32, slot order) and the final bf16 rounding.  Simulating
exactly that rounding chain on oracle values must stay inside the output
tolerances the GPU parity tests use, with room to spare for the fp32
accumulation differences of the real kernels."""
import numpy as np
import torch

import oracle
from mixture_value_projection_amd import inputs
from paritylib import MAX_ABS, REL_L2


def _slot_outputs(name, T=None):
    w = inputs.WORKLOADS[name]
    L = inputs.make_workload(name, T=T) if T else inputs.make_workload(name)
    x = L["x"].double().numpy()
    r = oracle.route(x, L["router_w"].double().numpy(), L["router_b"].double().numpy(),
                     w.shape.k, w.shape.scale)
    y = np.zeros((x.shape[0], w.shape.k, w.shape.N))
    for e in np.unique(r.idx):
        rows, slots = np.nonzero(r.idx == e)
        z = x[rows] @ L["expert_w"][e].double().numpy().T
        y[rows, slots] = r.w[rows, slots, None] * oracle.silu(z)
    return y


def _chain(y, partial_dtype):
    s = y[:, 0].astype(np.float32).astype(partial_dtype).astype(np.float32)
    for j in range(1, y.shape[1]):
        s = (s + y[:, j].astype(np.float32).astype(partial_dtype).astype(np.float32)).astype(np.float32)
    return torch.from_numpy(s).to(torch.bfloat16).double().numpy()


def test_fp16_slot_partials_within_tolerance():
    for name, T in (("decode", None), ("prefill", 1024)):
        y = _slot_outputs(name, T)
        exact = y.sum(1)
        out = _chain(y, np.float16)
        err = np.abs(out - exact)
        rel = np.linalg.norm(out - exact) / np.linalg.norm(exact)
        assert err.max() <= 0.9 * MAX_ABS, (name, err.max())
        assert rel <= 0.5 * REL_L2, (name, rel)
        # The fp16 step adds little next to the final bf16 rounding.
        ref = _chain(y, np.float32)
        assert np.abs(out - ref).max() <= 4 * 2.0 ** -11 * np.abs(y).max() + 2 * 2.0 ** -8 * np.abs(exact).max()
