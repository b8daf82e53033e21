"""Find the Zipf bias scale of the skewed-routing workload.

The workload asks for a router bias that makes per-expert load follow a
Zipf(1.1) law with the hottest experts drawing about 10x the mean number of
tokens.  An exact Zipf(1.1) load over 64 experts is impossible at top-4 (the
rank-1 share would exceed every token), so the bias is
b_e = beta * (ln p_pi(e) - mean ln p) and beta is chosen by bisection so that
max load / mean load = 10 on the workload's own seeded tokens (T = 32768).

Routing uses only the CPU oracle.  Prints the resulting beta (rounded to a
float that is exact in binary), which is stored as ``ZIPF_BETA`` in
``mixture_value_projection_amd/inputs.py`` and checked by
``tests/test_oracle_pins.py::test_skewed_workload_load_ratio``.

Run from the repository root:  python tests/golden/calibrate_zipf_bias.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))

from mixture_value_projection_amd import inputs  # noqa: E402
from oracle import route  # noqa: E402


def load_ratio(beta: float, x, shape) -> float:
    r = inputs.make_router(shape, 0, bias="zipf", zipf_beta=beta)
    rt = route(x, r["router_w"], r["router_b"], shape.k, shape.scale)
    counts = np.bincount(rt.idx.ravel(), minlength=shape.E)
    return counts.max() / counts.mean()


def main() -> None:
    w = inputs.WORKLOADS["skewed"]
    shape = w.shape
    x = inputs.make_tokens(shape.T, shape.d, w.seed)
    lo, hi = 0.0, 1.0
    for _ in range(20):
        mid = 0.5 * (lo + hi)
        if load_ratio(mid, x, shape) < 10.0:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi) * 1024) / 1024
    print(f"beta = {beta!r}  max/mean = {load_ratio(beta, x, shape):.3f}")


if __name__ == "__main__":
    main()
