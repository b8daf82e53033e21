"""Values rebuilt from stored routing (mova_value_from_routing) vs the oracle.

* Fed the routing mova_value_forward reported, the rebuild returns the same
  bits as the forward call, on both execution paths.
* Arbitrary stored routing -- repeated ids, unused slots marked by ids
  outside [0, E), zero and fp16-rounded weights -- against
  ``oracle.rebuild_values`` under the output parity rules, with the decode
  and grouped paths agreeing bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from mixture_value_projection_amd import binding, inputs
import paritylib as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu_only():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    binding.load_library()
    yield
    binding.set_override("path", None)


def with_path(path, fn):
    binding.set_override("path", path)
    try:
        r = fn()
        torch.cuda.synchronize()
        return r
    finally:
        binding.set_override("path", None)


SHAPES = [
    # T, d, E, k, H, D
    (8, 2560, 64, 4, 8, 128),      # token-major decode kernel (T * k <= 48)
    (5, 256, 8, 3, 2, 32),
    (37, 256, 8, 2, 2, 32),
    (64, 2560, 64, 4, 8, 128),
    (300, 512, 16, 4, 2, 64),
    (4096, 2560, 64, 4, 8, 128),
]


@pytest.mark.parametrize("T,d,E,k,H,D", SHAPES)
def test_rebuild_from_own_routing_is_bitwise(T, d, E, k, H, D):
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=H, head_dim=D)
    g = P.to_gpu_inputs(inputs.make_layer(shape, T + 5, torch.bfloat16, "uniform"))
    paths = ["grouped"] + (["decode"] if T <= 256 else [])
    for path in paths:
        say(f"rebuild own routing T={T} d={d} E={E} k={k} {path}")
        idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        w = torch.empty(T, k, dtype=torch.float32, device=DEV)
        fwd = with_path(path, lambda: binding.value_forward(
            g["x"], g["router_w"], g["router_b"], g["expert_w"], k, 2.5, H, D,
            topk_idx=idx, topk_w=w))
        reb = with_path(path, lambda: binding.value_from_routing(g["x"], idx, w, g["expert_w"], H, D))
        assert torch.equal(reb, fwd)


def stored_routing(T, E, k, seed):
    """Ids with repeats and unused slots (-1, -7, E, 1000).  Weights as the
    router makes them -- positive, summing to the scale 2.5 per token, so the
    outputs stay in the range the parity rules are set for -- with some
    zeroed, and rounded to fp16 as a compact cache would keep them."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    bad = rng.random((T, k)) < 0.15
    idx[bad] = rng.choice(np.array([-1, -7, E, 1000], dtype=np.int32), size=int(bad.sum()))
    w = rng.uniform(0.05, 1.0, size=(T, k))
    w = 2.5 * w / w.sum(axis=1, keepdims=True)
    w[rng.random((T, k)) < 0.05] = 0.0
    w = w.astype(np.float16).astype(np.float32)
    return idx, w


@pytest.mark.parametrize("T,d,E,k,H,D", SHAPES)
def test_rebuild_stored_routing_matches_oracle(T, d, E, k, H, D):
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=H, head_dim=D)
    g = P.to_gpu_inputs(inputs.make_layer(shape, T + 9, torch.bfloat16, "uniform"))
    idx, w = stored_routing(T, E, k, seed=T)
    gi = torch.as_tensor(idx, device=DEV)
    gw = torch.as_tensor(w, device=DEV)
    o = P.oracle_inputs(g)
    rows = np.arange(T) if T <= 1024 else np.unique(np.r_[np.random.default_rng(1).choice(T, 1500, replace=False), 0, T - 1])
    ref = oracle.rebuild_values(o["x"][rows], o["expert_w"], idx[rows], w[rows])
    outs = {}
    for path in ["grouped"] + (["decode"] if T <= 256 else []):
        say(f"rebuild stored routing T={T} d={d} E={E} k={k} {path}")
        out = with_path(path, lambda: binding.value_from_routing(g["x"], gi, gw, g["expert_w"], H, D))
        sel = out.reshape(T, -1)[torch.as_tensor(rows, device=DEV)]
        say(f"  {P.check_output(sel, ref, what=f'rebuild/{path}')}")
        outs[path] = out
    if len(outs) == 2:
        assert torch.equal(outs["grouped"], outs["decode"])


@pytest.mark.parametrize("T", [90, 10])
def test_rebuild_all_slots_unused_is_zero(T):
    d, E, k, H, D = 256, 8, 3, 2, 64
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=H, head_dim=D)
    g = P.to_gpu_inputs(inputs.make_layer(shape, 3, torch.bfloat16, "uniform"))
    gi = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
    gi[::2, 1] = E
    gw = torch.ones(T, k, dtype=torch.float32, device=DEV)
    for path in ("grouped", "decode"):
        out = with_path(path, lambda: binding.value_from_routing(g["x"], gi, gw, g["expert_w"], H, D))
        assert torch.count_nonzero(out) == 0


BOUNDARY_LOADS = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 95, 96, 97, 175, 176, 177, 191, 192,
                  193, 271, 272, 273, 351, 352, 353]
TILE_SHAPES = ["352x256", "256x256", "128x256", "128x128", "128x128s4", "128x128w4"]


def test_tile_row_boundaries_every_tile():
    """Experts whose row counts sit on either side of every tile's row-block,
    half-tile and tile boundaries (16-row MFMA blocks; 32 / 64 / 96 / 176 / 192
    / 272 rows, where a wave's valid rows stop fitting the first half of its
    blocks; 128 / 256 / 352-row tiles), rebuilt from stored routing with the
    tokens shuffled so that the gathered rows are scattered: every tile shape
    against the oracle, and all with the same bits."""
    E, k, d, H, D = len(BOUNDARY_LOADS), 1, 256, 5, 64
    T = sum(BOUNDARY_LOADS)
    rng = np.random.default_rng(77)
    idx = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), BOUNDARY_LOADS)).reshape(T, k)
    w = np.ones((T, k), dtype=np.float32)  # keeps |out| inside the parity rules' range
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=H, head_dim=D)
    g = P.to_gpu_inputs(inputs.make_layer(shape, 91, torch.bfloat16, "uniform"))
    gi = torch.as_tensor(idx, device=DEV)
    gw = torch.as_tensor(w, device=DEV)
    o = P.oracle_inputs(g)
    ref = oracle.rebuild_values(o["x"], o["expert_w"], idx, w)
    outs = {}
    try:
        for tile in TILE_SHAPES:
            binding.set_override("gemm_tile", tile)
            say(f"row boundaries: tile {tile}, T={T} E={E} d={d} N={H * D}")
            out = with_path("grouped", lambda: binding.value_from_routing(g["x"], gi, gw,
                                                                          g["expert_w"], H, D))
            say(f"  {P.check_output(out.reshape(T, -1), ref, what=f'tile {tile}')}")
            outs[tile] = out
    finally:
        binding.set_override("gemm_tile", None)
    for tile, out in outs.items():
        assert torch.equal(out, outs[TILE_SHAPES[0]]), f"{tile} differs from {TILE_SHAPES[0]}"
