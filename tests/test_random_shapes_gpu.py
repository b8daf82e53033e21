"""Seeded random shapes through every entry point, against the CPU oracle.

Shapes are drawn from fixed seeds across the supported domain (token counts
from 1 to a few thousand, widths in steps of 64, 1 to 64 value experts or up
to 128 FFN experts, k up to 8), capped so that the float64 oracle finishes in
seconds.  Value path: both execution paths where they apply and a drawn tile
shape, checked against the oracle and against each other bit for bit.  Dense
projection: both kernels where they apply.  FFN: routing and outputs.
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
TILES = ["256x256", "128x256", "128x128", "128x128s3", "128x128s4", "128x128w4", "352x256"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu_only():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    binding.load_library()
    yield
    for v in ("path", "gemm_tile", "dense_path"):
        binding.set_override(v, None)


def value_shape(seed):
    rng = np.random.default_rng(1000 + seed)
    while True:
        T = int(np.exp(rng.uniform(0, np.log(3000))))
        d = 64 * int(rng.integers(1, 33))
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        D = int(rng.choice([32, 64, 128]))
        H = int(rng.integers(1, 17))
        if (H * D) % 64 or H * D > 2048:
            continue
        if T * k * d * H * D <= 1.5e9:
            return T, d, E, k, H, D, TILES[int(rng.integers(len(TILES)))]


@pytest.mark.parametrize("seed", range(16))
def test_value_forward_random_shape(seed):
    T, d, E, k, H, D, tile = value_shape(seed)
    say(f"value seed={seed}: T={T} d={d} E={E} k={k} H={H} D={D} tile={tile}")
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=H, head_dim=D)
    g = P.to_gpu_inputs(inputs.make_layer(shape, 50 + seed, torch.bfloat16, "uniform"))
    outs = {}
    for path in ["grouped"] + (["decode"] if T <= 256 else []):
        binding.set_override("path", path)
        binding.set_override("gemm_tile", tile)
        idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        w = torch.empty(T, k, dtype=torch.float32, device=DEV)
        out = binding.value_forward(g["x"], g["router_w"], g["router_b"], g["expert_w"], k, 2.5,
                                    H, D, topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        binding.set_override("path", None)
        binding.set_override("gemm_tile", None)
        st = P.full_check(g, k, 2.5, H, D, out, idx, w, what=f"seed {seed} {path}")
        say(f"  {path}: {st}")
        outs[path] = out
    if len(outs) == 2:
        assert torch.equal(outs["grouped"], outs["decode"])


@pytest.mark.parametrize("seed", range(8))
def test_dense_random_shape(seed):
    rng = np.random.default_rng(2000 + seed)
    T = int(np.exp(rng.uniform(0, np.log(5000))))
    d = 64 * int(rng.integers(1, 41))
    N = 64 * int(rng.integers(1, 33))
    say(f"dense seed={seed}: T={T} d={d} N={N}")
    x = inputs.make_tokens(T, d, 60 + seed).to(DEV)
    w = inputs.make_dense_vproj(inputs.LayerShape(T=T, d=d, E=1, k=1, n_kv_heads=N // 64,
                                                  head_dim=64), 60 + seed).to(DEV)
    ref = oracle.dense_value_proj(x.cpu().double().numpy(), w.cpu().double().numpy())
    for path in ["tiled"] + (["skinny"] if T <= 256 else []):
        binding.set_override("dense_path", path)
        out = binding.dense_value_proj(x, w, N // 64, 64).reshape(T, N)
        torch.cuda.synchronize()
        binding.set_override("dense_path", None)
        say(f"  {path}: {P.check_dense_output(out, ref, what=f'dense seed {seed} {path}')}")


@pytest.mark.parametrize("seed", range(6))
def test_ffn_random_shape(seed):
    rng = np.random.default_rng(3000 + seed)
    T = int(np.exp(rng.uniform(0, np.log(600))))
    d = 64 * int(rng.integers(1, 9))
    E = int(rng.integers(1, 129))
    k = int(rng.integers(1, min(E, 8) + 1))
    inter = 64 * int(rng.integers(1, 5))
    inter_s = 64 * int(rng.integers(0, 4))
    sh = inputs.FfnShape(T=T, d=d, E=E, k=k, inter=inter, inter_shared=inter_s, scale=1.0)
    say(f"ffn seed={seed}: T={T} d={d} E={E} k={k} inter={inter} shared={inter_s}")
    L = inputs.make_ffn_layer(sh, 70 + seed)
    g = {kk: v.to(DEV).contiguous() for kk, v in L.items()}
    gu = binding.ffn_pack_gate_up(g["gate_w"], g["up_w"])
    sgu = binding.ffn_pack_gate_up(g["shared_gate_w"], g["shared_up_w"]) if inter_s else None
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    out = binding.ffn_moe_forward(g["x"], g["router_w"], g["router_b"], gu, g["down_w"], k, 1.0,
                                  sgu, g.get("shared_down_w"), topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    o = {kk: v.double().numpy() for kk, v in L.items()}
    rc = P.check_routing(idx, w, oracle.route(o["x"], o["router_w"], o["router_b"], k, 1.0), 1.0)
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            e = int(rc.effective_idx[t, j])
            ref[t] += rc.effective_w[t, j] * oracle.swiglu_expert(
                o["x"][t:t + 1], o["gate_w"][e], o["up_w"][e], o["down_w"][e])[0]
    if inter_s:
        ref += oracle.swiglu_expert(o["x"], o["shared_gate_w"], o["shared_up_w"], o["shared_down_w"])
    say(f"  {P.check_output(out, ref, what=f'ffn seed {seed}')}")
