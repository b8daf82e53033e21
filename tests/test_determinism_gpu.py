"""Bitwise reproducibility of the HIP path: repeated calls, other streams, and
any split of the tokens into calls give identical bits (the design has no
float atomics, and both router block shapes and both expert paths add the
same products in the same order)."""
import pytest
import torch

from mixture_value_projection_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_layer(T, seed=0):
    shape = inputs.LayerShape(T=T, d=2560, E=64, k=4, n_kv_heads=8, head_dim=128)
    t = inputs.make_layer(shape, seed, torch.bfloat16, "uniform")
    return {k: v.to(DEV) for k, v in t.items()}


def fwd(g, x=None, out=None):
    return binding.value_forward(g["x"] if x is None else x, g["router_w"], g["router_b"],
                                 g["expert_w"], 4, 2.5, 8, 128, out=out)


def test_repeat_and_stream_bitwise():
    g = gpu_layer(4096)
    a = fwd(g).clone()
    b = fwd(g).clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = fwd(g).clone()
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


# The router's workgroup shape depends on the call's token count (16, 32 or 64
# tokens per workgroup); (8192, 4096) and (17000, 4250) cross those shapes.
@pytest.mark.parametrize("T,chunk", [(4096, 512), (256, 64), (130, 13), (8192, 4096), (17000, 4250)])
def test_chunking_bitwise(T, chunk):
    g = gpu_layer(T, seed=T)
    whole = fwd(g).clone()
    parts = torch.empty_like(whole)
    for c0 in range(0, T, chunk):
        fwd(g, x=g["x"][c0:c0 + chunk], out=parts[c0:c0 + chunk])
    torch.cuda.synchronize()
    assert torch.equal(whole, parts)


@pytest.mark.parametrize("T,chunk", [(20000, 3000), (40000, 12000)])
def test_route_chunking_bitwise(T, chunk):
    g = gpu_layer(T, seed=T)
    idx, w = binding.route(g["x"], g["router_w"], g["router_b"], 4, 2.5)
    for c0 in range(0, T, chunk):
        i2, w2 = binding.route(g["x"][c0:c0 + chunk], g["router_w"], g["router_b"], 4, 2.5)
        assert torch.equal(idx[c0:c0 + chunk], i2) and torch.equal(w[c0:c0 + chunk], w2)


@pytest.mark.parametrize("T", [64, 1000])
def test_graph_replay_matches_eager(T):
    """A captured call replays to the eager result every time, with eager work
    and synchronisations between the replays (decode path at T=64, grouped
    path at T=1000)."""
    g = gpu_layer(T, seed=3)
    ws = torch.empty(binding.workspace_bytes(T, 2560, 64, 4, 8, 128), dtype=torch.uint8, device=DEV)
    eager = fwd_ws(g, ws).clone()
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd_ws(g, ws, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd_ws(g, ws, out)
    for rep in range(4):
        out.zero_()
        other = fwd(gpu_layer(80, seed=rep))   # unrelated eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"
        del other


def fwd_ws(g, ws, out=None):
    return binding.value_forward(g["x"], g["router_w"], g["router_b"], g["expert_w"], 4, 2.5, 8, 128,
                                 out=out, workspace=ws)
