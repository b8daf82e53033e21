"""mova_value_forward_noalloc (static scratch, no workspace) against
mova_value_forward (caller's workspace), through the C ABI.

Both run the same kernels, so the outputs and the reported routing must be
identical bit for bit.  Two calls in a row on each path, the second with a
smaller input, so the second call runs on scratch the first one left behind:
* decode path: the decode layer at T = 64, then T = 37;
* grouped path: the prefill chunk at T = 4096, then T = 300.
The prefill outputs are also checked against the oracle on a seeded sample of
tokens (routing rule on every token).
"""
import sys

import numpy as np
import pytest
import torch

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


def _both(g, T, sh):
    """(noalloc out, idx, w), (workspace out, idx, w) for the first T tokens."""
    x = g["x"][:T].contiguous()
    H, D = sh.n_kv_heads, sh.head_dim
    outs = []
    for which in ("noalloc", "workspace"):
        out = torch.full((T, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        idx = torch.full((T, sh.k), -7, dtype=torch.int32, device=DEV)
        w = torch.full((T, sh.k), float("nan"), dtype=torch.float32, device=DEV)
        if which == "noalloc":
            before = torch.cuda.memory_allocated()
            binding.value_forward_noalloc(x, g["router_w"], g["router_b"], g["expert_w"], sh.k,
                                          sh.scale, out, topk_idx=idx, topk_w=w)
            assert torch.cuda.memory_allocated() == before
        else:
            binding.value_forward(x, g["router_w"], g["router_b"], g["expert_w"], sh.k, sh.scale,
                                  H, D, out=out, topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        outs.append((out, idx, w))
    return outs


@pytest.mark.parametrize("name,T1,T2", [("decode", 64, 37), ("prefill", 4096, 300)])
def test_noalloc_matches_workspace_entry_point(name, T1, T2):
    sh = inputs.WORKLOADS[name].shape
    say(f"noalloc {name}: T={T1} then T={T2}")
    g = P.to_gpu_inputs(inputs.make_workload(name, T=T1), DEV)
    for T in (T1, T2):
        (o1, i1, w1), (o2, i2, w2) = _both(g, T, sh)
        assert torch.equal(i1, i2), f"{name} T={T}: routing differs"
        assert torch.equal(w1.view(torch.int32), w2.view(torch.int32)), f"{name} T={T}: weights"
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"{name} T={T}: outputs"
        rows = np.random.default_rng(T).choice(T, size=min(T, 256), replace=False)
        st = P.full_check({k: (v[:T] if k == "x" else v) for k, v in g.items()}, sh.k, sh.scale,
                          sh.n_kv_heads, sh.head_dim, o1, i1, w1, tokens=np.sort(rows),
                          what=f"noalloc {name} T={T}")
        say(f"  T={T}: bitwise equal to the workspace entry point; oracle {st}")


def test_noalloc_refuses_calls_beyond_its_scratch():
    sh = inputs.WORKLOADS["prefill"].shape
    T = 8192
    assert binding.workspace_bytes(T, sh.d, sh.E, sh.k, sh.n_kv_heads, sh.head_dim) > \
        binding.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, sh.d, dtype=torch.bfloat16, device=DEV)
    rw = torch.zeros(sh.E, sh.d, dtype=torch.bfloat16, device=DEV)
    ew = torch.zeros(sh.E, sh.N, sh.d, dtype=torch.bfloat16, device=DEV)
    out = torch.full((T, sh.n_kv_heads, sh.head_dim), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(binding.MovaError, match="SCRATCH"):
        binding.value_forward_noalloc(x, rw, None, ew, sh.k, sh.scale, out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call must leave the output untouched"


@pytest.mark.parametrize("name,T,T_other", [("decode", 64, 37), ("prefill", 1024, 300)])
def test_noalloc_graph_replays(name, T, T_other):
    """The entry point is meant for code under graph capture: one call
    captured into a HIP graph, replayed four times with an eager call of
    another size on the same scratch before each replay, gives the eager
    call's bits (output and routing) on every replay."""
    sh = inputs.WORKLOADS[name].shape
    H, D = sh.n_kv_heads, sh.head_dim
    say(f"noalloc graph {name}: T={T}, eager T={T_other} between replays")
    g = P.to_gpu_inputs(inputs.make_workload(name, T=T), DEV)
    out = torch.empty(T, H, D, dtype=torch.bfloat16, device=DEV)
    idx = torch.empty(T, sh.k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, sh.k, dtype=torch.float32, device=DEV)
    xo = g["x"][:T_other].contiguous()
    out_o = torch.empty(T_other, H, D, dtype=torch.bfloat16, device=DEV)

    def call():
        binding.value_forward_noalloc(g["x"], g["router_w"], g["router_b"], g["expert_w"], sh.k,
                                      sh.scale, out, topk_idx=idx, topk_w=w)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = (out.clone(), idx.clone(), w.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(4):
        out.fill_(float("nan"))
        idx.fill_(-7)
        w.fill_(float("nan"))
        binding.value_forward_noalloc(xo, g["router_w"], g["router_b"], g["expert_w"], sh.k,
                                      sh.scale, out_o)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[0].view(torch.int16)), f"replay {rep}: outputs"
        assert torch.equal(idx, eager[1]), f"replay {rep}: routing"
        assert torch.equal(w.view(torch.int32), eager[2].view(torch.int32)), f"replay {rep}: weights"
    rows = np.random.default_rng(T + 1).choice(T, size=min(T, 128), replace=False)
    st = P.full_check(g, sh.k, sh.scale, H, D, out, idx, w, tokens=np.sort(rows),
                      what=f"noalloc graph {name} T={T}")
    say(f"  four replays bitwise equal to the eager call; oracle {st}")
    del graph
