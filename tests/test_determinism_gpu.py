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


@pytest.mark.parametrize("T", [4, 64, 1000])
def test_graph_replay_matches_eager(T):
    """A captured call replays to the eager result every time, with eager work
    and synchronisations between the replays (token-major kernel with the
    selection fused at T=4, decode path at T=64, grouped path at T=1000)."""
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


def _layer(T, d, E, k, heads, hd, seed, mode):
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=heads, head_dim=hd)
    g = {n: v.to(DEV) for n, v in inputs.make_layer(shape, seed, torch.bfloat16, "uniform").items()}
    if mode == "ties":
        # Experts 2j and 2j + 1 score alike: the lower index must rank first.
        g["router_w"][1::2] = g["router_w"][0::2][: E // 2]
        g["router_b"].zero_()
    elif mode == "one_expert":
        # Every token's first choice is expert E // 2 (all T tokens hit it).
        g["router_b"][E // 2] = 50.0
    return g


def _run(g, k, heads, hd, forced):
    for name, val in forced.items():
        binding.set_override(name, val)
    T = g["x"].shape[0]
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    out = binding.value_forward(g["x"], g["router_w"], g["router_b"], g["expert_w"], k, 2.5, heads,
                                hd, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    for name in forced:
        binding.set_override(name, None)
    return out, idx, w


@pytest.mark.parametrize("T,d,E,k,heads,hd,mode", [
    (64, 2560, 64, 4, 8, 128, "uniform"),
    (1, 512, 64, 4, 2, 128, "uniform"),
    (5, 512, 16, 8, 1, 64, "uniform"),
    (100, 512, 64, 1, 2, 128, "uniform"),
    (256, 512, 64, 4, 2, 128, "uniform"),
    (160, 2560, 64, 4, 8, 128, "uniform"),   # 16-pair passes up to 10 pairs per expert on average
    (150, 512, 64, 4, 2, 128, "one_expert"),  # ... and an expert of 150 pairs in ten of them
    (137, 512, 40, 6, 1, 128, "ties"),
    (256, 512, 64, 4, 1, 128, "one_expert"),
    (250, 1024, 7, 3, 1, 64, "one_expert"),
])
def test_decode_and_grouped_paths_bitwise(T, d, E, k, heads, hd, mode):
    """The decode path (two-kernel router, weight-streaming experts) and the
    grouped path (LDS-staged router, dispatch, grouped GEMM) give the same routing,
    weights and output bits, also with tied scores and with every token on
    one expert."""
    g = _layer(T, d, E, k, heads, hd, seed=T + E, mode=mode)
    print(f"paths T={T} d={d} E={E} k={k} N={heads * hd} {mode}", flush=True)
    dec = _run(g, k, heads, hd, {"path": "decode"})
    grp = _run(g, k, heads, hd, {"path": "grouped"})
    for name, a, b in zip(("out", "idx", "w"), dec, grp):
        assert torch.equal(a, b), f"{name}: decode path differs from the grouped path"
    if mode == "ties":
        # Experts 2j and 2j + 1 tie, so 2j + 1 is only ever taken after 2j.
        for row in dec[1].cpu().tolist():
            for pos, e in enumerate(row):
                if e % 2 == 1:
                    assert e - 1 in row[:pos], f"tie order broken in {row}"
    if mode == "one_expert":
        assert bool((dec[1][:, 0] == E // 2).all())




@pytest.mark.parametrize("T,d,E,k,mode", [(4096, 2560, 64, 4, "uniform"), (1000, 320, 40, 8, "uniform"),
                                          (777, 192, 7, 3, "uniform"), (8192, 2560, 64, 4, "uniform"),
                                          (33, 2560, 64, 6, "uniform"), (1000, 512, 64, 4, "ties"),
                                          (600, 2560, 64, 8, "one_expert")])
def test_router_configs_bitwise(T, d, E, k, mode):
    """Every router configuration (16, 32 or 64 tokens per workgroup; 2 to 4
    LDS stages) gives the same routing bits, and the grouped path built on its
    dispatch chunks the same output bits, also with tied scores and with every
    token on one expert."""
    g = _layer(T, d, E, k, 1, 64, seed=T + d, mode=mode)
    binding.set_override("path", "grouped")
    res = {}
    kinds = ("16", "32s4", "32s3", "64")
    for kind in kinds:
        binding.set_override("router", kind)
        print(f"router {kind} T={T} d={d} E={E} k={k} {mode}", flush=True)
        idx, w = binding.route(g["x"], g["router_w"], g["router_b"], k, 2.5)
        out = binding.value_forward(g["x"], g["router_w"], g["router_b"], g["expert_w"], k, 2.5,
                                    1, 64)
        torch.cuda.synchronize()
        res[kind] = (idx, w, out)
    binding.set_override("router", None)
    binding.set_override("path", None)
    for kind in kinds[1:]:
        for name, a, b in zip(("idx", "w", "out"), res[kind], res["16"]):
            assert torch.equal(a, b), f"{kind}: {name} differs from the 16-token router"
    if mode == "ties":
        for row in res["16"][0].cpu().tolist():
            for pos, e in enumerate(row):
                if e % 2 == 1:
                    assert e - 1 in row[:pos], f"tie order broken in {row}"


@pytest.mark.parametrize("groups", ["1", "2"])
@pytest.mark.parametrize("T,d,E,k,heads,hd", [(64, 2560, 64, 4, 1, 128), (64, 2560, 64, 4, 4, 128),
                                              (100, 512, 16, 3, 3, 64), (256, 256, 40, 8, 1, 64),
                                              (7, 320, 5, 2, 2, 32)])
def test_decode_column_groups_bitwise(groups, T, d, E, k, heads, hd):
    """The decode kernel with one or two 16-column groups per wave (narrow
    outputs, e.g. one GPU's share of the heads, take one) gives the grouped
    path's bits."""
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=heads, head_dim=hd)
    g = {n: v.to(DEV) for n, v in inputs.make_layer(shape, T + E + heads, torch.bfloat16, "uniform").items()}
    print(f"decode groups={groups} T={T} d={d} E={E} k={k} N={heads * hd}", flush=True)
    binding.set_override("decode_groups", groups)
    dec = _run(g, k, heads, hd, {"path": "decode"})
    binding.set_override("decode_groups", None)
    grp = _run(g, k, heads, hd, {"path": "grouped"})
    for name, a, b in zip(("out", "idx", "w"), dec, grp):
        assert torch.equal(a, b), f"{name}: decode ({groups} groups) differs from the grouped path"


@pytest.mark.parametrize("T,d,E,k,heads,hd", [(1, 2560, 64, 4, 8, 128), (3, 2560, 64, 4, 8, 128),
                                              (8, 2560, 64, 8, 8, 128), (16, 3072, 64, 4, 2, 128),
                                              (5, 64, 7, 3, 1, 64), (2, 256, 64, 1, 1, 128),
                                              (16, 512, 40, 4, 4, 64)])
def test_decode_chain_kernel_bitwise(T, d, E, k, heads, hd):
    """The small-T kernels (a chain's k steps split over four waves, the
    accumulator handed on; and token-major with the combine fused) give the
    grouped path's bits."""
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=heads, head_dim=hd)
    g = {n: v.to(DEV) for n, v in inputs.make_layer(shape, 7 * T + d, torch.bfloat16, "uniform").items()}
    print(f"decode chain T={T} d={d} E={E} k={k} N={heads * hd}", flush=True)
    binding.set_override("decode_chain", "on")
    dec = _run(g, k, heads, hd, {"path": "decode"})
    binding.set_override("decode_chain", "off")
    reg = _run(g, k, heads, hd, {"path": "decode"})
    binding.set_override("decode_chain", "token")
    tok = _run(g, k, heads, hd, {"path": "decode"})
    binding.set_override("decode_chain", None)
    grp = _run(g, k, heads, hd, {"path": "grouped"})
    for name, a, b, c, e in zip(("out", "idx", "w"), dec, reg, grp, tok):
        assert torch.equal(a, c), f"{name}: chain kernel differs from the grouped path"
        assert torch.equal(b, c), f"{name}: decode kernel differs from the grouped path"
        assert torch.equal(e, c), f"{name}: token-major kernel differs from the grouped path"


@pytest.mark.parametrize("Ts", [(4, 64), (64, 1000), (1000, 2048)])
def test_concurrent_streams_bitwise(Ts):
    """Two calls in flight at once on two streams, each with its own
    workspace and output (different paths where the token counts differ),
    give the bits of the same calls made alone."""
    gs = [gpu_layer(T, seed=20 + i) for i, T in enumerate(Ts)]
    wss = [torch.empty(binding.workspace_bytes(T, 2560, 64, 4, 8, 128), dtype=torch.uint8, device=DEV)
           for T in Ts]
    refs = [fwd_ws(g, ws).clone() for g, ws in zip(gs, wss)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in Ts]
    outs = [torch.empty_like(r) for r in refs]
    print(f"two streams T={Ts}", flush=True)
    for rep in range(10):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for g, ws, o, s in zip(gs, wss, outs, streams):
            with torch.cuda.stream(s):
                fwd_ws(g, ws, o)
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), f"rep {rep}: stream {i} (T={Ts[i]}) differs"
