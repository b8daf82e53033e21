"""FFN mixture of experts (mova_ffn_moe_forward) vs the CPU oracle.

Routing: the index / weight rules of ``paritylib.check_routing`` on every
token.  Outputs: the output rules on every token (sampled rows at T = 4096),
against the oracle evaluated with the GPU's choice on near-tie tokens.  Also:
the gate/up interleaving, a token's row not depending on the other tokens,
and no shared expert.
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


def gpu_layer(sh, seed):
    L = inputs.make_ffn_layer(sh, seed)
    g = {k: v.to(DEV).contiguous() for k, v in L.items()}
    g["gate_up_w"] = binding.ffn_pack_gate_up(g["gate_w"], g["up_w"])
    if sh.inter_shared:
        g["shared_gate_up_w"] = binding.ffn_pack_gate_up(g["shared_gate_w"], g["shared_up_w"])
    return L, g


def run_ffn(g, sh, x=None):
    x = g["x"] if x is None else x
    T = x.shape[0]
    idx = torch.empty(T, sh.k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, sh.k, dtype=torch.float32, device=DEV)
    out = binding.ffn_moe_forward(x, g["router_w"], g["router_b"], g["gate_up_w"], g["down_w"],
                                  sh.k, sh.scale, g.get("shared_gate_up_w"),
                                  g.get("shared_down_w"), topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    return out, idx, w


def ffn_reference(L, sh, rows, eff_idx, eff_w):
    """The oracle's experts on the given rows with the routing to check."""
    o = {k: v.double().numpy() for k, v in L.items()}
    x = o["x"][rows]
    out = np.zeros((len(rows), sh.d))
    for n, t in enumerate(rows):
        for j in range(sh.k):
            e = int(eff_idx[t, j])
            out[n] += eff_w[t, j] * oracle.swiglu_expert(x[n:n + 1], o["gate_w"][e], o["up_w"][e],
                                                         o["down_w"][e])[0]
    if sh.inter_shared:
        out += oracle.swiglu_expert(x, o["shared_gate_w"], o["shared_up_w"], o["shared_down_w"])
    return out


CASES = [
    # T, d, E, k, inter, inter_shared
    (37, 256, 12, 3, 64, 64),
    (64, 2560, 100, 8, 768, 768),
    (300, 512, 100, 8, 128, 0),
    (200, 192, 8, 8, 64, 128),
    (256, 256, 100, 8, 64, 192),
    (100, 128, 128, 8, 64, 0),     # E at its maximum: every lane holds two experts
    (20, 64, 1, 1, 64, 64, 1.0),   # one expert, k = 1 (scale 1: the whole scale lands on
                                   # one expert, and 2.5 would push |out| past the range
                                   # the max-abs rule is set for)
    (257, 256, 100, 8, 64, 192),
    (2048, 2560, 100, 8, 768, 768),  # 256 x 256 tiles (the experts average 164 rows)
    (4096, 2560, 100, 8, 768, 768),
]


@pytest.mark.parametrize("case", CASES)
def test_ffn_matches_oracle(case):
    T, d, E, k, inter, inter_s = case[:6]
    scale = case[6] if len(case) > 6 else 2.5
    sh = inputs.FfnShape(T=T, d=d, E=E, k=k, inter=inter, inter_shared=inter_s, scale=scale)
    say(f"ffn T={T} d={d} E={E} k={k} inter={inter} shared={inter_s}")
    L, g = gpu_layer(sh, seed=T + E)
    out, idx, w = run_ffn(g, sh)
    o = {kk: v.double().numpy() for kk, v in L.items()}
    ref = oracle.route(o["x"], o["router_w"], o["router_b"], k, sh.scale)
    rc = P.check_routing(idx, w, ref, sh.scale)
    rows = np.arange(T) if T <= 512 else np.unique(
        np.r_[np.random.default_rng(3).choice(T, 200, replace=False), 0, T - 1])
    want = ffn_reference(L, sh, rows, rc.effective_idx, rc.effective_w)
    got = out[torch.as_tensor(rows, device=DEV)]
    st = P.check_output(got, want, what=f"ffn T={T}")
    say(f"  {st} near_ties={rc.near_ties}")


def test_ffn_pack_gate_up_layout():
    E, inter, d = 3, 64, 128
    gate = torch.randn(E, inter, d, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    up = torch.randn(E, inter, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    got = binding.ffn_pack_gate_up(gate.to(DEV), up.to(DEV)).cpu()
    want = torch.empty(E, 2 * inter, d, dtype=torch.bfloat16)
    for b in range(inter // 16):
        want[:, 32 * b:32 * b + 16] = gate[:, 16 * b:16 * b + 16]
        want[:, 32 * b + 16:32 * b + 32] = up[:, 16 * b:16 * b + 16]
    assert torch.equal(got, want)


def test_ffn_rows_do_not_depend_on_other_tokens():
    # Both calls above 256 tokens: the same kernels (the shared expert's
    # split-k kernel below 257 tokens sums in another order than the tiled one).
    sh = inputs.FfnShape(T=600, d=512, E=100, k=8, inter=128, inter_shared=64)
    L, g = gpu_layer(sh, seed=9)
    full, idx, w = run_ffn(g, sh)
    part, idx2, w2 = run_ffn(g, sh, g["x"][123:423].contiguous())
    assert torch.equal(idx[123:423], idx2) and torch.equal(w[123:423], w2)
    assert torch.equal(full[123:423], part)
    again, _, _ = run_ffn(g, sh)
    assert torch.equal(full, again)


@pytest.mark.parametrize("E,k,ties", [(100, 8, None), (128, 8, "planes"), (100, 8, "pairs"),
                                      (12, 3, None), (64, 4, None), (65, 5, "planes")])
def test_ffn_router_kernels_bitwise(E, k, ties):
    """From 1024 tokens on, the FFN routes with the LDS-staged router (two
    experts per selecting lane); below, with its two-kernel router.  Both give
    the same routing bits: a call of 1536 tokens against calls on slices of
    it, also with experts j and j + 64 tied (the two lanes' planes) or
    experts 2j and 2j + 1 tied (lower index first)."""
    sh = inputs.FfnShape(T=1536, d=512, E=E, k=k, inter=64, inter_shared=0)
    L, g = gpu_layer(sh, seed=E + k)
    if ties == "planes" and E > 64:
        g["router_w"][64:E] = g["router_w"][0:E - 64]
        g["router_b"].zero_()
    elif ties == "pairs":
        g["router_w"][1::2] = g["router_w"][0::2][: E // 2]
        g["router_b"].zero_()
    say(f"ffn router E={E} k={k} ties={ties}")
    _, idx, w = run_ffn(g, sh)
    for a, b in ((0, 700), (700, 1400), (1400, 1536)):
        _, i2, w2 = run_ffn(g, sh, g["x"][a:b].contiguous())
        assert torch.equal(idx[a:b], i2) and torch.equal(w[a:b], w2), (a, b)
    rows = idx.cpu().tolist()
    for row in rows:
        assert len(set(row)) == k
        for pos, e in enumerate(row):
            if ties == "planes" and e >= 64:
                assert e - 64 in row[:pos], f"plane tie order broken in {row}"
            if ties == "pairs" and e % 2 == 1:
                assert e - 1 in row[:pos], f"pair tie order broken in {row}"


@pytest.mark.parametrize("T,d,E,k,inter,inter_s", [
    (64, 2560, 100, 8, 768, 768),
    (1, 256, 12, 3, 64, 64),
    (256, 192, 128, 8, 64, 128),   # d % 128 != 0: half a column slice in the down projection
    (100, 512, 100, 8, 128, 0),
    (200, 128, 1, 1, 64, 64),      # every token on one expert: 200 pairs, passes of 32
])
def test_ffn_decode_and_grouped_paths_bitwise(T, d, E, k, inter, inter_s):
    """Few tokens take the weight-streaming decode kernel for the routed
    experts; forcing the grouped GEMM instead gives the same bits."""
    sh = inputs.FfnShape(T=T, d=d, E=E, k=k, inter=inter, inter_shared=inter_s,
                         scale=1.0 if k == 1 else 2.5)
    say(f"ffn paths T={T} d={d} E={E} k={k} inter={inter} shared={inter_s}")
    L, g = gpu_layer(sh, seed=T + 7 * E)
    res = {}
    for path in ("decode", "grouped"):
        binding.set_override("path", path)
        res[path] = run_ffn(g, sh)
    binding.set_override("path", None)
    for name, a, b in zip(("out", "idx", "w"), res["decode"], res["grouped"]):
        assert torch.equal(a, b), f"{name}: decode path differs from the grouped path"


@pytest.mark.parametrize("T", [64, 600])
def test_ffn_shared_expert_side_stream(T):
    """The shared expert runs on the library's side stream, overlapping the
    router and the routed experts; the result is the bits of running it on
    the caller's stream (the serial override), also when the call is captured in a
    graph and replayed with other work in between."""
    sh = inputs.FfnShape(T=T, d=512, E=100, k=8, inter=128, inter_shared=256)
    say(f"ffn side stream T={T}")
    L, g = gpu_layer(sh, seed=T + 1)
    binding.set_override("serial", "on")
    serial = run_ffn(g, sh)
    binding.set_override("serial", None)
    side = run_ffn(g, sh)
    for name, a, b in zip(("out", "idx", "w"), side, serial):
        assert torch.equal(a, b), f"{name}: side stream changed the result"
    # Graph capture of the forked call, replayed with eager calls between.
    ws = torch.empty(binding.ffn_workspace_bytes(T, sh.d, sh.E, sh.k, sh.inter, sh.inter_shared),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty(T, sh.d, dtype=torch.bfloat16, device=DEV)

    def call():
        binding.ffn_moe_forward(g["x"], g["router_w"], g["router_b"], g["gate_up_w"],
                                g["down_w"], sh.k, sh.scale, g["shared_gate_up_w"],
                                g["shared_down_w"], out=out, workspace=ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(4):
        out.zero_()
        other = run_ffn(g, sh, g["x"][: T // 2].contiguous())   # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, serial[0]), f"replay {rep} differs"
        del other


def test_ffn_concurrent_host_threads():
    """Two host threads call the FFN on their own streams and workspaces (their
    shared experts share the library's side stream): every result matches the
    same call made alone."""
    import threading
    sh = inputs.FfnShape(T=64, d=512, E=100, k=8, inter=128, inter_shared=256)
    L, g = gpu_layer(sh, seed=5)
    xs = [g["x"], inputs.make_tokens(sh.T, sh.d, 77, torch.bfloat16).to(DEV)]
    refs = [run_ffn(g, sh, x)[0].clone() for x in xs]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            ws = torch.empty(binding.ffn_workspace_bytes(sh.T, sh.d, sh.E, sh.k, sh.inter,
                                                         sh.inter_shared),
                             dtype=torch.uint8, device=DEV)
            out = torch.empty(sh.T, sh.d, dtype=torch.bfloat16, device=DEV)
            for rep in range(20):
                with torch.cuda.stream(s):
                    out.zero_()
                    binding.ffn_moe_forward(xs[i], g["router_w"], g["router_b"], g["gate_up_w"],
                                            g["down_w"], sh.k, sh.scale, g["shared_gate_up_w"],
                                            g["shared_down_w"], out=out, workspace=ws)
                s.synchronize()
                if not torch.equal(out, refs[i]):
                    errors.append(f"thread {i} rep {rep} differs")
                    return
        except Exception as exc:  # reported below
            errors.append(f"thread {i}: {exc!r}")

    say("ffn two host threads")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors


FFN_TILES = ["256x256", "128x256", "128x128", "128x128s3", "128x128s4", "128x128w4", "352x256"]


@pytest.mark.parametrize("T,d,E,k,inter,inter_s", [(300, 512, 12, 4, 128, 64), (700, 320, 20, 8, 64, 0)])
def test_ffn_every_tile_shape(T, d, E, k, inter, inter_s):
    """The FFN's grouped GEMMs (SwiGLU gate/up, weighted down) in every tile
    shape: each against the oracle, and all of them with the same bits."""
    sh = inputs.FfnShape(T=T, d=d, E=E, k=k, inter=inter, inter_shared=inter_s)
    L, g = gpu_layer(sh, seed=T + E)
    o = {kk: v.double().numpy() for kk, v in L.items()}
    ref = oracle.route(o["x"], o["router_w"], o["router_b"], k, sh.scale)
    binding.set_override("path", "grouped")
    outs = {}
    for tile in FFN_TILES:
        binding.set_override("gemm_tile", tile)
        say(f"ffn tile {tile}: T={T} d={d} E={E} k={k} inter={inter} shared={inter_s}")
        out, idx, w = run_ffn(g, sh)
        if tile == FFN_TILES[0]:
            rc = P.check_routing(idx, w, ref, sh.scale)
            rows = np.arange(T)
            want = ffn_reference(L, sh, rows, rc.effective_idx, rc.effective_w)
            say(f"  {P.check_output(out, want, what=f'ffn tile {tile}')}")
        outs[tile] = out
    binding.set_override("gemm_tile", None)
    binding.set_override("path", None)
    for tile, out in outs.items():
        assert torch.equal(out, outs[FFN_TILES[0]]), f"{tile} differs from {FFN_TILES[0]}"


@pytest.mark.parametrize("T,d,E,k,inter,inter_s", [(1, 2560, 100, 8, 768, 768), (2, 512, 128, 8, 128, 0),
                                                   (8, 256, 12, 3, 64, 64), (5, 320, 100, 8, 64, 64)])
def test_ffn_chain_kernel_bitwise(T, d, E, k, inter, inter_s):
    """The small-T chain kernel in the SwiGLU and weighted-linear modes
    (E up to 128) gives the grouped path's bits."""
    sh = inputs.FfnShape(T=T, d=d, E=E, k=k, inter=inter, inter_shared=inter_s)
    say(f"ffn chain T={T} d={d} E={E} k={k} inter={inter} shared={inter_s}")
    L, g = gpu_layer(sh, seed=3 * T + E)
    res = {}
    for tag, env in (("chain", {"path": "decode", "decode_chain": "on"}),
                     ("stream", {"path": "decode", "decode_chain": "off"}),
                     ("grouped", {"path": "grouped"})):
        for name, val in env.items():
            binding.set_override(name, val)
        res[tag] = run_ffn(g, sh)
        for name in env:
            binding.set_override(name, None)
    for tag in ("chain", "stream"):
        for name, a, b in zip(("out", "idx", "w"), res[tag], res["grouped"]):
            assert torch.equal(a, b), f"{tag}: {name} differs from the grouped path"
