"""HIP path vs the CPU oracle, through the C ABI (ctypes binding).

Acceptance rules are in tests/paritylib.py.  Cases: the tiny fp32 layer,
ragged shapes on both execution paths (weight-streaming decode and grouped
GEMM), the edge cases of the method (one expert, k = E, all tokens tied onto
the same experts, zero input, k = 8), and every workload at its full size:
the decode step and prefill chunk in full, the skewed and chunked workloads
with routing checked on every token and outputs on a seeded sample plus all
near-tie tokens and the hottest expert's tokens.
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
    binding.set_override("gemm_tile", None)


def run_forward(g, k, scale, H, D, path=None):
    if path is None:
        binding.set_override("path", None)
    else:
        binding.set_override("path", path)
    T = g["x"].shape[0]
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    out = binding.value_forward(g["x"], g["router_w"], g["router_b"], g["expert_w"], k, scale,
                                H, D, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    binding.set_override("path", None)
    return out, idx, w


def layer(T, d, E, k, H, D, seed, bias="uniform"):
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=H, head_dim=D)
    return P.to_gpu_inputs(inputs.make_layer(shape, seed, torch.bfloat16, bias)), shape


def test_tiny_workload():
    w = inputs.WORKLOADS["tiny"]
    sh = w.shape
    say(f"tiny: {sh}")
    g = P.to_gpu_inputs(inputs.make_workload("tiny"))
    for path in ("decode", "grouped"):
        out, idx, wt = run_forward(g, sh.k, sh.scale, sh.n_kv_heads, sh.head_dim, path)
        assert out.shape == (sh.T, sh.n_kv_heads, sh.head_dim)
        st = P.full_check(g, sh.k, sh.scale, sh.n_kv_heads, sh.head_dim, out, idx, wt, what=f"tiny/{path}")
        say(f"  {path}: {st}")


RAGGED = [
    # T, d, E, k, H, D
    (1, 256, 8, 2, 2, 32),
    (5, 512, 16, 4, 1, 64),
    (17, 256, 64, 4, 8, 16),
    (63, 320, 33, 3, 3, 64),
    (64, 2560, 64, 4, 8, 128),
    (65, 256, 8, 2, 2, 64),
    (100, 512, 64, 8, 4, 64),
    (129, 192, 5, 5, 1, 192),
    (300, 1024, 64, 4, 8, 128),
    (1000, 256, 64, 6, 2, 96),
    (100, 8192, 16, 2, 1, 64),     # long rows: 256 k steps
    (700, 320, 64, 3, 2, 64),      # router residue classes of unequal length
]


@pytest.mark.parametrize("T,d,E,k,H,D", RAGGED)
def test_ragged_shapes_both_paths(T, d, E, k, H, D):
    say(f"ragged T={T} d={d} E={E} k={k} H={H} D={D}")
    g, sh = layer(T, d, E, k, H, D, seed=T * 7 + E)
    paths = ["grouped"] + (["decode"] if T <= 256 else [])
    outs = {}
    for path in paths:
        out, idx, w = run_forward(g, k, 2.5, H, D, path)
        st = P.full_check(g, k, 2.5, H, D, out, idx, w, what=f"{path} {T}x{d} E{E} k{k}")
        say(f"  {path}: {st}")
        outs[path] = (out, idx, w)
    if len(outs) == 2:
        # Same routing bits and same expert arithmetic: the two paths agree exactly.
        a, b = outs["grouped"], outs["decode"]
        assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
        assert torch.equal(a[0], b[0])


GEMM_TILES = ["256x256", "128x256", "128x128", "128x128s3", "128x128s4", "128x128w4", "352x256"]


@pytest.mark.parametrize("T,d,E,k,H,D", [(200, 512, 16, 4, 2, 64), (700, 320, 33, 3, 3, 64),
                                         (4096, 2560, 64, 4, 8, 128)])
def test_grouped_gemm_every_tile_shape(T, d, E, k, H, D):
    """Each tile shape of the grouped GEMM against the oracle; all of them (and
    the decode path where it applies) give the same bits, since every output's
    MFMA chain runs over the k steps in the same order."""
    g, sh = layer(T, d, E, k, H, D, seed=T + 3 * E)
    outs = {}
    for tile in GEMM_TILES:
        binding.set_override("gemm_tile", tile)
        say(f"grouped tile {tile}: T={T} d={d} E={E} k={k} H={H} D={D}")
        out, idx, w = run_forward(g, k, 2.5, H, D, "grouped")
        binding.set_override("gemm_tile", None)
        st = P.full_check(g, k, 2.5, H, D, out, idx, w, what=f"tile {tile}")
        say(f"  {st}")
        outs[tile] = out
    if T <= 256:
        outs["decode"] = run_forward(g, k, 2.5, H, D, "decode")[0]
    ref = outs["256x256"]
    for name, o in outs.items():
        assert torch.equal(o, ref), f"{name} differs from 256x256"


def test_widest_output_both_paths():
    """N at the top of the supported domain (128 heads x 128 = 16384 columns)."""
    T, d, E, k, H, D = 70, 256, 4, 2, 128, 128
    say(f"widest output T={T} d={d} E={E} k={k} N={H * D}")
    g, sh = layer(T, d, E, k, H, D, seed=1601)
    outs = {}
    for path in ("grouped", "decode"):
        out, idx, w = run_forward(g, k, 2.5, H, D, path)
        st = P.full_check(g, k, 2.5, H, D, out, idx, w, what=f"{path} N={H * D}")
        say(f"  {path}: {st}")
        outs[path] = (out, idx, w)
    a, b = outs["grouped"], outs["decode"]
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]) and torch.equal(a[0], b[0])


def test_million_tokens():
    """2^20 tokens in one call (narrow layer, k = 8): large grids, a 16K-chunk
    dispatch table and 64-bit offsets.  Routing checked on every token, outputs
    on a seeded sample plus every near-tie token."""
    T, d, E, k, H, D = 1 << 20, 64, 64, 8, 1, 64
    say(f"million tokens T={T} d={d} E={E} k={k} N={H * D}")
    g, sh = layer(T, d, E, k, H, D, seed=2027)
    out, idx, w = run_forward(g, k, 2.5, H, D)
    o = P.oracle_inputs(g)
    ref = oracle.route(o["x"], o["router_w"], o["router_b"], k, 2.5)
    ties = np.nonzero(ref.margin <= P.MARGIN)[0][:4096]
    rows = sample_rows(T, 2048, 13, extra=list(ties))
    st = P.full_check(g, k, 2.5, H, D, out, idx, w, tokens=rows, ref=ref, what="2^20 tokens")
    say(f"  rows={rows.size} {st}")
    del out, idx, w, g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [40, 600])
def test_bias_omitted_equals_zero_bias(T):
    """router_b = NULL means a zero bias: same bits as passing zeros, both paths."""
    d, E, k, H, D = 512, 32, 4, 2, 64
    g, sh = layer(T, d, E, k, H, D, seed=T + 5)
    g_none = dict(g, router_b=None)
    g_zero = dict(g, router_b=torch.zeros(E, dtype=torch.float32, device=DEV))
    for path in ("grouped", "decode") if T <= 256 else ("grouped",):
        a = run_forward(g_none, k, 2.5, H, D, path)
        b = run_forward(g_zero, k, 2.5, H, D, path)
        assert all(torch.equal(u, v) for u, v in zip(a, b)), path
        st = P.full_check(g_none, k, 2.5, H, D, *a, what=f"{path} no bias")
        say(f"  {path} T={T}: {st}")
    i1, w1 = binding.route(g["x"], g["router_w"], None, k, 2.5)
    i2, w2 = binding.route(g["x"], g["router_w"], g_zero["router_b"], k, 2.5)
    assert torch.equal(i1, i2) and torch.equal(w1, w2)


@pytest.mark.parametrize("T", [64, 1000])
def test_power_of_two_scale_is_exact(T):
    """Doubling the scale doubles weights and outputs bit for bit (every
    rounding step, fp16 partials and the bf16 output included, commutes with
    multiplication by 2)."""
    d, E, k, H, D = 2560, 64, 4, 8, 128
    g, sh = layer(T, d, E, k, H, D, seed=T + 9)
    o1, i1, w1 = run_forward(g, k, 2.5, H, D)
    o2, i2, w2 = run_forward(g, k, 5.0, H, D)
    assert torch.equal(i1, i2)
    assert torch.equal(w2, 2 * w1)
    assert torch.equal(o2.float(), 2 * o1.float())


def test_single_expert():
    g, sh = layer(40, 256, 1, 1, 2, 32, seed=1)
    for path in ("decode", "grouped"):
        out, idx, w = run_forward(g, 1, 2.5, 2, 32, path)
        assert (idx == 0).all()
        P.full_check(g, 1, 2.5, 2, 32, out, idx, w, what=f"E=1 {path}")


def test_k_equals_E():
    g, sh = layer(90, 256, 6, 6, 1, 64, seed=2)
    out, idx, w = run_forward(g, 6, 2.5, 1, 64)
    P.full_check(g, 6, 2.5, 1, 64, out, idx, w, what="k=E")


@pytest.mark.parametrize("T", [64, 700])
def test_all_tokens_tied_onto_same_experts(T):
    """Identical router rows and zero bias: every token ties across all experts and
    the lower indices win, so experts 0..k-1 receive every token (c_e = T)."""
    g, sh = layer(T, 512, 16, 4, 2, 64, seed=3, bias="zero")
    g["router_w"] = g["router_w"][:1].expand(16, -1).contiguous()
    out, idx, w = run_forward(g, 4, 2.5, 2, 64)
    expect = torch.arange(4, dtype=torch.int32, device=DEV).expand(T, 4)
    assert torch.equal(idx, expect)
    assert torch.allclose(w, torch.full_like(w, 2.5 / 4), atol=1e-6, rtol=0)
    P.full_check(g, 4, 2.5, 2, 64, out, idx, w, what=f"all tied T={T}")


def test_zero_input_gives_zero_output():
    g, sh = layer(80, 256, 8, 2, 2, 32, seed=4)
    g["x"].zero_()
    out, idx, w = run_forward(g, 2, 2.5, 2, 32)
    assert (out.float() == 0).all()
    b = g["router_b"].cpu().numpy()
    order = sorted(range(8), key=lambda e: (-b[e], e))[:2]
    assert (idx.cpu().numpy() == np.array(order)).all()


def test_max_k_and_wide_layer():
    g, sh = layer(200, 4096, 64, 8, 16, 128, seed=5)
    out, idx, w = run_forward(g, 8, 2.5, 16, 128)
    P.full_check(g, 8, 2.5, 16, 128, out, idx, w, what="k=8 d=4096 N=2048")


def test_empty_call():
    g, sh = layer(8, 256, 8, 2, 2, 32, seed=6)
    x = g["x"][:0]
    out = binding.value_forward(x, g["router_w"], g["router_b"], g["expert_w"], 2, 2.5, 2, 32)
    assert out.shape == (0, 2, 32)
    idx, w = binding.route(x, g["router_w"], g["router_b"], 2)
    assert idx.shape == (0, 2)


def test_route_only_matches_forward_routing():
    for T in (48, 1000):
        g, sh = layer(T, 2560, 64, 4, 8, 128, seed=T)
        _, idx_f, w_f = run_forward(g, 4, 2.5, 8, 128)
        idx_r, w_r = binding.route(g["x"], g["router_w"], g["router_b"], 4, 2.5)
        torch.cuda.synchronize()
        assert torch.equal(idx_f, idx_r) and torch.equal(w_f, w_r)
        o = P.oracle_inputs(g)
        P.check_routing(idx_r, w_r, oracle.route(o["x"], o["router_w"], o["router_b"], 4, 2.5), 2.5)


# ---------------------------------------------------------------- full-size workloads

def workload_inputs(name, layer_no=0, T=None):
    return P.to_gpu_inputs(inputs.make_workload(name, layer=layer_no, T=T))


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_workload_full(name):
    sh = inputs.WORKLOADS[name].shape
    say(f"{name}: full parity, {sh}")
    g = workload_inputs(name)
    out, idx, w = run_forward(g, sh.k, sh.scale, sh.n_kv_heads, sh.head_dim)
    st = P.full_check(g, sh.k, sh.scale, sh.n_kv_heads, sh.head_dim, out, idx, w, what=name)
    say(f"  {st}")


@pytest.mark.parametrize("T", [1, 2, 4, 8, 16])
def test_small_batch_full_size(T):
    """Small-batch decode at the value layer's full size (the token-major
    kernel with the selection and the combine fused, T * k <= 64): every
    token against the oracle."""
    sh = inputs.WORKLOADS["decode"].shape
    say(f"small batch T={T}: full parity")
    g = workload_inputs("decode", T=T)
    out, idx, w = run_forward(g, sh.k, sh.scale, sh.n_kv_heads, sh.head_dim)
    st = P.full_check(g, sh.k, sh.scale, sh.n_kv_heads, sh.head_dim, out, idx, w,
                      what=f"small batch T={T}")
    say(f"  {st}")


def sample_rows(T, n, seed, extra=()):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    rows.update(int(r) for r in extra)
    rows.update([0, T - 1])
    return np.array(sorted(rows))


def test_skewed_workload():
    w = inputs.WORKLOADS["skewed"]
    sh = w.shape
    say(f"skewed: routing on all {sh.T} tokens, outputs sampled")
    g = workload_inputs("skewed")
    out, idx, wt = run_forward(g, sh.k, sh.scale, sh.n_kv_heads, sh.head_dim)
    o = P.oracle_inputs(g)
    ref = oracle.route(o["x"], o["router_w"], o["router_b"], sh.k, sh.scale)
    counts = np.bincount(ref.idx.ravel(), minlength=sh.E)
    hot = int(counts.argmax())
    hot_rows = np.nonzero((ref.idx == hot).any(axis=1))[0][:: max(1, counts.max() // 256)]
    ties = np.nonzero(ref.margin <= P.MARGIN)[0]
    rows = sample_rows(sh.T, 1024, 11, extra=list(hot_rows) + list(ties))
    st = P.full_check(g, sh.k, sh.scale, sh.n_kv_heads, sh.head_dim, out, idx, wt,
                      tokens=rows, ref=ref, what="skewed")
    say(f"  rows={rows.size} hot expert={hot} ({counts.max()} tokens) {st}")


def test_chunked_workload_layers():
    """65536 tokens as 8 calls of 8192 through 4 layers with distinct weights."""
    w = inputs.WORKLOADS["chunked"]
    sh = w.shape
    total = sh.T * w.chunks
    x = inputs.make_tokens(total, sh.d, w.seed).to(DEV)
    for layer_no in range(w.layers):
        say(f"chunked: layer {layer_no}")
        wts = P.to_gpu_inputs({"x": x[:1].cpu(),
                               **inputs.make_weights(sh, w.seed, torch.bfloat16, w.bias, layer_no)})
        out = torch.empty(total, sh.n_kv_heads, sh.head_dim, dtype=torch.bfloat16, device=DEV)
        idx = torch.empty(total, sh.k, dtype=torch.int32, device=DEV)
        wt = torch.empty(total, sh.k, dtype=torch.float32, device=DEV)
        for c in range(w.chunks):
            s = slice(c * sh.T, (c + 1) * sh.T)
            binding.value_forward(x[s], wts["router_w"], wts["router_b"], wts["expert_w"], sh.k,
                                  sh.scale, sh.n_kv_heads, sh.head_dim, out=out[s],
                                  topk_idx=idx[s], topk_w=wt[s])
        torch.cuda.synchronize()
        g = dict(wts, x=x)
        o = P.oracle_inputs(g)
        ref = oracle.route(o["x"], o["router_w"], o["router_b"], sh.k, sh.scale)
        ties = np.nonzero(ref.margin <= P.MARGIN)[0]
        rows = sample_rows(total, 2048, 100 + layer_no, extra=ties)
        st = P.full_check(g, sh.k, sh.scale, sh.n_kv_heads, sh.head_dim, out, idx, wt,
                          tokens=rows, ref=ref, what=f"chunked layer {layer_no}")
        say(f"  {st}")
        del wts, g, o
