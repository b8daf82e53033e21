"""Dense value projection (the matched GQA baseline) vs the CPU oracle.

Both kernels are covered on every shape they accept: the split-k kernel (up
to 256 tokens) and the tiled GEMM, forced with the dense_path override.  Shapes span
several tiles with ragged tails in T, d and N; the decode and prefill
workloads run at full size, the 32768-token prefill on sampled rows.
Acceptance rules: ``paritylib.check_dense_output``.
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
    binding.set_override("dense_path", None)
    binding.set_override("gemm_tile", None)


def dense_inputs(T, d, N, seed):
    sh = inputs.LayerShape(T=T, d=d, E=1, k=1, n_kv_heads=N // 64, head_dim=64)
    x = inputs.make_tokens(T, d, seed).to(DEV)
    w = inputs.make_dense_vproj(sh, seed).to(DEV)
    return x, w


def run_dense(x, w, path=None):
    if path is None:
        binding.set_override("dense_path", None)
    else:
        binding.set_override("dense_path", path)
    out = binding.dense_value_proj(x, w, n_kv_heads=w.shape[0] // 64, head_dim=64)
    torch.cuda.synchronize()
    binding.set_override("dense_path", None)
    return out.reshape(x.shape[0], -1)


def ref_rows(x, w, rows=None):
    xo = x.cpu().double().numpy()
    if rows is not None:
        xo = xo[rows]
    return oracle.dense_value_proj(xo, w.cpu().double().numpy())


SHAPES = [
    # T, d, N
    (1, 64, 64),
    (5, 128, 192),
    (16, 2560, 1024),
    (17, 256, 64),
    (47, 320, 128),
    (64, 2560, 1024),
    (100, 448, 320),
    (129, 2560, 1024),
    (256, 2560, 1024),
    (256, 640, 16384),
]


@pytest.mark.parametrize("T,d,N", SHAPES)
def test_dense_shapes_both_kernels(T, d, N):
    x, w = dense_inputs(T, d, N, seed=T + d + N)
    ref = ref_rows(x, w)
    outs = {}
    for path in ("skinny", "tiled"):
        say(f"dense T={T} d={d} N={N} {path}")
        outs[path] = run_dense(x, w, path)
        st = P.check_dense_output(outs[path], ref, what=f"dense/{path} T={T} d={d} N={N}")
        say(f"  {st}")


TILED = [(257, 2560, 1024), (300, 192, 320), (1000, 2560, 1024), (2049, 704, 512),
         (4096, 2560, 1024), (70000, 64, 64)]


@pytest.mark.parametrize("T,d,N", TILED)
def test_dense_tiled_shapes(T, d, N):
    x, w = dense_inputs(T, d, N, seed=T + d + N)
    say(f"dense tiled T={T} d={d} N={N}")
    out = run_dense(x, w)
    rows = None if T * d * N <= 4096 * 2560 * 1024 else P_sample(T, 2000, seed=T)
    ref = ref_rows(x, w, rows)
    g = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    say(f"  {P.check_dense_output(g, ref, what=f'dense tiled T={T}')}")


@pytest.mark.parametrize("T,d,N", [(300, 192, 320), (1000, 2560, 1024), (4096, 2560, 1024)])
def test_dense_every_tile_shape(T, d, N):
    """Each tile shape of the tiled GEMM's dense mode against the oracle, and
    the same bits from all of them (one in-order MFMA chain per output)."""
    x, w = dense_inputs(T, d, N, seed=T + N)
    ref = ref_rows(x, w)
    outs = {}
    for tile in ("256x256", "128x256", "128x128", "128x128s3", "128x128s4", "128x128w4"):
        binding.set_override("gemm_tile", tile)
        say(f"dense tile {tile}: T={T} d={d} N={N}")
        outs[tile] = run_dense(x, w, "tiled")
        binding.set_override("gemm_tile", None)
        say(f"  {P.check_dense_output(outs[tile], ref, what=f'dense tile {tile}')}")
    for tile, o in outs.items():
        assert torch.equal(o, outs["256x256"]), f"{tile} differs from 256x256"


def P_sample(T, n, seed):
    rng = np.random.default_rng(seed)
    rows = rng.choice(T, size=min(n, T), replace=False)
    return np.unique(np.concatenate([rows, [0, T - 1]]))


@pytest.mark.parametrize("name", ["decode", "prefill", "chunked", "skewed"])
def test_dense_at_workload_sizes(name):
    """Every workload's token count at the real layer shape (d=2560, N=1024)."""
    sh = inputs.WORKLOADS[name].shape
    x = inputs.make_tokens(sh.T, sh.d, inputs.WORKLOADS[name].seed).to(DEV)
    w = inputs.make_dense_vproj(sh, inputs.WORKLOADS[name].seed).to(DEV)
    say(f"dense workload {name}: T={sh.T}")
    out = binding.dense_value_proj(x, w, sh.n_kv_heads, sh.head_dim)
    torch.cuda.synchronize()
    assert out.shape == (sh.T, sh.n_kv_heads, sh.head_dim)
    out = out.reshape(sh.T, -1)
    rows = None if sh.T <= 4096 else P_sample(sh.T, 3000, seed=7)
    ref = ref_rows(x, w, rows)
    g = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    say(f"  {P.check_dense_output(g, ref, what=f'dense {name}')}")


@pytest.mark.parametrize("path,T", [("skinny", 200), ("tiled", 200), ("tiled", 3000)])
def test_dense_rows_do_not_depend_on_T(path, T):
    """A token's output row is the same bits whatever the other tokens are."""
    x, w = dense_inputs(T, 2560, 1024, seed=11)
    full = run_dense(x, w, path)
    part = run_dense(x[37:37 + T // 3].contiguous(), w, path)
    assert torch.equal(full[37:37 + T // 3], part)
    again = run_dense(x, w, path)
    assert torch.equal(full, again)


def test_dense_zero_and_empty():
    x, w = dense_inputs(40, 256, 128, seed=3)
    z = torch.zeros_like(x)
    for path in ("skinny", "tiled"):
        assert torch.count_nonzero(run_dense(z, w, path)) == 0
    empty = torch.empty(0, 256, dtype=torch.bfloat16, device=DEV)
    out = binding.dense_value_proj(empty, w, n_kv_heads=2, head_dim=64)
    assert out.shape == (0, 2, 64)


def test_dense_selector_weight_is_exact():
    """Unit-vector weight rows copy x's columns exactly (one nonzero product)."""
    T, d, N = 300, 512, 128
    x = inputs.make_tokens(T, d, 5).to(DEV)
    perm = torch.randperm(d, generator=torch.Generator().manual_seed(2))[:N]
    w = torch.zeros(N, d, dtype=torch.bfloat16)
    w[torch.arange(N), perm] = 1.0
    w = w.to(DEV)
    for path in ("skinny", "tiled"):
        if path == "skinny":
            out = run_dense(x[:256].contiguous(), w, path)
            assert torch.equal(out, x[:256][:, perm.to(DEV)])
        else:
            out = run_dense(x, w, path)
            assert torch.equal(out, x[:, perm.to(DEV)])
