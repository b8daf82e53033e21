"""Value projection stored into a paged value cache, vs the CPU oracle.

The pool is filled with a sentinel first.  Checks, on both execution paths
(decode weight stream and grouped GEMM):
* the pool equals ``oracle.paged_value_write`` of the oracle's values: rows
  at valid slots within the output parity rules, every other row still the
  sentinel, bit for bit;
* pool rows are bitwise the rows of the contiguous output of the same call,
  and of a plain ``mova_value_forward`` call;
* padding (-1) and out-of-pool slots store nothing; ``out`` may be omitted.
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
SENTINEL = -3.0


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu_only():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    binding.load_library()
    yield
    binding.set_override("path", None)


def make_slots(T, num_slots, seed, pad_every=7):
    """Distinct slots in random order; every pad_every-th token padded (-1),
    and two tokens past the pool (num_slots, num_slots + 5) when T >= 20."""
    rng = np.random.default_rng(seed)
    slots = rng.permutation(num_slots)[:T].astype(np.int64)
    slots[::pad_every] = -1
    if T >= 20:
        slots[3] = num_slots
        slots[11] = num_slots + 5
    return slots


def rows_of(t, idx, n):
    """t[idx] on the device after checking on the host that every index is in
    [0, n) (an out-of-range device gather faults the GPU)."""
    idx = np.asarray(idx, dtype=np.int64)
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < n), "gather index out of range"
    assert t.shape[0] == n
    return t[torch.as_tensor(idx, device=t.device)]


def run_paged(g, k, scale, H, D, pool, slots, path, with_out=True):
    binding.set_override("path", path)
    T = g["x"].shape[0]
    out = torch.empty(T, H, D, dtype=torch.bfloat16, device=DEV) if with_out else None
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    binding.value_forward_paged(g["x"], g["router_w"], g["router_b"], g["expert_w"], k, scale,
                                pool, torch.as_tensor(slots, device=DEV), out=out,
                                topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    binding.set_override("path", None)
    return out, idx, w


CASES = [
    # T, d, E, k, H, D, num_blocks, block_size, path
    (64, 2560, 64, 4, 8, 128, 12, 16, "decode"),
    (64, 2560, 64, 4, 8, 128, 12, 16, "grouped"),
    (37, 256, 16, 4, 2, 64, 5, 8, "decode"),
    (8, 2560, 64, 4, 8, 128, 12, 16, "decode"),   # token-major decode kernel (T * k <= 48)
    (3, 256, 16, 4, 2, 64, 5, 8, "decode"),
    (300, 512, 32, 4, 4, 64, 40, 16, "grouped"),
    (1000, 256, 8, 2, 1, 64, 1100, 1, "grouped"),
    (4096, 2560, 64, 4, 8, 128, 160, 32, "grouped"),
]


@pytest.mark.parametrize("T,d,E,k,H,D,nb,bs,path", CASES)
def test_paged_store_matches_oracle(T, d, E, k, H, D, nb, bs, path):
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=H, head_dim=D)
    g = P.to_gpu_inputs(inputs.make_layer(shape, T + nb, torch.bfloat16, "uniform"))
    slots = make_slots(T, nb * bs, seed=T)
    say(f"paged T={T} d={d} E={E} k={k} H={H} D={D} pool={nb}x{bs} {path}")
    pool = torch.full((nb, bs, H, D), SENTINEL, dtype=torch.bfloat16, device=DEV)
    out, idx, w = run_paged(g, k, 2.5, H, D, pool, slots, path)
    # Output parity on every token (routing rules, then values).
    st = P.full_check(g, k, 2.5, H, D, out, idx, w, what=f"paged/{path}")
    say(f"  out: {st}")
    # Pool against the oracle's paged store of the oracle's values.
    o = P.oracle_inputs(g)
    ref = oracle.route(o["x"], o["router_w"], o["router_b"], k, 2.5)
    rc = P.check_routing(idx, w, ref, 2.5)
    vals = oracle.combine_experts(o["x"], o["expert_w"], rc.effective_idx, rc.effective_w)
    want = oracle.paged_value_write(np.full((nb, bs, H, D), SENTINEL), vals.reshape(T, H, D), slots)
    got = pool.float().cpu().double().numpy()
    flat_got, flat_want = got.reshape(nb * bs, -1), want.reshape(nb * bs, -1)
    valid = slots[(slots >= 0) & (slots < nb * bs)]
    untouched = np.setdiff1d(np.arange(nb * bs), valid)
    assert np.array_equal(flat_got[untouched], flat_want[untouched]), "a row no slot names changed"
    P.check_output(torch.from_numpy(flat_got[valid]), flat_want[valid], what=f"pool/{path}")
    # Pool rows are the output rows, bit for bit.
    tok = np.nonzero((slots >= 0) & (slots < nb * bs))[0]
    pool_rows = rows_of(pool.reshape(nb * bs, -1), slots[tok], nb * bs)
    assert torch.equal(pool_rows, rows_of(out.reshape(T, -1), tok, T))
    say(f"  pool: {len(valid)} rows stored, {len(untouched)} untouched")


@pytest.mark.parametrize("path,T", [("decode", 200), ("grouped", 200), ("decode", 12)])
def test_paged_without_out_equals_plain_forward(path, T):
    d, E, k, H, D, nb, bs = 2560, 64, 4, 8, 128, 16, 16
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=H, head_dim=D)
    g = P.to_gpu_inputs(inputs.make_layer(shape, 21, torch.bfloat16, "uniform"))
    slots = make_slots(T, nb * bs, seed=4, pad_every=5)
    say(f"paged no-out T={T} {path}")
    pool = torch.full((nb, bs, H, D), SENTINEL, dtype=torch.bfloat16, device=DEV)
    run_paged(g, k, 2.5, H, D, pool, slots, path, with_out=False)
    binding.set_override("path", path)
    plain = binding.value_forward(g["x"], g["router_w"], g["router_b"], g["expert_w"], k, 2.5, H, D)
    torch.cuda.synchronize()
    binding.set_override("path", None)
    tok = np.nonzero((slots >= 0) & (slots < nb * bs))[0]
    assert torch.equal(rows_of(pool.reshape(nb * bs, -1), slots[tok], nb * bs),
                       rows_of(plain.reshape(T, -1), tok, T))
    rest = np.setdiff1d(np.arange(nb * bs), slots[tok])
    assert (rows_of(pool.reshape(nb * bs, -1), rest, nb * bs) == SENTINEL).all()


def test_paged_all_padding_and_empty():
    T, d, E, k, H, D = 50, 256, 8, 2, 2, 64
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=H, head_dim=D)
    g = P.to_gpu_inputs(inputs.make_layer(shape, 2, torch.bfloat16, "uniform"))
    pool = torch.full((4, 16, H, D), SENTINEL, dtype=torch.bfloat16, device=DEV)
    slots = np.full(T, -1, dtype=np.int64)
    slots[::2] = 64 + np.arange(0, T, 2)  # all past the 64-slot pool
    for path in ("decode", "grouped"):
        out, idx, w = run_paged(g, k, 2.5, H, D, pool, slots, path)
        assert (pool == SENTINEL).all()
        P.full_check(g, k, 2.5, H, D, out, idx, w, what=f"padding/{path}")
    empty = {kk: (v[:0].contiguous() if kk == "x" else v) for kk, v in g.items()}
    binding.value_forward_paged(empty["x"], g["router_w"], g["router_b"], g["expert_w"], k, 2.5,
                                pool, torch.empty(0, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert (pool == SENTINEL).all()
