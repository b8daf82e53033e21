"""The compact routing record on the GPU, against the oracle.

* mova_value_forward_record: the output equals mova_value_forward's bit for
  bit; the record equals ``oracle.pack_routing_record`` of the routing the
  call used (ids and fp16 bits exact), and that routing passes the oracle's
  routing rule;
* mova_value_from_record: equals mova_value_from_routing given the unpacked
  routing, bit for bit, and ``oracle.rebuild_from_record`` within the output
  rule; ids >= E mark unused slots.
Both expert paths (the decode kernels at T <= 256, dispatch + grouped GEMM
above) are covered.
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


def layer(T, d, E, k, heads, hd, seed):
    shape = inputs.LayerShape(T=T, d=d, E=E, k=k, n_kv_heads=heads, head_dim=hd)
    return {n: v.to(DEV) for n, v in inputs.make_layer(shape, seed, torch.bfloat16, "uniform").items()}


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


SHAPES = [
    # T, d, E, k, heads, hd
    (64, 2560, 64, 4, 8, 128),    # decode workload's layer (decode kernels)
    (4096, 2560, 64, 4, 8, 128),  # prefill chunk (grouped GEMM)
    (1, 2560, 64, 4, 8, 128),     # one token (chain kernel)
    (37, 256, 8, 2, 2, 32),       # tiny layer shape
    (300, 512, 59, 5, 4, 128),    # k = 5 (a full id word), E not a power of two
]


@pytest.mark.parametrize("T,d,E,k,heads,hd", SHAPES)
def test_forward_record_and_rebuild(T, d, E, k, heads, hd):
    g = layer(T, d, E, k, heads, hd, seed=T + 31 * k)
    say(f"record T={T} d={d} E={E} k={k} N={heads * hd}")
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    plain = binding.value_forward(g["x"], g["router_w"], g["router_b"], g["expert_w"], k, 2.5, heads,
                                  hd, topk_idx=idx, topk_w=w)
    out, ids, w16 = binding.value_forward_record(g["x"], g["router_w"], g["router_b"], g["expert_w"],
                                                 k, 2.5, heads, hd)
    torch.cuda.synchronize()
    assert same(out, plain), "the record variant changed the output"
    want_ids, want_w16 = oracle.pack_routing_record(idx.cpu().numpy(), w.cpu().double().numpy())
    np.testing.assert_array_equal(ids.cpu().numpy().view(np.uint32), want_ids)
    np.testing.assert_array_equal(w16.cpu().numpy().view(np.uint16), want_w16.view(np.uint16))
    o = P.oracle_inputs(g)
    ref = oracle.route(o["x"], o["router_w"], o["router_b"], k, 2.5)
    ridx, _ = oracle.unpack_routing_record(ids.cpu().numpy().view(np.uint32), w16.cpu().numpy(), k)
    P.check_routing(ridx, w.cpu(), ref, 2.5)
    # Rebuild from the record: the same bits as the rebuild from the unpacked
    # routing, and the oracle's rebuild from the record.
    reb = binding.value_from_record(g["x"], ids, w16, g["expert_w"], heads, hd)
    reb2 = binding.value_from_routing(g["x"], torch.as_tensor(ridx, dtype=torch.int32, device=DEV),
                                      w16.float().contiguous(), g["expert_w"], heads, hd)
    torch.cuda.synchronize()
    assert same(reb, reb2)
    rows = np.arange(T) if T <= 512 else np.sort(np.random.default_rng(T).choice(T, 512, replace=False))
    want = oracle.rebuild_from_record(o["x"][rows], o["expert_w"], ids.cpu().numpy().view(np.uint32)[rows],
                                      w16.cpu().numpy()[rows], k)
    st = P.check_output(reb.reshape(T, -1)[torch.as_tensor(rows, device=DEV)], want, f"rebuild T={T}")
    say(f"  record exact; rebuild bitwise equal to the routing rebuild; oracle {st}")


def test_record_with_unused_slots():
    """An id >= E (E < 64) marks an unused slot; a zero weight adds nothing."""
    T, d, E, k, heads, hd = 50, 512, 40, 4, 4, 128
    g = layer(T, d, E, k, heads, hd, seed=7)
    rng = np.random.default_rng(7)
    idx = rng.integers(0, E, size=(T, k))
    idx[::3, 1] = 63       # unused (>= E)
    idx[::5, 2] = E        # unused (== E)
    w = rng.uniform(0.1, 1.0, size=(T, k))
    w[::7, 0] = 0.0        # zero weight
    ids, w16 = oracle.pack_routing_record(idx, w)
    out = binding.value_from_record(g["x"], torch.as_tensor(ids.view(np.int32), device=DEV),
                                    torch.as_tensor(w16, device=DEV), g["expert_w"], heads, hd)
    torch.cuda.synchronize()
    o = P.oracle_inputs(g)
    want = oracle.rebuild_from_record(o["x"], o["expert_w"], ids, w16, k)
    st = P.check_output(out.reshape(T, -1), want, "record with unused slots")
    say(f"record with unused slots: {st}")
