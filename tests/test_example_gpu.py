"""The C example (examples/value_forward.c, built next to the library by
build()): a plain C program calls mova_workspace_bytes and
mova_value_forward through the C ABI and writes its inputs and results;
the same inputs through the Python binding give the same bits."""
import os
import subprocess

import numpy as np
import pytest
import torch

from mixture_value_projection_amd import binding, build

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_c_example_matches_binding(tmp_path):
    exe = build.EXAMPLE
    assert os.path.exists(exe), "the C example is compiled by build()"
    path = tmp_path / "run.bin"
    print("c example", flush=True)
    r = subprocess.run([exe, str(path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("mova "), r.stdout
    raw = path.read_bytes()
    T, d, E, k, H, D = np.frombuffer(raw, dtype=np.int32, count=6).tolist()
    N = H * D
    off = 24

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=off).copy()
        off += a.nbytes
        return a

    bf16 = lambda a, shape: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).reshape(shape)
    x = bf16(take(np.uint16, T * d), (T, d))
    rw = bf16(take(np.uint16, E * d), (E, d))
    rb = torch.from_numpy(take(np.float32, E))
    ew = bf16(take(np.uint16, E * N * d), (E, N, d))
    out_c = take(np.uint16, T * N)
    idx_c = take(np.int32, T * k)
    w_c = take(np.float32, T * k)
    assert off == len(raw)

    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    out = binding.value_forward(x.to(DEV), rw.to(DEV), rb.to(DEV), ew.to(DEV), k, 2.5, H, D,
                                topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().view(torch.int16).numpy().reshape(-1).view(np.uint16), out_c)
    assert np.array_equal(idx.cpu().numpy().reshape(-1), idx_c)
    assert np.array_equal(w.cpu().numpy().reshape(-1), w_c)
