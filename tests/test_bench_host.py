"""Host-side checks of bench.py's result assembly (no GPU): the secondary
line builders accept the result dicts each workload runner produces."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixture_value_projection_amd import inputs  # noqa: E402


def test_prefill_line_single_layer_and_chunked():
    sh = inputs.WORKLOADS["prefill"].shape
    single = dict(shape=sh, seconds=1e-3, tokens=sh.T * 5, calls=5, stage_ms=0.15,
                  stage_records=5, graph_seconds=1e-3, graph_calls=5, touched=64, max_load=300,
                  mean_load=256.0, max_abs_out=3.0)
    d = bench.prefill_line("prefill", single)
    assert d["tokens_per_s"] > 0 and 0 < d["frac_bf16_peak"] < 1
    shc = inputs.WORKLOADS["chunked"].shape
    chunked = dict(shape=shc, seconds=1e-2, tokens=shc.T * 8 * 2, layer_tokens=shc.T * 8 * 4 * 2,
                   calls=64, stage_ms=0.24, stage_records=64, graph_seconds=1e-2, graph_calls=64,
                   graph_tokens=shc.T * 8 * 2, graph_layer_tokens=shc.T * 8 * 4 * 2)
    d = bench.prefill_line("chunked", chunked)
    assert d["tflops"] > 0


def test_dense_line():
    r = dict(T=4096, d=2560, N=1024, us=30.0, kernel_us=29.0, launches_timed=64,
             hipblaslt_us=30.0)
    d = bench.dense_line("prefill", r, 200.0)
    assert d["mova_over_dense"] == pytest.approx(200.0 / 30.0)
    assert 0 < d["dense_frac_bf16_peak"] < 1
