"""Seeded synthetic inputs for the MoVA routed value projection.

This module only draws random tensors; it holds none of the layer's
arithmetic (no routing, no projection, no activation).  Both the HIP path's
tests/benchmark and the CPU oracle's tests take their inputs from here, so the
two sides always see identical values.

Shapes and distributions follow the layer described on the page "MoVA: routing
the value vectors, and why the KV cache does not notice" (section "Where the
routing happens": a 2560->64 router, 64 value experts of 2560 -> 8*128, top-4,
scale 2.5) and the K2-Horizon config facts quoted in its section "So what does
it cost?".  Everything is drawn on the CPU with a ``torch.Generator`` so that a
seed names the same tensors on every machine:

* x ~ N(0, 1), router W ~ N(0, 0.02), expert W ~ N(0, 1/sqrt(d)); the second
  argument of N is the standard deviation;
* router bias ~ U(-0.01, 0.01), zero, or a Zipf-shaped bias (see
  ``zipf_bias``);
* tensor order is fixed (x, router W, router bias, expert W, and the dense
  v_proj weight of the matched baseline) and each tensor has its own sub-seed
  (seed + 0 .. seed + 4); layer ``l`` of a multi-layer workload adds
  ``100 * l`` to the weight sub-seeds;
* floating values are drawn in fp32 and rounded to bf16 (round to nearest
  even) unless the workload is fp32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = [
    "LayerShape",
    "Workload",
    "WORKLOADS",
    "ZIPF_S",
    "ZIPF_BETA",
    "zipf_bias",
    "make_layer",
    "make_tokens",
    "make_router",
    "make_experts",
    "make_weights",
    "make_dense_vproj",
    "make_workload",
    "FfnShape",
    "FFN_WORKLOADS",
    "make_ffn_layer",
]

# Zipf exponent of the skewed-routing workload, and the scale of the bias that
# produces it.  The bias b_e = beta * (ln p_pi(e) - mean_e ln p) with
# p_r proportional to r^-ZIPF_S; beta was found by bisection with
# tests/golden/calibrate_zipf_bias.py (which routes with the CPU oracle only) so
# that the hottest expert draws about 10x the mean number of tokens at T=32768.
ZIPF_S = 1.1
ZIPF_BETA = 0.12890625


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Sizes of one MoVA value layer.

    T tokens of width d are routed over E experts, k of which are evaluated per
    token; each expert maps d -> n_kv_heads * head_dim.
    """

    T: int
    d: int
    E: int
    k: int
    n_kv_heads: int
    head_dim: int
    scale: float = 2.5

    @property
    def N(self) -> int:
        return self.n_kv_heads * self.head_dim


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named synthetic workload: a layer shape plus how to draw its tensors."""

    name: str
    shape: LayerShape
    dtype: torch.dtype
    bias: str  # "zero" | "uniform" | "zipf"
    seed: int = 0
    layers: int = 1
    chunks: int = 1  # the T tokens are fed as `chunks` equal calls
    description: str = ""


_LAYER = dict(d=2560, E=64, k=4, n_kv_heads=8, head_dim=128, scale=2.5)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", LayerShape(T=16, d=256, E=8, k=2, n_kv_heads=2, head_dim=32),
        torch.float32, "zero",
        description="T=16, d=256, E=8 experts 256->64 (2x32), top-2, zero bias, fp32"),
    "decode": Workload(
        "decode", LayerShape(T=64, **_LAYER), torch.bfloat16, "uniform",
        description="decode step: T=64, d=2560, E=64 experts 2560->1024 (8x128), top-4, bf16"),
    "prefill": Workload(
        "prefill", LayerShape(T=4096, **_LAYER), torch.bfloat16, "uniform",
        description="prefill chunk: T=4096, same layer, roughly uniform routing, bf16"),
    "skewed": Workload(
        "skewed", LayerShape(T=32768, **_LAYER), torch.bfloat16, "zipf",
        description="skewed prefill: T=32768, Zipf(1.1)-shaped router bias, hottest ~10x mean, bf16"),
    "chunked": Workload(
        "chunked", LayerShape(T=8192, **_LAYER), torch.bfloat16, "uniform",
        layers=4, chunks=8,
        description="long chunked prefill: 65536 tokens as 8 calls of 8192 through 4 layers, bf16"),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _round(t: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    return t if dtype == torch.float32 else t.to(dtype)


def zipf_bias(E: int, beta: float = ZIPF_BETA, s: float = ZIPF_S, seed: int = 0) -> torch.Tensor:
    """Router bias whose per-expert log-preference follows a Zipf(s) law.

    Rank r (1-based) has preference p_r proportional to r^-s; a seeded
    permutation pi assigns ranks to experts so the hot experts are not simply
    the lowest indices.  Returns fp32 [E] with zero mean.
    """
    g = _gen(seed)
    perm = torch.randperm(E, generator=g)
    ranks = torch.arange(1, E + 1, dtype=torch.float64)
    logp = -s * torch.log(ranks)
    logp = logp - torch.logsumexp(logp, 0)
    centred = logp - logp.mean()
    return (beta * centred[perm]).to(torch.float32)


def make_tokens(T: int, d: int, seed: int, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """x [T, d] ~ N(0, 1), drawn in fp32 then rounded to ``dtype``."""
    return _round(torch.randn(T, d, generator=_gen(seed)), dtype)


def make_router(shape: LayerShape, seed: int, dtype: torch.dtype = torch.bfloat16,
                bias: str = "uniform", layer: int = 0,
                zipf_beta: Optional[float] = None) -> Dict[str, torch.Tensor]:
    """Router weight [E, d] (``dtype``) and router bias [E] (fp32)."""
    E, d = shape.E, shape.d
    base = seed + 100 * layer
    router_w = _round(torch.randn(E, d, generator=_gen(base + 1)) * 0.02, dtype)
    if bias == "zero":
        router_b = torch.zeros(E, dtype=torch.float32)
    elif bias == "uniform":
        router_b = (torch.rand(E, generator=_gen(base + 2)) * 0.02 - 0.01).to(torch.float32)
    elif bias == "zipf":
        router_b = zipf_bias(E, ZIPF_BETA if zipf_beta is None else zipf_beta, seed=base + 2)
    else:
        raise ValueError(f"unknown bias kind {bias!r}")
    return {"router_w": router_w, "router_b": router_b}


def make_experts(shape: LayerShape, seed: int, dtype: torch.dtype = torch.bfloat16,
                 layer: int = 0) -> torch.Tensor:
    """Stacked expert weights [E, N, d] ~ N(0, 1/sqrt(d)).

    nn.Linear layout (out-features major, in-features contiguous), one [N, d]
    matrix per expert, bias-free.
    """
    std = 1.0 / math.sqrt(shape.d)
    g = _gen(seed + 100 * layer + 3)
    return _round(torch.randn(shape.E, shape.N, shape.d, generator=g) * std, dtype)


def make_dense_vproj(shape: LayerShape, seed: int, dtype: torch.dtype = torch.bfloat16,
                     layer: int = 0) -> torch.Tensor:
    """Plain value-projection weight [N, d] ~ N(0, 1/sqrt(d)) of a dense layer
    (nn.Linear layout, bias-free), the matched baseline of the experts; its
    own sub-seed is seed + 100 * layer + 4."""
    std = 1.0 / math.sqrt(shape.d)
    g = _gen(seed + 100 * layer + 4)
    return _round(torch.randn(shape.N, shape.d, generator=g) * std, dtype)


def make_weights(shape: LayerShape, seed: int, dtype: torch.dtype = torch.bfloat16,
                 bias: str = "uniform", layer: int = 0,
                 zipf_beta: Optional[float] = None) -> Dict[str, torch.Tensor]:
    """``make_router`` plus ``expert_w`` from ``make_experts``."""
    out = make_router(shape, seed, dtype, bias, layer, zipf_beta)
    out["expert_w"] = make_experts(shape, seed, dtype, layer)
    return out


def make_layer(shape: LayerShape, seed: int = 0, dtype: torch.dtype = torch.bfloat16,
               bias: str = "uniform", layer: int = 0,
               zipf_beta: Optional[float] = None) -> Dict[str, torch.Tensor]:
    """All tensors of one layer call: x plus ``make_weights``.  CPU tensors."""
    out = {"x": make_tokens(shape.T, shape.d, seed, dtype)}
    out.update(make_weights(shape, seed, dtype, bias, layer, zipf_beta))
    return out


def make_workload(name: str, layer: int = 0, T: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Tensors of a named workload (one layer).  ``T`` overrides the token count
    (the chunked workload's full token stream is T * chunks tokens)."""
    w = WORKLOADS[name]
    shape = w.shape if T is None else dataclasses.replace(w.shape, T=T)
    return make_layer(shape, w.seed, w.dtype, w.bias, layer)


# ---------------------------------------------------------------- FFN MoE

@dataclasses.dataclass(frozen=True)
class FfnShape:
    """Sizes of one FFN mixture-of-experts layer: T tokens of width d, E SwiGLU
    experts of intermediate width ``inter`` (k per token) and a shared expert
    of width ``inter_shared`` (0 = none)."""

    T: int
    d: int
    E: int
    k: int
    inter: int
    inter_shared: int
    scale: float = 2.5


# The pages give 100 experts with top-8 routing plus one shared expert, but no
# expert width; 768 makes the model's parameter count come out at the page's
# total (see the design notes) and is used for both expert kinds.
_FFN = dict(d=2560, E=100, k=8, inter=768, inter_shared=768)

FFN_WORKLOADS: Dict[str, FfnShape] = {
    "ffn_decode": FfnShape(T=64, **_FFN),
    "ffn_prefill": FfnShape(T=4096, **_FFN),
}


def make_ffn_layer(shape: FfnShape, seed: int = 0,
                   dtype: torch.dtype = torch.bfloat16) -> Dict[str, torch.Tensor]:
    """x [T, d] ~ N(0, 1); router W [E, d] ~ N(0, 0.02), bias ~ U(-0.01, 0.01);
    gate / up [E, inter, d] ~ N(0, 1/sqrt(d)); down [E, d, inter] ~
    N(0, 1/sqrt(inter)); the shared expert's three matrices likewise.
    Sub-seeds seed + 10 .. seed + 17.  CPU tensors (bias fp32)."""
    T, d, E, I, Is = shape.T, shape.d, shape.E, shape.inter, shape.inter_shared
    out = {
        "x": _round(torch.randn(T, d, generator=_gen(seed + 10)), dtype),
        "router_w": _round(torch.randn(E, d, generator=_gen(seed + 11)) * 0.02, dtype),
        "router_b": (torch.rand(E, generator=_gen(seed + 12)) * 0.02 - 0.01).to(torch.float32),
        "gate_w": _round(torch.randn(E, I, d, generator=_gen(seed + 13)) / math.sqrt(d), dtype),
        "up_w": _round(torch.randn(E, I, d, generator=_gen(seed + 14)) / math.sqrt(d), dtype),
        "down_w": _round(torch.randn(E, d, I, generator=_gen(seed + 15)) / math.sqrt(I), dtype),
    }
    if Is > 0:
        g = _gen(seed + 16)
        out["shared_gate_w"] = _round(torch.randn(Is, d, generator=g) / math.sqrt(d), dtype)
        out["shared_up_w"] = _round(torch.randn(Is, d, generator=g) / math.sqrt(d), dtype)
        out["shared_down_w"] = _round(torch.randn(d, Is, generator=_gen(seed + 17)) / math.sqrt(Is),
                                      dtype)
    return out
