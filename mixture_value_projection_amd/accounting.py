"""Algorithmic work of the MoVA routed value projection (host-side arithmetic).

Counts what the method must do -- k expert projections per token plus the
router -- not the dense work over all E experts that routing avoids.  The
page "MoVA: routing the value vectors, and why the KV cache does not notice",
section "So what does it cost?", gives the per-layer and per-token figures
these functions reproduce (tested): 64 * 2560 * 1024 value-expert parameters
per layer, 7,549,747,200 over 45 layers, about 10.49M multiply-accumulates
per token for four experts, a 2.62M-parameter dense v_proj and a router of
about 164K parameters.

MI355X peaks used for roofline fractions (AMD public figures): 8 TB/s HBM3E,
2.5 PFLOP/s dense bf16 MFMA.
"""
from __future__ import annotations

HBM_PEAK_BPS = 8.0e12
BF16_MFMA_PEAK_FLOPS = 2.5e15


def expert_macs_per_token(d: int, k: int, N: int) -> int:
    """k experts of d -> N each: k * d * N multiply-accumulates."""
    return k * d * N


def router_macs_per_token(d: int, E: int) -> int:
    return d * E


def router_params(d: int, E: int) -> int:
    """Router weight plus bias."""
    return d * E + E


def value_expert_params(E: int, N: int, d: int) -> int:
    """Bias-free experts: E matrices of N x d."""
    return E * N * d


def dense_vproj_params(d: int, N: int) -> int:
    return d * N


def flops_per_token(d: int, E: int, k: int, N: int) -> int:
    """2 * (expert MACs + router MACs); SiLU and the k-way sum are not counted."""
    return 2 * (expert_macs_per_token(d, k, N) + router_macs_per_token(d, E))


def bytes_per_call(T: int, touched: int, d: int, E: int, N: int, k: int,
                   export_routing: bool = False, elt: int = 2) -> int:
    """Minimum HBM bytes of one call: each touched expert's weights once, the
    router weight and fp32 bias, x in, out written; plus idx/w if exported."""
    b = touched * N * d * elt + E * d * elt + E * 4 + T * d * elt + T * N * elt
    if export_routing:
        b += T * k * 8
    return b


def expert_kernel_bytes(T: int, touched: int, d: int, N: int, elt: int = 2) -> int:
    """Algorithmic bytes of the expert stage alone: touched experts' weights
    plus the token rows it reads (router weights are read by the router)."""
    return touched * N * d * elt + T * d * elt


def roofline_seconds(flops: float, nbytes: float) -> float:
    return max(flops / BF16_MFMA_PEAK_FLOPS, nbytes / HBM_PEAK_BPS)
