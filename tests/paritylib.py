"""Acceptance rules for comparing the HIP path with the CPU oracle.

Indices, per token (ids and scores are the oracle's float64 selection
scores sel = sigmoid(logit) + bias):
* the k ids are distinct and in [0, E);
* a token whose oracle margin (k-th minus (k+1)-th selection score) exceeds
  MARGIN must choose the oracle's set exactly;
* a token at or below MARGIN is a near tie: a set S is valid when no expert
  left out scores more than MARGIN above the lowest chosen one, i.e.
  min_{e in S} sel_e >= max_{e not in S} sel_e - MARGIN; the token's output
  is then compared with the oracle recomputed on the GPU's choice;
* order: the k ids are reported by (selection score desc, index asc), so on
  every token no id may score more than MARGIN above an id reported before
  it, and ids whose oracle scores are exactly equal come in increasing
  index order.  Where adjacent scores differ by more than MARGIN this fixes
  the oracle's order exactly.

Weights: |w_gpu - w_oracle| <= W_TOL for each matched expert, and the k
weights sum to the scale within W_TOL.

Outputs (bf16): max |gpu - oracle| <= MAX_ABS and
||gpu - oracle||_2 / ||oracle||_2 <= REL_L2 over all compared elements.

Dense value projection (one fp32 sum per output, rounded once to bf16): on
top of the two output rules, every element is within half a bf16 step of the
oracle (|gpu - oracle| <= 2^-8 |oracle| + DENSE_ATOL, DENSE_ATOL covering the
fp32 accumulation), and at least DENSE_MATCH of the elements equal the
oracle's value rounded to bf16 (they differ only where the fp32 sum lands on
the other side of a rounding midpoint).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

import oracle

MARGIN = 1e-4
W_TOL = 1e-4
MAX_ABS = 2e-2
REL_L2 = 5e-3
DENSE_ATOL = 1e-3
DENSE_MATCH = 0.99


@dataclasses.dataclass
class RouteCheck:
    near_ties: int
    differing_sets: int
    effective_idx: np.ndarray
    effective_w: np.ndarray


def check_routing(gpu_idx, gpu_w, ref: oracle.Routing, scale: float, tokens=None) -> RouteCheck:
    """Apply the index / weight rules; returns the routing the output check uses.

    ``tokens`` (optional) names which oracle rows the GPU rows correspond to.
    """
    gi = np.asarray(gpu_idx.cpu() if hasattr(gpu_idx, "cpu") else gpu_idx).astype(np.int64)
    gw = np.asarray(gpu_w.cpu() if hasattr(gpu_w, "cpu") else gpu_w).astype(np.float64)
    rows = np.arange(gi.shape[0]) if tokens is None else np.asarray(tokens)
    T, k = gi.shape
    E = ref.sel.shape[1]
    assert ((gi >= 0) & (gi < E)).all(), "expert index out of range"
    srt = np.sort(gi, axis=1)
    rep = np.nonzero((srt[:, 1:] == srt[:, :-1]).any(axis=1))[0] if k > 1 else np.zeros(0, int)
    assert rep.size == 0, f"token {rows[rep[0]]}: repeated expert in {gi[rep[0]]}"
    np.testing.assert_allclose(gw.sum(axis=1), scale, atol=W_TOL, rtol=0)
    assert (gw > 0).all()

    ref_idx = ref.idx[rows]
    margin = ref.margin[rows]
    sel = ref.sel[rows]
    s = ref.s[rows]
    clear = margin > MARGIN
    same_set = (srt == np.sort(ref_idx, axis=1)).all(axis=1)
    bad = np.nonzero(clear & ~same_set)[0]
    assert bad.size == 0, (f"{bad.size} tokens with margin > {MARGIN} chose other experts; "
                           f"first: row {rows[bad[0]]} gpu {gi[bad[0]]} oracle {ref_idx[bad[0]]} "
                           f"margin {margin[bad[0]]:.3e}")
    # Near ties: no expert left out may beat the lowest chosen one by more
    # than MARGIN.
    chosen_sel = np.take_along_axis(sel, gi, axis=1)
    left_out = np.ones(sel.shape, dtype=bool)
    np.put_along_axis(left_out, gi, False, axis=1)
    best_left = np.where(left_out, sel, -np.inf).max(axis=1) if k < E else np.full(T, -np.inf)
    far = np.nonzero(chosen_sel.min(axis=1) < best_left - MARGIN)[0]
    assert far.size == 0, (f"row {rows[far[0]]}: chose {gi[far[0]]} (lowest score "
                           f"{chosen_sel[far[0]].min():.6f}) over an expert scoring "
                           f"{best_left[far[0]]:.6f}")
    # Order: (score desc, index asc), up to MARGIN between the scores.
    for a in range(k):
        for b in range(a + 1, k):
            inv = chosen_sel[:, b] > chosen_sel[:, a] + MARGIN
            tie_inv = (chosen_sel[:, b] == chosen_sel[:, a]) & (gi[:, b] < gi[:, a])
            wrong = np.nonzero(inv | tie_inv)[0]
            assert wrong.size == 0, (f"row {rows[wrong[0]]}: experts reported as {gi[wrong[0]]}, "
                                     f"not by (score desc, index asc); scores "
                                     f"{chosen_sel[wrong[0]]}")
    # Weights recomputed by the oracle's rule for the GPU's set.
    chosen_s = np.take_along_axis(s, gi, axis=1)
    w_for_gpu_set = scale * chosen_s / chosen_s.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(gw, w_for_gpu_set, atol=W_TOL, rtol=0)
    return RouteCheck(near_ties=int((~clear).sum()), differing_sets=int((~same_set).sum()),
                      effective_idx=gi, effective_w=w_for_gpu_set)


def check_output(gpu_out, ref_out, what: str = "") -> dict:
    g = gpu_out.float().cpu().double().numpy().reshape(ref_out.shape[0], -1) \
        if hasattr(gpu_out, "float") else np.asarray(gpu_out, dtype=np.float64).reshape(ref_out.shape[0], -1)
    r = np.asarray(ref_out, dtype=np.float64).reshape(ref_out.shape[0], -1)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - r)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(g - r) / denom) if denom > 0 else float(np.linalg.norm(g))
    assert max_abs <= MAX_ABS, f"{what}: max abs error {max_abs:.4g} > {MAX_ABS}"
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.4g} > {REL_L2}"
    return {"max_abs": max_abs, "rel_l2": rel, "max_ref": float(np.abs(r).max()) if r.size else 0.0}


def to_gpu_inputs(layer: dict, device="cuda") -> dict:
    """bf16 device copies (fp32 tensors are rounded to bf16, as the GPU path is bf16)."""
    out = {}
    for key in ("x", "router_w", "expert_w"):
        out[key] = layer[key].to(torch.bfloat16).to(device).contiguous()
    out["router_b"] = None if layer.get("router_b") is None else \
        layer["router_b"].to(torch.float32).to(device).contiguous()
    return out


def oracle_inputs(gpu_inputs: dict) -> dict:
    """The exact values the GPU sees, upcast to float64 on the CPU."""
    return {k: (None if v is None else v.cpu().double().numpy()) for k, v in gpu_inputs.items()}


def full_check(gpu_inputs: dict, k: int, scale: float, H: int, D: int, out, idx, w,
               tokens: Optional[np.ndarray] = None, ref: Optional[oracle.Routing] = None,
               what: str = "") -> dict:
    """Routing rule on all rows, output rule on ``tokens`` (all rows if None)."""
    o = oracle_inputs(gpu_inputs)
    if ref is None:
        ref = oracle.route(o["x"], o["router_w"], o["router_b"], k, scale)
    rc = check_routing(idx, w, ref, scale)
    rows = np.arange(o["x"].shape[0]) if tokens is None else np.asarray(tokens)
    ref_out = oracle.combine_experts(o["x"][rows], o["expert_w"], rc.effective_idx[rows],
                                     rc.effective_w[rows])
    g = out.reshape(out.shape[0], -1)[torch.as_tensor(rows, device=out.device)]
    stats = check_output(g, ref_out, what)
    stats.update(near_ties=rc.near_ties, differing_sets=rc.differing_sets)
    return stats


def check_dense_output(gpu_out, ref_out, what: str = "") -> dict:
    """The dense projection's rules (module docstring) on [rows, N] outputs."""
    stats = check_output(gpu_out, ref_out, what)
    g = gpu_out.float().cpu().double().numpy().reshape(ref_out.shape[0], -1)
    r = np.asarray(ref_out, dtype=np.float64).reshape(ref_out.shape[0], -1)
    excess = np.abs(g - r) - (2.0 ** -8) * np.abs(r)
    worst = float(excess.max()) if excess.size else 0.0
    assert worst <= DENSE_ATOL, f"{what}: an element is {worst:.3g} beyond half a bf16 step"
    rb = torch.from_numpy(r).to(torch.bfloat16).double().numpy()
    match = float((g == rb).mean()) if g.size else 1.0
    assert match >= DENSE_MATCH, f"{what}: only {match:.4f} of elements equal bf16(oracle)"
    stats.update(bf16_match=match)
    return stats
