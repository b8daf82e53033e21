"""Benchmark of the MoVA routed value projection on one MI355X.

A step is one mova_value_forward call (router, dispatch, expert projection,
combine) on one batch of seeded synthetic tokens with inputs already resident
in HBM.  The headline workload is the decode step (T=64, d=2560, 64 experts
of 2560->1024, top-4, bf16); the prefill workloads (T=4096 chunk, T=32768
skewed, 8x8192 chunked through 4 layers) are measured as secondary lines in
the same JSON object unless --headline-only is given, and so is the matched
dense GQA v_proj (one 2560->1024 weight, no routing) at each workload's
token count, with the MoVA / dense time ratio.

Layer weights are rotated over several copies (>= 1.3 GB in total) so the
256 MB Infinity Cache cannot serve them between steps.

Prints ONE JSON line.  Algorithmic work: 2*(k*d*N + d*E) FLOP per token;
bytes = touched experts' weights once + router weights + x + out.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from mixture_value_projection_amd import accounting, binding, inputs  # noqa: E402

METRIC = "MoVA value-proj tokens/sec + % bf16 MFMA peak (prefill) / % HBM BW (decode)"
DEV = "cuda:0"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_copies(shape, seed, dtype, bias, n_copies, layer=0):
    """n_copies device copies of one layer's weights (same values, distinct memory)."""
    w = inputs.make_weights(shape, seed, dtype, bias, layer)
    base = {k: v.to(DEV) for k, v in w.items()}
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(n_copies - 1)]
    return copies


def timed_calls(calls, steps, warmup, stage):
    """Run warmup + steps calls; returns (seconds for the steps, stage ms avg)."""
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    binding.timing_enable(steps * 64, stages=(stage,))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rec = binding.timing_read()
    binding.timing_enable(0)
    tot, cnt = rec[binding.STAGES.index(stage)]
    return t1 - t0, (tot / cnt if cnt else float("nan")), cnt


# Every measured line replays a HIP graph at least REPLAYS times and reports
# the median replay; a replay runs at least MIN_CALLS // REPLAYS calls (so a
# line times at least MIN_CALLS calls whatever --steps is).
REPLAYS = 5
MIN_CALLS = 64


def graph_time(calls, warmup, per_graph=None, replays=REPLAYS):
    """Capture ``per_graph`` calls (cycling through ``calls``) into one HIP
    graph and replay it ``replays`` times, each replay bracketed by device
    synchronisation; returns (median seconds of one replay, per_graph).
    Inputs, outputs and workspaces are preallocated, so the captured work is
    exactly the eager work.  Default per_graph: a multiple of len(calls) of at
    least MIN_CALLS / replays calls."""
    if per_graph is None:
        want = max(len(calls), -(-MIN_CALLS // replays))
        per_graph = len(calls) * -(-want // len(calls))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(max(1, warmup)):
            calls[i % len(calls)]()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            calls[i % len(calls)]()
    g.replay()  # untimed: first replay
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    del g
    return float(np.median(times)), per_graph


def run_single_layer(name, steps, warmup, copies, T=None, graph_calls=None):
    """One layer of a named workload (T overrides its token count): `steps`
    eager calls with stage events (the expert kernel's launch time), then the
    median of REPLAYS graph replays of `graph_calls` calls (default: at least
    MIN_CALLS / REPLAYS)."""
    w = inputs.WORKLOADS[name]
    sh = w.shape if T is None else dataclasses.replace(w.shape, T=T)
    x = inputs.make_tokens(sh.T, sh.d, w.seed, w.dtype).to(DEV)
    cps = make_copies(sh, w.seed, w.dtype, w.bias, copies)
    out = torch.empty(sh.T, sh.n_kv_heads, sh.head_dim, dtype=torch.bfloat16, device=DEV)
    idx = torch.empty(sh.T, sh.k, dtype=torch.int32, device=DEV)
    ws = torch.empty(binding.workspace_bytes(sh.T, sh.d, sh.E, sh.k, sh.n_kv_heads, sh.head_dim),
                     dtype=torch.uint8, device=DEV)
    binding.value_forward(x, cps[0]["router_w"], cps[0]["router_b"], cps[0]["expert_w"], sh.k,
                          sh.scale, sh.n_kv_heads, sh.head_dim, out=out, topk_idx=idx, workspace=ws)
    torch.cuda.synchronize()
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=sh.E)
    touched = int((counts > 0).sum())
    max_abs_out = float(out.float().abs().max())  # the parity budget assumes |out| < 8

    def mk(c):
        return lambda: binding.value_forward(x, c["router_w"], c["router_b"], c["expert_w"], sh.k,
                                             sh.scale, sh.n_kv_heads, sh.head_dim, out=out,
                                             workspace=ws)
    calls = [mk(c) for c in cps]
    secs, stage_ms, nrec = timed_calls(calls, steps, warmup, "experts")
    gsecs, gcalls = graph_time(calls, warmup, per_graph=graph_calls)
    tokens = sh.T * steps
    return dict(shape=sh, seconds=secs, tokens=tokens, calls=steps, stage_ms=stage_ms,
                stage_records=nrec, graph_seconds=gsecs, graph_calls=gcalls,
                touched=touched, max_load=int(counts.max()), mean_load=float(counts.mean()),
                max_abs_out=max_abs_out)


def run_tp_shard(name, tp, steps, warmup):
    """One GPU's share of a workload under tensor parallelism over the KV
    heads: the router replicated, every expert's rows for heads [0, 8 / tp)
    (N = 1024 / tp), the workload's real T.  Weight copies are rotated so that
    together they exceed twice the 256 MB Infinity Cache."""
    w = inputs.WORKLOADS[name]
    sh = w.shape
    heads = sh.n_kv_heads // tp
    N = heads * sh.head_dim
    x = inputs.make_tokens(sh.T, sh.d, w.seed, w.dtype).to(DEV)
    full = inputs.make_weights(sh, w.seed, w.dtype, w.bias)
    base = {"router_w": full["router_w"].to(DEV), "router_b": full["router_b"].to(DEV),
            "expert_w": full["expert_w"][:, :N, :].contiguous().to(DEV)}
    del full
    shard_bytes = base["expert_w"].numel() * 2
    copies = max(4, -(-2 * 256 * 2**20 // shard_bytes))
    cps = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
    out = torch.empty(sh.T, heads, sh.head_dim, dtype=torch.bfloat16, device=DEV)
    idx = torch.empty(sh.T, sh.k, dtype=torch.int32, device=DEV)
    ws = torch.empty(binding.workspace_bytes(sh.T, sh.d, sh.E, sh.k, heads, sh.head_dim),
                     dtype=torch.uint8, device=DEV)
    binding.value_forward(x, base["router_w"], base["router_b"], base["expert_w"], sh.k, sh.scale,
                          heads, sh.head_dim, out=out, topk_idx=idx, workspace=ws)
    torch.cuda.synchronize()
    touched = int((np.bincount(idx.cpu().numpy().ravel(), minlength=sh.E) > 0).sum())
    calls = [(lambda c=c: binding.value_forward(x, c["router_w"], c["router_b"], c["expert_w"],
                                                sh.k, sh.scale, heads, sh.head_dim, out=out,
                                                workspace=ws)) for c in cps]
    gsecs, gcalls = graph_time(calls, warmup)
    us = 1e6 * gsecs / gcalls
    del cps, calls
    d = {"tp": tp, "workload": name, "T": sh.T, "n_kv_heads": heads, "N": N, "weight_copies": copies,
         "us_per_call": us, "tokens_per_s": sh.T / (us * 1e-6)}
    if name == "decode":
        nbytes = touched * N * sh.d * 2 + sh.T * sh.d * 2
        d["GB_per_s"] = nbytes / (us * 1e-6) / 1e9
        d["frac_hbm"] = nbytes / (us * 1e-6) / accounting.HBM_PEAK_BPS
    else:
        flops = 2.0 * sh.T * (sh.k * sh.d * N + sh.d * sh.E)
        d["tflops"] = flops / (us * 1e-6) / 1e12
        d["frac_bf16_peak"] = flops / (us * 1e-6) / accounting.BF16_MFMA_PEAK_FLOPS
    return d


def run_ep_shard(name, ep, steps, warmup):
    """One GPU's share of a workload under expert parallelism: experts
    [0, E / ep) with the routing the replicated router chose, every slot on
    another GPU's expert marked unused (-1).  mova_value_from_routing then
    runs only this GPU's pairs and writes its partial sums [T, N], the input
    of the reduce-scatter that would combine the GPUs' shares."""
    w = inputs.WORKLOADS[name]
    sh = w.shape
    e_local = sh.E // ep
    x = inputs.make_tokens(sh.T, sh.d, w.seed, w.dtype).to(DEV)
    full = inputs.make_weights(sh, w.seed, w.dtype, w.bias)
    rw, rb = full["router_w"].to(DEV), full["router_b"].to(DEV)
    base = full["expert_w"][:e_local].contiguous().to(DEV)
    del full
    shard_bytes = base.numel() * 2
    copies = max(4, -(-2 * 256 * 2**20 // shard_bytes))
    cps = [base] + [base.clone() for _ in range(copies - 1)]
    idx, wts = binding.route(x, rw, rb, sh.k, sh.scale)
    local = torch.where(idx < e_local, idx, torch.full_like(idx, -1)).contiguous()
    pairs = int((local >= 0).sum())
    touched = int(torch.unique(local[local >= 0]).numel())
    out = torch.empty(sh.T, sh.n_kv_heads, sh.head_dim, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(binding.workspace_bytes(sh.T, sh.d, e_local, sh.k, sh.n_kv_heads, sh.head_dim),
                     dtype=torch.uint8, device=DEV)
    calls = [(lambda c=c: binding.value_from_routing(x, local, wts, c, sh.n_kv_heads, sh.head_dim,
                                                     out=out, workspace=ws)) for c in cps]
    gsecs, gcalls = graph_time(calls, warmup)
    us = 1e6 * gsecs / gcalls
    del cps, calls
    d = {"ep": ep, "workload": name, "T": sh.T, "experts": e_local, "local_pairs": pairs,
         "weight_copies": copies, "us_per_call": us}
    if name == "decode":
        nbytes = touched * sh.N * sh.d * 2 + sh.T * sh.d * 2
        d["GB_per_s"] = nbytes / (us * 1e-6) / 1e9
        d["frac_hbm"] = nbytes / (us * 1e-6) / accounting.HBM_PEAK_BPS
    else:
        flops = 2.0 * pairs * sh.d * sh.N
        d["tflops"] = flops / (us * 1e-6) / 1e12
        d["frac_bf16_peak"] = flops / (us * 1e-6) / accounting.BF16_MFMA_PEAK_FLOPS
    return d


def run_paged_decode(steps, warmup, copies, block_size=16, num_blocks=4096):
    """The decode step with its value rows stored straight into a paged pool
    (num_blocks x block_size slots of [8, 128] bf16, 128 MB) at distinct
    random slots, no contiguous output."""
    w = inputs.WORKLOADS["decode"]
    sh = w.shape
    x = inputs.make_tokens(sh.T, sh.d, w.seed, w.dtype).to(DEV)
    cps = make_copies(sh, w.seed, w.dtype, w.bias, copies)
    pool = torch.zeros(num_blocks, block_size, sh.n_kv_heads, sh.head_dim, dtype=torch.bfloat16,
                       device=DEV)
    g = torch.Generator().manual_seed(5)
    slots = torch.randperm(num_blocks * block_size, generator=g)[:sh.T].to(DEV)
    ws = torch.empty(binding.workspace_bytes(sh.T, sh.d, sh.E, sh.k, sh.n_kv_heads, sh.head_dim),
                     dtype=torch.uint8, device=DEV)

    def mk(c):
        return lambda: binding.value_forward_paged(x, c["router_w"], c["router_b"], c["expert_w"],
                                                   sh.k, sh.scale, pool, slots, workspace=ws)
    calls = [mk(c) for c in cps]
    gsecs, gcalls = graph_time(calls, warmup)
    # Unfused reference: the plain forward, then a separate scatter of the
    # contiguous rows into the pool (torch index_copy_).
    out = torch.empty(sh.T, sh.n_kv_heads, sh.head_dim, dtype=torch.bfloat16, device=DEV)
    flat = pool.view(num_blocks * block_size, sh.N)

    def mk2(c):
        def f():
            binding.value_forward(x, c["router_w"], c["router_b"], c["expert_w"], sh.k, sh.scale,
                                  sh.n_kv_heads, sh.head_dim, out=out, workspace=ws)
            flat.index_copy_(0, slots, out.view(sh.T, sh.N))
        return f
    usecs, ucalls = graph_time([mk2(c) for c in cps], warmup)
    return 1e6 * gsecs / gcalls, 1e6 * usecs / ucalls


def run_rebuild(name, steps, warmup, copies):
    """Values of the workload's tokens rebuilt from stored x_t and their
    compact routing records (mova_value_from_record), as a compact cache that
    keeps x_t and the record instead of v_t would have to at attention time;
    also the forward that writes the records (mova_value_forward_record)
    against the plain forward.  Returns (rebuild us, record-writing forward
    us, plain forward us)."""
    w = inputs.WORKLOADS[name]
    sh = w.shape
    x = inputs.make_tokens(sh.T, sh.d, w.seed, w.dtype).to(DEV)
    cps = make_copies(sh, w.seed, w.dtype, w.bias, copies)
    out = torch.empty(sh.T, sh.n_kv_heads, sh.head_dim, dtype=torch.bfloat16, device=DEV)
    ids = torch.empty(sh.T, dtype=torch.int32, device=DEV)
    w16 = torch.empty(sh.T, sh.k, dtype=torch.float16, device=DEV)
    ws = torch.empty(binding.workspace_bytes(sh.T, sh.d, sh.E, sh.k, sh.n_kv_heads, sh.head_dim),
                     dtype=torch.uint8, device=DEV)
    binding.value_forward_record(x, cps[0]["router_w"], cps[0]["router_b"], cps[0]["expert_w"],
                                 sh.k, sh.scale, sh.n_kv_heads, sh.head_dim, out=out,
                                 record_ids=ids, record_w=w16, workspace=ws)
    calls = [(lambda c=c: binding.value_from_record(x, ids, w16, c["expert_w"], sh.n_kv_heads,
                                                    sh.head_dim, out=out, workspace=ws))
             for c in cps]
    gsecs, gcalls = graph_time(calls, warmup)
    rec = [(lambda c=c: binding.value_forward_record(
        x, c["router_w"], c["router_b"], c["expert_w"], sh.k, sh.scale, sh.n_kv_heads, sh.head_dim,
        out=out, record_ids=ids, record_w=w16, workspace=ws)) for c in cps]
    rsecs, rcalls = graph_time(rec, warmup)
    plain = [(lambda c=c: binding.value_forward(
        x, c["router_w"], c["router_b"], c["expert_w"], sh.k, sh.scale, sh.n_kv_heads, sh.head_dim,
        out=out, workspace=ws)) for c in cps]
    psecs, pcalls = graph_time(plain, warmup)
    return 1e6 * gsecs / gcalls, 1e6 * rsecs / rcalls, 1e6 * psecs / pcalls


def run_ffn(name, steps, warmup, copies=2):
    """The FFN mixture of experts (100 SwiGLU experts of width 768, top-8, one
    shared expert) at a workload's token count; expert weights rotated over
    `copies` device copies (1.2 GB each)."""
    sh = inputs.FFN_WORKLOADS[name]
    L = inputs.make_ffn_layer(sh, 0)
    x = L["x"].to(DEV)
    layers = []
    for c in range(copies):
        g = {k: v.to(DEV) for k, v in L.items() if k != "x"}
        g["gate_up_w"] = binding.ffn_pack_gate_up(g.pop("gate_w"), g.pop("up_w"))
        g["shared_gate_up_w"] = binding.ffn_pack_gate_up(g.pop("shared_gate_w"),
                                                         g.pop("shared_up_w"))
        layers.append(g)
    out = torch.empty(sh.T, sh.d, dtype=torch.bfloat16, device=DEV)
    idx = torch.empty(sh.T, sh.k, dtype=torch.int32, device=DEV)
    ws = torch.empty(binding.ffn_workspace_bytes(sh.T, sh.d, sh.E, sh.k, sh.inter, sh.inter_shared),
                     dtype=torch.uint8, device=DEV)
    binding.ffn_moe_forward(x, layers[0]["router_w"], layers[0]["router_b"],
                            layers[0]["gate_up_w"], layers[0]["down_w"], sh.k, sh.scale,
                            layers[0]["shared_gate_up_w"], layers[0]["shared_down_w"], out=out,
                            topk_idx=idx, workspace=ws)
    torch.cuda.synchronize()
    touched = int((np.bincount(idx.cpu().numpy().ravel(), minlength=sh.E) > 0).sum())
    calls = [(lambda g=g: binding.ffn_moe_forward(
        x, g["router_w"], g["router_b"], g["gate_up_w"], g["down_w"], sh.k, sh.scale,
        g["shared_gate_up_w"], g["shared_down_w"], out=out, workspace=ws)) for g in layers]
    gsecs, gcalls = graph_time(calls, warmup)
    us = 1e6 * gsecs / gcalls
    flops = 2.0 * sh.T * (3 * sh.d * (sh.k * sh.inter + sh.inter_shared) + sh.d * sh.E)
    wbytes = 2.0 * 3 * sh.d * (touched * sh.inter + sh.inter_shared) + 2.0 * sh.E * sh.d
    del layers, calls
    return {"workload": name, "T": sh.T, "d": sh.d, "E": sh.E, "k": sh.k, "inter": sh.inter,
            "inter_shared": sh.inter_shared, "touched_experts": touched, "us_per_call": us,
            "tokens_per_s": sh.T / (us * 1e-6), "tflops": flops / (us * 1e-6) / 1e12,
            "frac_bf16_peak": flops / (us * 1e-6) / accounting.BF16_MFMA_PEAK_FLOPS,
            "weight_GB_per_s": wbytes / (us * 1e-6) / 1e9,
            "frac_hbm_weights": wbytes / (us * 1e-6) / accounting.HBM_PEAK_BPS}


def run_chunked(steps, warmup):
    """One step = the whole 65536-token stream through 4 layers (32 calls)."""
    w = inputs.WORKLOADS["chunked"]
    sh = w.shape
    total = sh.T * w.chunks
    x = inputs.make_tokens(total, sh.d, w.seed, w.dtype).to(DEV)
    layers = [make_copies(sh, w.seed, w.dtype, w.bias, 1, layer=l)[0] for l in range(w.layers)]
    outs = [torch.empty(total, sh.n_kv_heads, sh.head_dim, dtype=torch.bfloat16, device=DEV)
            for _ in range(w.layers)]
    ws = torch.empty(binding.workspace_bytes(sh.T, sh.d, sh.E, sh.k, sh.n_kv_heads, sh.head_dim),
                     dtype=torch.uint8, device=DEV)

    def step():
        for c in range(w.chunks):
            s = slice(c * sh.T, (c + 1) * sh.T)
            for l, L in enumerate(layers):
                binding.value_forward(x[s], L["router_w"], L["router_b"], L["expert_w"], sh.k,
                                      sh.scale, sh.n_kv_heads, sh.head_dim, out=outs[l][s],
                                      workspace=ws)
    secs, stage_ms, nrec = timed_calls([step], steps, warmup, "experts")
    gsecs, gsteps = graph_time([step], warmup, per_graph=2)  # 64 calls per replay
    return dict(shape=sh, seconds=secs, tokens=total * steps, layer_tokens=total * w.layers * steps,
                calls=steps * w.chunks * w.layers, stage_ms=stage_ms, stage_records=nrec,
                graph_seconds=gsecs, graph_calls=gsteps * w.chunks * w.layers,
                graph_tokens=total * gsteps, graph_layer_tokens=total * w.layers * gsteps)


def run_dense(name, steps, warmup, copies=64):
    """The matched dense v_proj (one [N, d] weight) at a workload's token count.

    The weight is rotated over `copies` device copies (64 x 5.2 MB > the 256 MB
    Infinity Cache), as a model's other layers would evict it between calls.
    hipBLASLt (torch.matmul) on the same operands is timed beside it as a
    library reference."""
    w = inputs.WORKLOADS[name]
    sh = w.shape
    x = inputs.make_tokens(sh.T, sh.d, w.seed, w.dtype).to(DEV)
    base = inputs.make_dense_vproj(sh, w.seed, w.dtype).to(DEV)
    wts = [base] + [base.clone() for _ in range(copies - 1)]
    out = torch.empty(sh.T, sh.n_kv_heads, sh.head_dim, dtype=torch.bfloat16, device=DEV)
    wsb = binding.dense_workspace_bytes(sh.T, sh.d, sh.n_kv_heads, sh.head_dim)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV)
    calls = [(lambda wt=wt: binding.dense_value_proj(x, wt, sh.n_kv_heads, sh.head_dim, out=out,
                                                     workspace=ws)) for wt in wts]
    n = max(steps, copies)
    secs, stage_ms, nrec = timed_calls(calls, n, warmup, "dense")
    gsecs, gcalls = graph_time(calls, warmup)
    out2 = torch.empty(sh.T, sh.N, dtype=torch.bfloat16, device=DEV)
    mm = [(lambda wt=wt: torch.matmul(x, wt.t(), out=out2)) for wt in wts]
    msecs, mcalls = graph_time(mm, warmup)
    del wts, calls, mm
    return dict(T=sh.T, d=sh.d, N=sh.N, us=1e6 * gsecs / gcalls, kernel_us=1e3 * stage_ms,
                launches_timed=nrec, hipblaslt_us=1e6 * msecs / mcalls)


def dense_line(name, r, mova_us):
    T, d, N = r["T"], r["d"], r["N"]
    flops = 2.0 * T * d * N
    nbytes = 2.0 * (N * d + T * d + T * N)
    line = {"workload": name, "T": T, "dense_us": r["us"], "dense_call_events_us": r["kernel_us"],
            "hipblaslt_us": r["hipblaslt_us"], "mova_us": mova_us,
            "mova_over_dense": mova_us / r["us"],
            "mova_over_hipblaslt": mova_us / r["hipblaslt_us"],
            "dense_tflops": flops / (r["us"] * 1e-6) / 1e12,
            "dense_frac_bf16_peak": flops / (r["us"] * 1e-6) / accounting.BF16_MFMA_PEAK_FLOPS,
            "dense_GB_per_s": nbytes / (r["us"] * 1e-6) / 1e9,
            "dense_frac_hbm": nbytes / (r["us"] * 1e-6) / accounting.HBM_PEAK_BPS}
    return line


def prefill_line(name, r):
    sh = r["shape"]
    fpt = accounting.flops_per_token(sh.d, sh.E, sh.k, sh.N)
    gtokens = r.get("graph_tokens", sh.T * r["graph_calls"])
    glayer_tokens = r.get("graph_layer_tokens", gtokens)
    tflops = glayer_tokens * fpt / r["graph_seconds"] / 1e12
    per_call_tokens = sh.T
    gemm_flops = 2 * per_call_tokens * sh.k * sh.d * sh.N
    gemm_tflops = gemm_flops / (r["stage_ms"] * 1e-3) / 1e12
    return {
        "workload": name,
        "tokens_per_s": gtokens / r["graph_seconds"],
        "ms_per_call": 1e3 * r["graph_seconds"] / r["graph_calls"],
        "eager_tokens_per_s": r["tokens"] / r["seconds"],
        "tflops": tflops,
        "frac_bf16_peak": tflops * 1e12 / accounting.BF16_MFMA_PEAK_FLOPS,
        "grouped_gemm_us": 1e3 * r["stage_ms"],
        "grouped_gemm_tflops": gemm_tflops,
        "grouped_gemm_frac": gemm_tflops * 1e12 / accounting.BF16_MFMA_PEAK_FLOPS,
    }


# HBM traffic of the decode kernel, measured by rocprofv3 counter passes and
# recorded with the hash of the kernel's sources; reported only while those
# sources are unchanged.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_kernel_T64_traffic.md")
DECODE_SOURCES = [os.path.join(ROOT, "mixture_value_projection_amd", "csrc", f)
                  for f in ("decode.hip", "common.h")]


def decode_source_hash():
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """Bytes per launch from the committed counter record, or None."""
    try:
        with open(TRAFFIC_RECORD) as fh:
            text = fh.read()
    except OSError:
        return None
    m = re.search(r"traffic-record: source_sha256=([0-9a-f]+) traffic_bytes=(\d+)", text)
    if m is None or m.group(1) != decode_source_hash():
        return None
    return int(m.group(2))


def copy_calibration(mib, reps=5):
    """Plain device-to-device copies of a known size (a reference for HBM counters)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=DEV).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {n} bytes")


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _oracle_rate(o, sh, T, min_seconds):
    """tokens/s of the float64 oracle on the first T tokens, repeated for at
    least min_seconds (at least once)."""
    import oracle
    x = o["x"][:T]
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.value_forward(x, o["router_w"], o["router_b"], o["expert_w"], sh.k, sh.scale,
                             sh.n_kv_heads, sh.head_dim)
        calls += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            return T * calls / el, calls, el


def cpu_baseline():
    """The CPU oracle (float64 numpy, as it stands) on the host's cores:
    * the decode workload (T=64) on every BLAS thread, ~8 s: the reported value;
    * the prefill chunk (T=4096) on every BLAS thread, once or more (~3 s);
    * a 512-token subset of the prefill chunk on one BLAS thread (~3 s): the
      per-core rate."""
    sys.path.insert(0, ROOT)
    from threadpoolctl import threadpool_info, threadpool_limits
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    out = {}
    for name in ("decode", "prefill"):
        w = inputs.WORKLOADS[name]
        t = inputs.make_layer(w.shape, w.seed, w.dtype, w.bias)
        out[name] = (w.shape, {k: v.double().numpy() for k, v in t.items()})
    sh, o = out["decode"]
    dec, dcalls, dsec = _oracle_rate(o, sh, sh.T, 8.0)
    sh, o = out["prefill"]
    pre, pcalls, psec = _oracle_rate(o, sh, sh.T, 3.0)
    with threadpool_limits(limits=1, user_api="blas"):
        one, ocalls, osec = _oracle_rate(o, sh, 512, 3.0)
    return {"value": dec, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "prefill_tokens_per_s": pre, "per_core_tokens_per_s": one,
            "sample": f"float64 numpy oracle: decode workload (T=64) {dcalls}x in {dsec:.1f} s on "
                      f"{threads} BLAS threads (value); prefill chunk (T=4096) {pcalls}x in "
                      f"{psec:.1f} s on {threads} threads (prefill_tokens_per_s); its first 512 "
                      f"tokens {ocalls}x in {osec:.1f} s on 1 thread (per_core_tokens_per_s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated per step")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run plain device copies of MIB MiB (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): this library has no "
              "multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load_library()
    torch.cuda.set_device(0)

    log("decode workload ...")
    r = run_single_layer("decode", args.steps, args.warmup, args.copies, graph_calls=args.steps)
    sh = r["shape"]
    step_s = r["graph_seconds"] / r["graph_calls"]
    tok_s = sh.T / step_s
    call_bytes = accounting.bytes_per_call(sh.T, r["touched"], sh.d, sh.E, sh.N, sh.k)
    kern_bytes = accounting.expert_kernel_bytes(sh.T, r["touched"], sh.d, sh.N)
    achieved = kern_bytes / (r["stage_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * step_s,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode step: T=64 tokens, d=2560, E=64 experts 2560->1024 "
                               "(8 KV heads x 128), top-4, scale 2.5, bf16, seeded synthetic "
                               "inputs, 4 rotated weight copies",
                   "T": sh.T, "d": sh.d, "E": sh.E, "k": sh.k, "n_kv_heads": sh.n_kv_heads,
                   "head_dim": sh.head_dim, "touched_experts": r["touched"]},
        "timing": f"median of {REPLAYS} replays of a HIP graph of exactly `steps` calls "
                  "(rotated weight copies), each replay bracketed by device synchronisation; "
                  "eager per-call launches give eager_tokens_per_s",
        "eager_tokens_per_s": r["tokens"] / r["seconds"],
        "max_abs_out": r["max_abs_out"],
        "whole_call": {"GB_per_s": call_bytes / step_s / 1e9,
                       "frac_hbm": call_bytes / step_s / accounting.HBM_PEAK_BPS,
                       "bytes": call_bytes},
        "roofline": {"kernel": "decode_kernel (expert weight stream)", "bound": "hbm",
                     "achieved": achieved, "peak": accounting.HBM_PEAK_BPS / 1e9, "unit": "GB/s",
                     "frac": achieved * 1e9 / accounting.HBM_PEAK_BPS,
                     "traffic": recorded_traffic(),
                     "bytes_per_launch": kern_bytes, "avg_launch_us": 1e3 * r["stage_ms"],
                     "launches_timed": r["stage_records"]},
    }
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
    if not args.headline_only:
        sec = []
        for name in ("prefill", "skewed"):
            log(f"{name} workload ...")
            rr = run_single_layer(name, MIN_CALLS, max(2, args.warmup // 4),
                                  args.copies if name == "prefill" else 2)
            d = prefill_line(name, rr)
            d["max_over_mean_load"] = rr["max_load"] / rr["mean_load"]
            d["max_abs_out"] = rr["max_abs_out"]
            sec.append(d)
            torch.cuda.empty_cache()
        log("chunked workload ...")
        rr = run_chunked(2, 1)
        sec.append(prefill_line("chunked", rr))
        line["secondary"] = sec
        torch.cuda.empty_cache()
        log("dense v_proj baseline ...")
        mova_us = {"decode": 1e6 * step_s}
        for d_ in sec:
            mova_us[d_["workload"]] = 1e3 * d_["ms_per_call"]
        gqa = []
        for name in ("decode", "prefill", "skewed", "chunked"):
            rr = run_dense(name, max(64, args.steps // 2), max(8, args.warmup))
            gqa.append(dense_line(name, rr, mova_us[name]))
            torch.cuda.empty_cache()
        line["gqa_baseline"] = gqa
        log("FFN mixture of experts ...")
        line["ffn_moe"] = [run_ffn("ffn_decode", args.steps, args.warmup),
                           run_ffn("ffn_prefill", MIN_CALLS, max(2, args.warmup // 4))]
        torch.cuda.empty_cache()
        log("compact-cache rebuild ...")
        shp = inputs.WORKLOADS["prefill"].shape
        rus, rec_us, plain_us = run_rebuild("prefill", MIN_CALLS, max(2, args.warmup // 4),
                                            args.copies)
        line["compact_cache_rebuild"] = {
            "tokens": shp.T, "us": rus, "us_per_cached_token": rus / shp.T,
            "forward_with_records_us": rec_us, "forward_us": plain_us,
            "bytes_per_token_value_cache": shp.N * 2,
            "bytes_per_token_record": 4 + 2 * shp.k,
            "bytes_per_token_compact": shp.d * 2 + 4 + 2 * shp.k,
            "note": "values of 4096 cached tokens rebuilt from stored x_t and their compact "
                    "routing records (6-bit ids in one 32-bit word, fp16 weights; no router); a "
                    "value cache reads the 2 KiB rows instead"}
        log("paged decode ...")
        pus, uus = run_paged_decode(args.steps, args.warmup, args.copies)
        line["paged_decode"] = {"us_per_step": pus, "plain_us_per_step": 1e6 * step_s,
                                "unfused_us_per_step": uus,
                                "tokens_per_s": sh.T / (pus * 1e-6),
                                "pool": "4096 blocks x 16 slots x [8, 128] bf16, distinct random "
                                        "slots, no contiguous output"}
        torch.cuda.empty_cache()
        log("small-batch decode ...")
        small = []
        for T in (1, 4, 8):  # the chain kernel, then one column group per wave
            rr = run_single_layer("decode", args.steps, args.warmup, args.copies, T=T)
            small.append({"T": T, "us_per_call": 1e6 * rr["graph_seconds"] / rr["graph_calls"],
                          "touched_experts": rr["touched"]})
            torch.cuda.empty_cache()
        line["small_batch_decode"] = small
        log("tensor-parallel shards ...")
        shards = []
        for tp in (2, 8):
            shards.append(run_tp_shard("decode", tp, args.steps, args.warmup))
            torch.cuda.empty_cache()
            shards.append(run_tp_shard("prefill", tp, MIN_CALLS, max(2, args.warmup // 4)))
            torch.cuda.empty_cache()
        line["tp_shard"] = shards
        log("expert-parallel shards ...")
        shards = []
        for ep in (2, 8):
            shards.append(run_ep_shard("decode", ep, args.steps, args.warmup))
            torch.cuda.empty_cache()
            shards.append(run_ep_shard("prefill", ep, MIN_CALLS, max(2, args.warmup // 4)))
            torch.cuda.empty_cache()
        line["ep_shard"] = shards
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
