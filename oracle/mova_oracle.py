"""Float64 CPU oracle of the MoVA routed value projection.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path.

What is computed, and where it is stated
----------------------------------------
Page "MoVA: routing the value vectors, and why the KV cache does not notice",
section "Where the routing happens", shows the attention layer's value path:

1. router logits are a bias-free linear map of the token (the router's weight
   only) from width d to E experts;
2. the logits go through a sigmoid and the router's bias is handed to the
   weight computation separately; the four (k) top experts are kept and their
   sigmoid scores are renormalised to sum to one and multiplied by 2.5;
3. each kept expert is a full d -> 8*128 linear map (no bias), SiLU is applied
   to each expert's output, and the k results are summed with the weights;
4. the (tokens, 1024) result is viewed as (tokens, 8, 128), column n being
   head n // 128, lane n % 128 -- the shape of a plain GQA value projection.

The same page's section "So what does it cost?" says the released combine is
a loop with one gather / project / index-add per touched expert;
``combine_experts`` follows that loop (it is the plainest correct order, not
a design for speed).  Matrix products use numpy's float64 matmul.

Readings where the pages leave a step open
------------------------------------------
* Bias role (parity unpinned).  The code passes the router bias separately
  from the linear map, and the page describes the weights as the kept
  experts' sigmoid scores divided by their sum and multiplied by 2.5.  The
  default reading ("select") adds the bias to the sigmoid
  scores for choosing experts only and weighs with the unbiased scores.  Two
  alternatives are kept for documentation: "logit" (sigmoid of logit + bias
  for both) and "weights" (biased scores used as weights too).
* Ties: equal selection scores go to the lower expert index, and the k
  selected experts are returned in order of (score desc, index asc).
* No epsilon in the renormalisation (k sigmoid values are each > 0).
* Experts have no bias: 64 * 2560 * 1024 * 45 = 7,549,747,200 value-expert
  parameters is the page's exact count, leaving no room for one.
* Router summation order (parity unpinned): float64 here; any fixed order is
  acceptable, near-ties are handled by the margin rule in the tests.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BIAS_ROLES = ("select", "logit", "weights")


def _f64(a) -> np.ndarray:
    """Upcast anything array-like (numpy, or torch via .numpy()) to float64."""
    if hasattr(a, "detach"):  # a torch tensor: go through float64 on the CPU
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + e^-z) in float64."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU z * sigmoid(z) (F.silu in the quoted code)."""
    return z * sigmoid(z)


def router_logits(x, router_w) -> np.ndarray:
    """Logits [T, E] = x [T, d] @ router_w[E, d]^T, the router's weight only
    (section "Where the routing happens": the linear map takes
    ``v_router.weight`` and no bias)."""
    return _f64(x) @ _f64(router_w).T


@dataclasses.dataclass
class Routing:
    """Per-token routing decision.

    idx [T, k] int64: selected experts ordered by (sel desc, index asc).
    w   [T, k] float64: renormalised scores times ``scale``.
    s   [T, E] float64: sigmoid scores.  sel [T, E]: selection scores.
    margin [T]: k-th largest minus (k+1)-th largest selection score
    (+inf when k == E).
    """

    idx: np.ndarray
    w: np.ndarray
    s: np.ndarray
    sel: np.ndarray
    margin: np.ndarray


def route(x, router_w, router_b, k: int, scale: float = 2.5,
          bias_role: str = "select") -> Routing:
    """Sigmoid router, top-k and renormalised weights.

    Page "MoVA: routing the value vectors ...", section "Where the routing
    happens": sigmoid scoring, top_k=4, scaling_factor=2.5; the weights are the
    kept experts' scores divided by their sum, times 2.5.  ``bias_role`` selects the
    reading of where the router bias enters (module docstring).
    """
    if bias_role not in BIAS_ROLES:
        raise ValueError(f"bias_role must be one of {BIAS_ROLES}")
    logits = router_logits(x, router_w)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    b = np.zeros(E) if router_b is None else _f64(router_b).reshape(E)
    if bias_role == "logit":
        s = sigmoid(logits + b)
        sel = s
    else:
        s = sigmoid(logits)
        sel = s + b
    # Order experts by selection score, descending, lower index first on ties.
    expert_ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((expert_ids, -sel), axis=1)
    idx = order[:, :k]
    ranked = np.take_along_axis(sel, order, axis=1)
    margin = ranked[:, k - 1] - ranked[:, k] if k < E else np.full(T, np.inf)
    chosen = np.take_along_axis(sel if bias_role == "weights" else s, idx, axis=1)
    w = scale * chosen / chosen.sum(axis=1, keepdims=True)
    return Routing(idx=idx, w=w, s=s, sel=sel, margin=margin)


def combine_experts(x, expert_w, idx, w) -> np.ndarray:
    """out [T, N] = sum_j w[t, j] * SiLU(W_{idx[t, j]} x_t).

    The released combine's loop (section "So what does it cost?"): for every
    touched expert, gather the tokens that chose it, apply that expert's
    linear map, SiLU, scale each row by its routing weight and index-add the
    rows into the output.
    """
    x = _f64(x)
    W = _f64(expert_w)
    idx = np.asarray(idx)
    w = _f64(w)
    T = x.shape[0]
    N = W.shape[1]
    out = np.zeros((T, N))
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)
        z = x[rows] @ W[e].T
        contrib = w[rows, slots][:, None] * silu(z)
        np.add.at(out, rows, contrib)
    return out


def value_forward(x, router_w, router_b, expert_w, k: int, scale: float = 2.5,
                  n_kv_heads: Optional[int] = None, head_dim: int = 128,
                  bias_role: str = "select"):
    """Full value path: routing, expert combine, GQA view.

    Returns (out [T, n_kv_heads, head_dim] float64, Routing).  The view puts
    column n at head n // head_dim, lane n % head_dim ("Where the routing
    happens": ``view(..., -1, 128)``).
    """
    r = route(x, router_w, router_b, k, scale, bias_role)
    out = combine_experts(x, expert_w, r.idx, r.w)
    N = out.shape[1]
    if n_kv_heads is None:
        n_kv_heads = N // head_dim
    if n_kv_heads * head_dim != N:
        raise ValueError("n_kv_heads * head_dim must equal the expert width")
    return out.reshape(out.shape[0], n_kv_heads, head_dim), r


def dense_value_proj(x, w_v) -> np.ndarray:
    """Plain GQA value projection V = x W_v^T (the dense layers' v_proj, section
    "So what does it cost?"), float64."""
    return _f64(x) @ _f64(w_v).T


def paged_value_write(cache, values, slot_mapping) -> np.ndarray:
    """Store each token's value vector in a paged pool (Option A of the page
    "IFM K2 Horizon Deep Dive: Inside Mixture-of-Value Attention (MoVA) ...",
    section "The Two Architectural Caching Strategies for MoVA": the routed
    projection is computed per token and the resulting vector is kept in the
    ordinary paged-attention memory pools; page 2's "Where the routing
    happens" hands that [8, 128] vector to the cache update).

    cache: [num_blocks, block_size, H, D]; values: [T, H, D]; slot_mapping:
    [T] integers.  Slot s is row s % block_size of block s // block_size.
    Reading (the pages do not fix the pool layout or padding): token-major
    blocks as above, and a slot outside [0, num_blocks * block_size) -- a
    negative padding slot in particular -- stores nothing.  Returns a new
    float64 array; the input is not modified.
    """
    out = _f64(cache).copy()
    vals = _f64(values)
    nb, bs = out.shape[0], out.shape[1]
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        s = int(s)
        if 0 <= s < nb * bs:
            out[s // bs, s % bs] = vals[t]
    return out


def rebuild_values(x, expert_w, idx, w) -> np.ndarray:
    """Value vectors rebuilt from a token's stored input and stored routing
    (Option B of the page "IFM K2 Horizon Deep Dive: Inside Mixture-of-Value
    Attention (MoVA) ...", section "The Two Architectural Caching Strategies
    for MoVA": the cache keeps x_t with the top-4 expert ids and 4 weights and
    materialises v_t when attention needs it).

    The same per-slot loop as ``combine_experts`` (page 2, "Where the routing
    happens": SiLU of each chosen expert's projection, weighted, summed),
    except that the routing is given.  Reading (the page does not say how an
    unused slot is marked): a slot whose id lies outside [0, E) adds nothing;
    ids may repeat, each slot counting once.  Returns [T, N] float64.
    """
    x = _f64(x)
    W = _f64(expert_w)
    idx = np.asarray(idx)
    w = _f64(w)
    E = W.shape[0]
    out = np.zeros((x.shape[0], W.shape[1]))
    for t in range(x.shape[0]):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            if not 0 <= e < E:
                continue
            z = W[e] @ x[t]
            out[t] += w[t, j] * silu(z)
    return out


# Bits per expert id in the compact routing record (E <= 64 experts).
RECORD_ID_BITS = 6
# Slots one 32-bit id word holds.
RECORD_MAX_K = 32 // RECORD_ID_BITS


def pack_routing_record(idx, w):
    """Compact routing record of a token (Option B of the page "IFM K2 Horizon
    Deep Dive: Inside Mixture-of-Value Attention (MoVA) ...", section "The Two
    Architectural Caching Strategies for MoVA": the cache keeps x_t together
    with the top-4 expert ids and four fp16 weights).

    Reading (the page's "16-bit mask" cannot hold four ids out of 64): the k
    ids of a token are packed at RECORD_ID_BITS bits each into one unsigned
    32-bit word, slot j in bits [6j, 6j + 6), so k <= 5; the k weights are
    rounded to fp16 (IEEE binary16, nearest even).  At k = 4 a record is
    4 + 8 = 12 bytes per token.

    idx [T, k] integers in [0, 64), w [T, k] -> (ids [T] uint32, w16 [T, k] float16).
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    if k > RECORD_MAX_K:
        raise ValueError(f"a record holds at most {RECORD_MAX_K} slots")
    if (idx < 0).any() or (idx >= (1 << RECORD_ID_BITS)).any():
        raise ValueError("expert ids must lie in [0, 64)")
    ids = np.zeros(T, dtype=np.uint64)
    for j in range(k):
        ids += idx[:, j].astype(np.uint64) << np.uint64(RECORD_ID_BITS * j)
    w16 = _f64(w).reshape(T, k).astype(np.float16)  # one rounding, nearest even
    return ids.astype(np.uint32), w16


def unpack_routing_record(ids, w16, k: int):
    """The inverse of ``pack_routing_record``: (idx [T, k] int64, w [T, k]
    float64 holding the fp16 values exactly)."""
    ids = np.asarray(ids, dtype=np.uint64)
    mask = np.uint64((1 << RECORD_ID_BITS) - 1)
    idx = np.stack([(ids >> np.uint64(RECORD_ID_BITS * j)) & mask for j in range(k)], axis=1)
    return idx.astype(np.int64), np.asarray(w16, dtype=np.float16).astype(np.float64).reshape(-1, k)


def rebuild_from_record(x, expert_w, ids, w16, k: int) -> np.ndarray:
    """Value vectors rebuilt from stored x_t and a stored compact record: the
    record unpacked, then ``rebuild_values`` (ids >= E mark unused slots)."""
    idx, w = unpack_routing_record(ids, w16, k)
    return rebuild_values(x, expert_w, idx, w)


def swiglu_expert(x, gate_w, up_w, down_w) -> np.ndarray:
    """One SwiGLU FFN expert, down( SiLU(gate x) * (up x) ), bias-free,
    nn.Linear weight layout ([out, in]).  Rows of x are tokens."""
    x = _f64(x)
    g = x @ _f64(gate_w).T
    u = x @ _f64(up_w).T
    return (silu(g) * u) @ _f64(down_w).T


def ffn_moe_forward(x, router_w, router_b, gate_w, up_w, down_w, k: int, scale: float,
                    shared=None):
    """FFN mixture of experts with top-k routing plus an optional shared
    expert (the thevalue.engineering page on the MoVA architecture, section
    "Dual sparsity": 100 FFN experts, top-8+1).  The pages fix neither the
    expert shape nor the routing function.  Readings: SwiGLU experts
    (``swiglu_expert``); routing by the value router's function (``route``:
    sigmoid scores, bias for selection, renormalised top-k times ``scale``);
    out = sum_j w_j expert_{idx_j}(x) + shared(x), with ``shared`` a
    (gate_w, up_w, down_w) triple or None.  Returns (out [T, d] float64,
    Routing).
    """
    x = _f64(x)
    r = route(x, router_w, router_b, k, scale)
    G, U, D = _f64(gate_w), _f64(up_w), _f64(down_w)
    out = np.zeros((x.shape[0], D.shape[1]))
    for t in range(x.shape[0]):
        for j in range(k):
            e = int(r.idx[t, j])
            out[t] += r.w[t, j] * swiglu_expert(x[t:t + 1], G[e], U[e], D[e])[0]
    if shared is not None:
        out += swiglu_expert(x, *shared)
    return out, r
