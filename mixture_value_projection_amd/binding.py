"""ctypes binding of ``libmova.so`` (the C ABI in include/mova.h).

Argument marshalling only: torch tensors are checked (device, dtype, shape,
contiguity), their device pointers and the current HIP stream are handed to
the library, and a negative status becomes ``MovaError``.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Tuple

import torch

from .build import LIBPATH

_LIB = None

MOVA_OK = 0
STAGES = ("router", "dispatch", "experts", "combine", "dense")


class MovaError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"{what}: {status_str(rc)} ({rc})")
        self.rc = rc


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmova.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    p = path or os.environ.get("MOVA_LIB", LIBPATH)
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m mixture_value_projection_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.mova_version.restype = i
    lib.mova_version.argtypes = []
    lib.mova_status_str.restype = ctypes.c_char_p
    lib.mova_status_str.argtypes = [i]
    lib.mova_workspace_bytes.restype = sz
    lib.mova_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.mova_route.restype = i
    lib.mova_route.argtypes = [vp, vp, vp, i, i, i, i, f, vp, vp, vp]
    lib.mova_value_forward.restype = i
    lib.mova_value_forward.argtypes = [vp, vp, vp, vp, i, i, i, i, f, i, i, vp, vp, vp, vp, sz, vp]
    lib.mova_value_forward_paged.restype = i
    lib.mova_value_forward_paged.argtypes = [vp, vp, vp, vp, i, i, i, i, f, i, i, vp, i, i, vp, vp,
                                             vp, vp, vp, sz, vp]
    lib.mova_value_forward_noalloc.restype = i
    lib.mova_value_forward_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, f, i, i, vp, vp, vp, vp]
    lib.mova_value_forward_record.restype = i
    lib.mova_value_forward_record.argtypes = [vp, vp, vp, vp, i, i, i, i, f, i, i, vp, vp, vp, vp,
                                              sz, vp]
    lib.mova_value_from_record.restype = i
    lib.mova_value_from_record.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, vp, vp, sz, vp]
    lib.mova_value_from_routing.restype = i
    lib.mova_value_from_routing.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, vp, vp, sz, vp]
    lib.mova_ffn_workspace_bytes.restype = sz
    lib.mova_ffn_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.mova_ffn_pack_gate_up.restype = i
    lib.mova_ffn_pack_gate_up.argtypes = [vp, vp, i, i, i, vp, vp]
    lib.mova_ffn_moe_forward.restype = i
    lib.mova_ffn_moe_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp, vp, i, i, i, f, vp, vp,
                                         vp, vp, sz, vp]
    lib.mova_dense_workspace_bytes.restype = sz
    lib.mova_dense_workspace_bytes.argtypes = [i, i, i, i]
    lib.mova_dense_value_proj.restype = i
    lib.mova_dense_value_proj.argtypes = [vp, vp, i, i, i, i, vp, vp, sz, vp]
    lib.mova_debug_override.restype = i
    lib.mova_debug_override.argtypes = [i, i]
    lib.mova_debug_override_get.restype = i
    lib.mova_debug_override_get.argtypes = [i]
    lib.mova_timing_enable.restype = i
    lib.mova_timing_enable.argtypes = [i, ctypes.c_uint]
    lib.mova_timing_read.restype = i
    lib.mova_timing_read.argtypes = [i, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    _LIB = lib
    return lib


def status_str(rc: int) -> str:
    return load_library().mova_status_str(int(rc)).decode()


def version() -> int:
    return load_library().mova_version()


def workspace_bytes(T: int, d: int, E: int, k: int, n_kv_heads: int, head_dim: int) -> int:
    n = load_library().mova_workspace_bytes(T, d, E, k, n_kv_heads, head_dim)
    if n == ctypes.c_size_t(-1).value:
        raise MovaError(-2, "mova_workspace_bytes")
    return n


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Tuple[int, ...], device) -> None:
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def route(x: torch.Tensor, router_w: torch.Tensor, router_b: Optional[torch.Tensor], k: int,
          scale: float = 2.5, topk_idx: Optional[torch.Tensor] = None,
          topk_w: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mova_route: returns (idx int32 [T, k], w float32 [T, k])."""
    lib = load_library()
    T, d = x.shape
    E = router_w.shape[0]
    dev = x.device
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(router_w, "router_w", torch.bfloat16, (E, d), dev)
    if router_b is not None:
        _check(router_b, "router_b", torch.float32, (E,), dev)
    if topk_idx is None:
        topk_idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty(T, k, dtype=torch.float32, device=dev)
    _check(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _check(topk_w, "topk_w", torch.float32, (T, k), dev)
    rc = lib.mova_route(_ptr(x), _ptr(router_w), _ptr(router_b), T, d, E, k, float(scale),
                        _ptr(topk_idx), _ptr(topk_w), _stream(dev))
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_route")
    return topk_idx, topk_w


def value_forward(x: torch.Tensor, router_w: torch.Tensor, router_b: Optional[torch.Tensor],
                  expert_w: torch.Tensor, k: int, scale: float = 2.5,
                  n_kv_heads: Optional[int] = None, head_dim: int = 128,
                  out: Optional[torch.Tensor] = None,
                  topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mova_value_forward: returns out bf16 [T, n_kv_heads, head_dim].

    ``topk_idx`` / ``topk_w`` (optional, int32 / float32 [T, k]) receive the
    routing; ``workspace`` (optional uint8 tensor) is reused when large enough.
    """
    lib = load_library()
    T, d = x.shape
    E, N, d2 = expert_w.shape
    if d2 != d:
        raise ValueError("expert_w's last dim must equal x's width")
    if n_kv_heads is None:
        n_kv_heads = N // head_dim
    if n_kv_heads * head_dim != N:
        raise ValueError("n_kv_heads * head_dim must equal the expert width")
    dev = x.device
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(router_w, "router_w", torch.bfloat16, (E, d), dev)
    if router_b is not None:
        _check(router_b, "router_b", torch.float32, (E,), dev)
    _check(expert_w, "expert_w", torch.bfloat16, (E, N, d), dev)
    if out is None:
        out = torch.empty(T, n_kv_heads, head_dim, dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, n_kv_heads, head_dim), dev)
    if topk_idx is not None:
        _check(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    if topk_w is not None:
        _check(topk_w, "topk_w", torch.float32, (T, k), dev)
    nbytes = workspace_bytes(T, d, E, k, n_kv_heads, head_dim)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    rc = lib.mova_value_forward(_ptr(x), _ptr(router_w), _ptr(router_b), _ptr(expert_w),
                                T, d, E, k, float(scale), n_kv_heads, head_dim, _ptr(out),
                                _ptr(topk_idx), _ptr(topk_w), _ptr(workspace),
                                workspace.numel(), _stream(dev))
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_value_forward")
    return out


# Size of the static scratch of mova_value_forward_noalloc (MOVA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 48 << 20


def value_forward_noalloc(x: torch.Tensor, router_w: torch.Tensor,
                          router_b: Optional[torch.Tensor], expert_w: torch.Tensor, k: int,
                          scale: float, out: torch.Tensor,
                          topk_idx: Optional[torch.Tensor] = None,
                          topk_w: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mova_value_forward_noalloc: mova_value_forward with the library's static
    scratch instead of a workspace.  ``out`` (bf16 [T, n_kv_heads, head_dim])
    is required, so this wrapper allocates nothing either."""
    lib = load_library()
    T, d = x.shape
    E, N, d2 = expert_w.shape
    if d2 != d:
        raise ValueError("expert_w's last dim must equal x's width")
    if out.dim() != 3 or out.shape[1] * out.shape[2] != N:
        raise ValueError("out must be [T, n_kv_heads, head_dim] with n_kv_heads * head_dim = N")
    H, D = out.shape[1], out.shape[2]
    dev = x.device
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(router_w, "router_w", torch.bfloat16, (E, d), dev)
    if router_b is not None:
        _check(router_b, "router_b", torch.float32, (E,), dev)
    _check(expert_w, "expert_w", torch.bfloat16, (E, N, d), dev)
    _check(out, "out", torch.bfloat16, (T, H, D), dev)
    if topk_idx is not None:
        _check(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    if topk_w is not None:
        _check(topk_w, "topk_w", torch.float32, (T, k), dev)
    rc = lib.mova_value_forward_noalloc(_ptr(x), _ptr(router_w), _ptr(router_b), _ptr(expert_w),
                                        T, d, E, k, float(scale), H, D, _ptr(out), _ptr(topk_idx),
                                        _ptr(topk_w), _stream(dev))
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_value_forward_noalloc")
    return out


def value_forward_paged(x: torch.Tensor, router_w: torch.Tensor, router_b: Optional[torch.Tensor],
                        expert_w: torch.Tensor, k: int, scale: float, v_cache: torch.Tensor,
                        slot_mapping: torch.Tensor, out: Optional[torch.Tensor] = None,
                        topk_idx: Optional[torch.Tensor] = None,
                        topk_w: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """mova_value_forward_paged: stores each token's value vector in
    ``v_cache`` (bf16 [num_blocks, block_size, n_kv_heads, head_dim]) at
    ``slot_mapping[t]`` (int64 [T]; slots outside the pool store nothing) and,
    if ``out`` is given, in ``out`` too.  Returns ``out``."""
    lib = load_library()
    T, d = x.shape
    E, N, d2 = expert_w.shape
    if d2 != d:
        raise ValueError("expert_w's last dim must equal x's width")
    if v_cache.dim() != 4:
        raise ValueError("v_cache must be [num_blocks, block_size, n_kv_heads, head_dim]")
    nb, bs, H, D = v_cache.shape
    if H * D != N:
        raise ValueError("v_cache's n_kv_heads * head_dim must equal the expert width")
    dev = x.device
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(router_w, "router_w", torch.bfloat16, (E, d), dev)
    if router_b is not None:
        _check(router_b, "router_b", torch.float32, (E,), dev)
    _check(expert_w, "expert_w", torch.bfloat16, (E, N, d), dev)
    _check(v_cache, "v_cache", torch.bfloat16, (nb, bs, H, D), dev)
    _check(slot_mapping, "slot_mapping", torch.int64, (T,), dev)
    if out is not None:
        _check(out, "out", torch.bfloat16, (T, H, D), dev)
    if topk_idx is not None:
        _check(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    if topk_w is not None:
        _check(topk_w, "topk_w", torch.float32, (T, k), dev)
    nbytes = workspace_bytes(T, d, E, k, H, D)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    rc = lib.mova_value_forward_paged(_ptr(x), _ptr(router_w), _ptr(router_b), _ptr(expert_w),
                                      T, d, E, k, float(scale), H, D, _ptr(v_cache), nb, bs,
                                      _ptr(slot_mapping), _ptr(out), _ptr(topk_idx), _ptr(topk_w),
                                      _ptr(workspace), workspace.numel(), _stream(dev))
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_value_forward_paged")
    return out


def value_from_routing(x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                       expert_w: torch.Tensor, n_kv_heads: Optional[int] = None,
                       head_dim: int = 128, out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mova_value_from_routing: value vectors rebuilt from stored inputs and
    stored routing (int32 ids, float32 weights [T, k]); ids outside [0, E)
    mark unused slots.  Returns bf16 [T, n_kv_heads, head_dim]."""
    lib = load_library()
    T, d = x.shape
    E, N, d2 = expert_w.shape
    k = topk_idx.shape[1] if topk_idx.dim() == 2 else -1
    if d2 != d:
        raise ValueError("expert_w's last dim must equal x's width")
    if n_kv_heads is None:
        n_kv_heads = N // head_dim
    if n_kv_heads * head_dim != N:
        raise ValueError("n_kv_heads * head_dim must equal the expert width")
    dev = x.device
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _check(topk_w, "topk_w", torch.float32, (T, k), dev)
    _check(expert_w, "expert_w", torch.bfloat16, (E, N, d), dev)
    if out is None:
        out = torch.empty(T, n_kv_heads, head_dim, dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, n_kv_heads, head_dim), dev)
    nbytes = workspace_bytes(T, d, E, k, n_kv_heads, head_dim)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    rc = lib.mova_value_from_routing(_ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(expert_w), T, d,
                                     E, k, n_kv_heads, head_dim, _ptr(out), _ptr(workspace),
                                     workspace.numel(), _stream(dev))
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_value_from_routing")
    return out


def value_forward_record(x: torch.Tensor, router_w: torch.Tensor,
                         router_b: Optional[torch.Tensor], expert_w: torch.Tensor, k: int,
                         scale: float = 2.5, n_kv_heads: Optional[int] = None, head_dim: int = 128,
                         out: Optional[torch.Tensor] = None,
                         record_ids: Optional[torch.Tensor] = None,
                         record_w: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None):
    """mova_value_forward_record: returns (out bf16 [T, H, D], record_ids int32
    [T] holding the uint32 words, record_w float16 [T, k])."""
    lib = load_library()
    T, d = x.shape
    E, N, d2 = expert_w.shape
    if d2 != d:
        raise ValueError("expert_w's last dim must equal x's width")
    if n_kv_heads is None:
        n_kv_heads = N // head_dim
    if n_kv_heads * head_dim != N:
        raise ValueError("n_kv_heads * head_dim must equal the expert width")
    dev = x.device
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(router_w, "router_w", torch.bfloat16, (E, d), dev)
    if router_b is not None:
        _check(router_b, "router_b", torch.float32, (E,), dev)
    _check(expert_w, "expert_w", torch.bfloat16, (E, N, d), dev)
    if out is None:
        out = torch.empty(T, n_kv_heads, head_dim, dtype=torch.bfloat16, device=dev)
    if record_ids is None:
        record_ids = torch.empty(T, dtype=torch.int32, device=dev)
    if record_w is None:
        record_w = torch.empty(T, k, dtype=torch.float16, device=dev)
    _check(out, "out", torch.bfloat16, (T, n_kv_heads, head_dim), dev)
    _check(record_ids, "record_ids", torch.int32, (T,), dev)
    _check(record_w, "record_w", torch.float16, (T, k), dev)
    nbytes = workspace_bytes(T, d, E, k, n_kv_heads, head_dim)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    rc = lib.mova_value_forward_record(_ptr(x), _ptr(router_w), _ptr(router_b), _ptr(expert_w),
                                       T, d, E, k, float(scale), n_kv_heads, head_dim, _ptr(out),
                                       _ptr(record_ids), _ptr(record_w), _ptr(workspace),
                                       workspace.numel(), _stream(dev))
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_value_forward_record")
    return out, record_ids, record_w


def value_from_record(x: torch.Tensor, record_ids: torch.Tensor, record_w: torch.Tensor,
                      expert_w: torch.Tensor, n_kv_heads: Optional[int] = None,
                      head_dim: int = 128, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mova_value_from_record: value vectors rebuilt from stored inputs and
    compact records (record_ids int32 [T] as uint32 words, record_w float16
    [T, k])."""
    lib = load_library()
    T, d = x.shape
    E, N, d2 = expert_w.shape
    k = record_w.shape[1] if record_w.dim() == 2 else -1
    if d2 != d:
        raise ValueError("expert_w's last dim must equal x's width")
    if n_kv_heads is None:
        n_kv_heads = N // head_dim
    if n_kv_heads * head_dim != N:
        raise ValueError("n_kv_heads * head_dim must equal the expert width")
    dev = x.device
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(record_ids, "record_ids", torch.int32, (T,), dev)
    _check(record_w, "record_w", torch.float16, (T, k), dev)
    _check(expert_w, "expert_w", torch.bfloat16, (E, N, d), dev)
    if out is None:
        out = torch.empty(T, n_kv_heads, head_dim, dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, n_kv_heads, head_dim), dev)
    nbytes = workspace_bytes(T, d, E, k, n_kv_heads, head_dim)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    rc = lib.mova_value_from_record(_ptr(x), _ptr(record_ids), _ptr(record_w), _ptr(expert_w), T, d,
                                    E, k, n_kv_heads, head_dim, _ptr(out), _ptr(workspace),
                                    workspace.numel(), _stream(dev))
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_value_from_record")
    return out


def ffn_workspace_bytes(T: int, d: int, E: int, k: int, inter: int, inter_shared: int) -> int:
    n = load_library().mova_ffn_workspace_bytes(T, d, E, k, inter, inter_shared)
    if n == ctypes.c_size_t(-1).value:
        raise MovaError(-2, "mova_ffn_workspace_bytes")
    return n


def ffn_pack_gate_up(gate_w: torch.Tensor, up_w: torch.Tensor) -> torch.Tensor:
    """mova_ffn_pack_gate_up: bf16 [E, inter, d] gate and up weights (or
    [inter, d] for the shared expert) -> the interleaved [E, 2 inter, d]
    (or [2 inter, d]) layout the FFN forward reads."""
    lib = load_library()
    squeeze = gate_w.dim() == 2
    g = gate_w.unsqueeze(0) if squeeze else gate_w
    u = up_w.unsqueeze(0) if squeeze else up_w
    E, inter, d = g.shape
    _check(g, "gate_w", torch.bfloat16, (E, inter, d), g.device)
    _check(u, "up_w", torch.bfloat16, (E, inter, d), g.device)
    dst = torch.empty(E, 2 * inter, d, dtype=torch.bfloat16, device=g.device)
    rc = lib.mova_ffn_pack_gate_up(_ptr(g), _ptr(u), E, inter, d, _ptr(dst), _stream(g.device))
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_ffn_pack_gate_up")
    return dst[0] if squeeze else dst


def ffn_moe_forward(x: torch.Tensor, router_w: torch.Tensor, router_b: Optional[torch.Tensor],
                    gate_up_w: torch.Tensor, down_w: torch.Tensor, k: int, scale: float,
                    shared_gate_up_w: Optional[torch.Tensor] = None,
                    shared_down_w: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, topk_idx: Optional[torch.Tensor] = None,
                    topk_w: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mova_ffn_moe_forward: returns bf16 [T, d].  gate_up_w comes from
    ``ffn_pack_gate_up``; the shared expert is optional."""
    lib = load_library()
    T, d = x.shape
    E, two_inter, d2 = gate_up_w.shape
    inter = two_inter // 2
    if d2 != d:
        raise ValueError("gate_up_w's last dim must equal x's width")
    inter_s = 0 if shared_gate_up_w is None else shared_gate_up_w.shape[0] // 2
    dev = x.device
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(router_w, "router_w", torch.bfloat16, (E, d), dev)
    if router_b is not None:
        _check(router_b, "router_b", torch.float32, (E,), dev)
    _check(gate_up_w, "gate_up_w", torch.bfloat16, (E, 2 * inter, d), dev)
    _check(down_w, "down_w", torch.bfloat16, (E, d, inter), dev)
    if inter_s:
        _check(shared_gate_up_w, "shared_gate_up_w", torch.bfloat16, (2 * inter_s, d), dev)
        _check(shared_down_w, "shared_down_w", torch.bfloat16, (d, inter_s), dev)
    if out is None:
        out = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, d), dev)
    if topk_idx is not None:
        _check(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    if topk_w is not None:
        _check(topk_w, "topk_w", torch.float32, (T, k), dev)
    nbytes = ffn_workspace_bytes(T, d, E, k, inter, inter_s)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    rc = lib.mova_ffn_moe_forward(_ptr(x), _ptr(router_w), _ptr(router_b), _ptr(gate_up_w),
                                  _ptr(down_w), E, k, inter, _ptr(shared_gate_up_w),
                                  _ptr(shared_down_w), inter_s, T, d, float(scale), _ptr(out),
                                  _ptr(topk_idx), _ptr(topk_w), _ptr(workspace), workspace.numel(),
                                  _stream(dev))
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_ffn_moe_forward")
    return out


def dense_workspace_bytes(T: int, d: int, n_kv_heads: int, head_dim: int) -> int:
    n = load_library().mova_dense_workspace_bytes(T, d, n_kv_heads, head_dim)
    if n == ctypes.c_size_t(-1).value:
        raise MovaError(-2, "mova_dense_workspace_bytes")
    return n


def dense_value_proj(x: torch.Tensor, w_v: torch.Tensor, n_kv_heads: Optional[int] = None,
                     head_dim: int = 128, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mova_dense_value_proj: the plain value projection x w_v^T as bf16
    [T, n_kv_heads, head_dim] (w_v is bf16 [n_kv_heads * head_dim, d])."""
    lib = load_library()
    T, d = x.shape
    N, d2 = w_v.shape
    if d2 != d:
        raise ValueError("w_v's last dim must equal x's width")
    if n_kv_heads is None:
        n_kv_heads = N // head_dim
    if n_kv_heads * head_dim != N:
        raise ValueError("n_kv_heads * head_dim must equal w_v's row count")
    dev = x.device
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(w_v, "w_v", torch.bfloat16, (N, d), dev)
    if out is None:
        out = torch.empty(T, n_kv_heads, head_dim, dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, n_kv_heads, head_dim), dev)
    nbytes = dense_workspace_bytes(T, d, n_kv_heads, head_dim)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    rc = lib.mova_dense_value_proj(_ptr(x), _ptr(w_v), T, d, n_kv_heads, head_dim, _ptr(out),
                                   _ptr(workspace), workspace.numel(), _stream(dev))
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_dense_value_proj")
    return out


# Kernel-choice overrides (mova_debug_override): name -> (key, {value name: value}).
OVERRIDES = {
    "path": (0, {"decode": 1, "grouped": 2}),
    "router": (1, {"16": 1, "32s4": 2, "32s3": 3, "64": 4}),
    "gemm_tile": (2, {"256x256": 1, "128x256": 2, "128x128": 3, "128x128s3": 4,
                      "128x128s4": 5, "128x128w4": 6, "352x256": 7}),
    "dense_path": (3, {"skinny": 1, "tiled": 2}),
    "decode_chain": (4, {"on": 1, "off": 2, "token": 3}),
    "decode_groups": (5, {"1": 1, "2": 2}),
    "serial": (6, {"on": 1}),
}


def set_override(name: str, value: Optional[str]) -> None:
    """Force one kernel choice for later calls (tests, measurements); value
    None restores the automatic choice."""
    key, values = OVERRIDES[name]
    v = 0 if value is None else values[str(value)]
    rc = load_library().mova_debug_override(key, v)
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_debug_override")


def get_override(name: str) -> Optional[str]:
    key, values = OVERRIDES[name]
    v = load_library().mova_debug_override_get(key)
    return None if v == 0 else {i: n for n, i in values.items()}[v]


def clear_overrides() -> None:
    for name in OVERRIDES:
        set_override(name, None)


class overrides:
    """Context manager: ``with overrides(path="grouped"): ...`` forces the
    named choices inside the block and restores the previous ones after."""

    def __init__(self, **kw):
        self.kw = kw
        self.saved = {}

    def __enter__(self):
        for name, value in self.kw.items():
            self.saved[name] = get_override(name)
            set_override(name, value)
        return self

    def __exit__(self, *exc):
        for name, value in self.saved.items():
            set_override(name, value)
        return False


def timing_enable(capacity: int, stages=STAGES) -> None:
    """Record HIP events around the named stages for up to ``capacity`` calls."""
    mask = 0
    for s in stages:
        mask |= 1 << STAGES.index(s)
    rc = load_library().mova_timing_enable(int(capacity), mask)
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_timing_enable")


def timing_read() -> List[Tuple[float, int]]:
    """[(total_ms, launches)] per stage, in the order of ``STAGES``."""
    n = len(STAGES)
    tot = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    rc = load_library().mova_timing_read(n, tot, cnt)
    if rc != MOVA_OK:
        raise MovaError(rc, "mova_timing_read")
    return [(tot[i], cnt[i]) for i in range(n)]
