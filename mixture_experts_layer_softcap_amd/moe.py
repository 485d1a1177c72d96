"""Thin ctypes binding of libmoe.so (C ABI declared in include/moe.h).

Argument marshalling only: every step runs in the library's HIP kernels.  Functions take
torch tensors that live on the current HIP device (uint16 tensors carry bf16 bits, uint8
tensors carry E4M3 codes) and enqueue on torch's current stream unless a stream is given.
A missing library raises immediately; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK = 0
MOE_E_INVAL = -1
MOE_E_NOSPC = -2
MOE_E_HIP = -3
MOE_E_DEVICE = -4

MOE_GEMM_FP8_B128 = 0
MOE_GEMM_BF16 = 1

MOE_EPI_STORE_F32 = 0
MOE_EPI_STORE_BF16 = 1
MOE_EPI_ROUTE_F32 = 2
MOE_EPI_SWIGLU_BF16 = 3

MOE_FWD_GRAPH = 1
MOE_FWD_STATIC_GRID = 2
MOE_FWD_STAGED = 4
MOE_FWD_ATOMIC_COMBINE = 64
MOE_FWD_ROUTE_KERNEL = 128
MOE_FWD_ROUTE_SELF = 256

MOE_QUEUE_WORDS = 16
MOE_QUEUE_HANDOFF_STATUS = 10
MOE_SCHED_AUTO = -1
MOE_SCHED_DISPATCH = 0
MOE_SCHED_STATIC = 1
MOE_SCHED_QUEUE = 2
MOE_SCHED_QUEUE_XCD = 3


def MOE_FWD_SCHED(s: int) -> int:
    return (s + 1) << 3

# entry points and their C signatures (names identical to include/moe.h)
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_device_check": (_I, []),
    "moe_router_logits": (_I, [_P, _I, _I, _P, _I, _P, _P]),
    "moe_route": (_I, [_P, _I, _I, _I, _F, _P, _P, _P]),
    "moe_route_quantize": (_I, [_P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P]),
    "moe_max_tasks": (_I, [_I, _I, _I, _I, _I]),
    "moe_build_layout": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P]),
    "moe_quant_sort_gather": (_I, [_P, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_sort_gather_bf16": (_I, [_P, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P]),
    "moe_quantize_weights": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_gemm_n_tile": (_I, [_I]),
    "moe_grouped_gemm": (_I, [_I, _P, _P, _I, _I, _P, _P, _I, _I, _P, _P, _I, _I, _P, _I,
                              _P, _P, _I, _P]),
    "moe_forward_kernels": (_I, [_I, _I, _I, _I, _I, _I, _I]),
    "moe_grouped_gemm_routed": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P]),
    "moe_route_grouped_gemm": (_I, [_P, _P, _I, _I, _I, _I, _F, _P, _P, _I, _P, _P, _P, _P, _P,
                                    _P]),
    "moe_grouped_gemm_gather": (_I, [_P, _P, _I, _I, _I, _P, _P, _I, _I, _P, _P, _I, _I, _P, _P,
                                     _P, _I, _P]),
    "moe_scatter": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_forward_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "moe_forward_workspace_offset": (ctypes.c_int64, [_I, _I, _I, _I, _I, _I]),
    "moe_forward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _S, _P]),
    "moe_forward_ex": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _S, _I, _I, _P]),
    "moe_forward_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P]),
    "moe_ffn_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "moe_ffn_workspace_offset": (ctypes.c_int64, [_I, _I, _I, _I, _I, _I]),
    "moe_ffn_forward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _S, _I, _I, _P]),
    "moe_swiglu_quant": (_I, [_P, _I, _I, _P, _P, _P]),
    "moe_mlp_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "moe_mlp_forward_kernels": (_I, [_I, _I, _I, _I, _I, _I]),
    "moe_mlp_workspace_offset": (ctypes.c_int64, [_I, _I, _I, _I, _I, _I]),
    "moe_mlp_forward": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _S, _I,
                             _P]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, name: str, status: int):
        msg = lib().moe_status_string(status).decode()
        super().__init__(f"{name} failed: {msg} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by mixture_experts_layer_softcap_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mixture_experts_layer_softcap_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _call(name: str, *args):
    rc = getattr(lib(), name)(*args)
    if rc != MOE_OK:
        raise MoeError(name, rc)
    return rc


def device_check() -> int:
    return lib().moe_device_check()


def route(logits, k: int, softcap: float, topk_ids, topk_weights, stream=None):
    M, E = logits.shape
    _call("moe_route", _ptr(logits), M, E, k, softcap, _ptr(topk_ids), _ptr(topk_weights),
          _stream(stream))


def route_quantize(logits, x, k: int, softcap: float, topk_ids, topk_weights, x_q, x_scales,
                   stream=None):
    """moe_route plus the per-token E4M3 quantisation of x (moe_route_quantize)."""
    M, E = logits.shape
    K = x.shape[1]
    _call("moe_route_quantize", _ptr(logits), _ptr(x), M, E, k, K, softcap, _ptr(topk_ids),
          _ptr(topk_weights), _ptr(x_q), _ptr(x_scales), _stream(stream))


def max_tasks(M: int, k: int, E: int, n_blocks: int, chunk_rows: int) -> int:
    v = lib().moe_max_tasks(M, k, E, n_blocks, chunk_rows)
    if v < 0:
        raise MoeError("moe_max_tasks", MOE_E_INVAL)
    return v


def build_layout(topk_ids, E: int, n_blocks: int, chunk_rows: int, counts, offsets, cursors,
                 tasks, ntasks, queue, sorted_route_ids=None, route_slots=None, stream=None):
    M, k = topk_ids.shape
    _call("moe_build_layout", _ptr(topk_ids), M, k, E, n_blocks, chunk_rows, _ptr(counts),
          _ptr(offsets), _ptr(cursors), _ptr(tasks), tasks.shape[0], _ptr(ntasks), _ptr(queue),
          _ptr(sorted_route_ids), _ptr(route_slots), _stream(stream))


def quant_sort_gather(x, topk_ids, E: int, cursors, sorted_route_ids, a_q, a_scales,
                      route_slots=None, stream=None):
    M, K = x.shape
    k = topk_ids.shape[1]
    _call("moe_quant_sort_gather", _ptr(x), M, K, _ptr(topk_ids), k, E, _ptr(cursors),
          _ptr(sorted_route_ids), _ptr(route_slots), _ptr(a_q), _ptr(a_scales),
          _stream(stream))


def quantize_weights(w, w_q, w_scales, stream=None):
    E, N, K = w.shape
    _call("moe_quantize_weights", _ptr(w), E, N, K, _ptr(w_q), _ptr(w_scales), _stream(stream))


def gemm_n_tile(mode: int) -> int:
    return lib().moe_gemm_n_tile(mode)


def grouped_gemm(mode: int, a, a_scales, w, w_scales, tasks, ntasks, chunk_rows: int, out,
                 epilogue: int, queue=None, sorted_route_ids=None, sched: int = MOE_SCHED_AUTO,
                 stream=None):
    rows, K = a.shape
    E, N, _ = w.shape
    _call("moe_grouped_gemm", mode, _ptr(a), _ptr(a_scales), rows, K, _ptr(w), _ptr(w_scales),
          E, N, _ptr(tasks), _ptr(ntasks), tasks.shape[0], chunk_rows, _ptr(queue), epilogue,
          _ptr(sorted_route_ids), _ptr(out), sched, _stream(stream))


def grouped_gemm_gather(x_q, x_scales, k: int, w_q, w_scales, tasks, ntasks, chunk_rows: int,
                        sorted_route_ids, rows, queue=None, sched: int = MOE_SCHED_AUTO,
                        stream=None):
    """Grouped FP8 GEMM gathering routed rows from token-major codes (moe_grouped_gemm_gather);
    rows f32 [M*k][N] at route ids."""
    M, K = x_q.shape
    E, N, _ = w_q.shape
    _call("moe_grouped_gemm_gather", _ptr(x_q), _ptr(x_scales), M, k, K, _ptr(w_q),
          _ptr(w_scales), E, N, _ptr(tasks), _ptr(ntasks), tasks.shape[0], chunk_rows,
          _ptr(sorted_route_ids), _ptr(rows), _ptr(queue), sched, _stream(stream))


def forward_kernels(M: int, E: int, k: int, K: int, N: int, chunk_rows: int = 0,
                    flags: int = 0) -> int:
    """Kernels moe_forward_ex launches for these arguments: 2 or 3 at small batches (route
    inside the GEMM or as a kernel of its own), 4 with LDS-tiled chunks, 5 staged."""
    n = lib().moe_forward_kernels(M, E, k, K, N, chunk_rows, flags)
    if n < 0:
        raise MoeError("moe_forward_kernels", n)
    return n


def route_grouped_gemm(logits, x, k: int, softcap: float, w_q, w_scales, topk_ids,
                       topk_weights, route_words, status, rows, stream=None):
    """The route inside the small-batch grouped FP8 GEMM (moe_route_grouped_gemm)."""
    M, E = logits.shape
    K = x.shape[1]
    N = w_q.shape[1]
    _call("moe_route_grouped_gemm", _ptr(logits), _ptr(x), M, E, k, K, softcap, _ptr(w_q),
          _ptr(w_scales), N, _ptr(topk_ids), _ptr(topk_weights), _ptr(route_words),
          _ptr(status), _ptr(rows), _stream(stream))


def grouped_gemm_routed(x, topk_ids, E: int, w_q, w_scales, rows, counts=None, offsets=None,
                        stream=None):
    """Small-batch grouped FP8 GEMM straight from routed ids (moe_grouped_gemm_routed)."""
    M, K = x.shape
    k = topk_ids.shape[1]
    N = w_q.shape[1]
    _call("moe_grouped_gemm_routed", _ptr(x), _ptr(topk_ids), M, k, E, K, _ptr(w_q),
          _ptr(w_scales), N, _ptr(rows), _ptr(counts), _ptr(offsets), _stream(stream))


def scatter(rows, topk_weights, topk_ids, E: int, out, route_slots=None, stream=None):
    M, k = topk_ids.shape
    N = rows.shape[1]
    _call("moe_scatter", _ptr(rows), _ptr(route_slots), _ptr(topk_weights), _ptr(topk_ids), M,
          k, E, N, _ptr(out), _stream(stream))


def forward_workspace_bytes(M: int, E: int, k: int, K: int, N: int) -> int:
    v = lib().moe_forward_workspace_bytes(M, E, k, K, N)
    if v == 0:
        raise MoeError("moe_forward_workspace_bytes", MOE_E_INVAL)
    return v


def forward_workspace_offset(M: int, E: int, k: int, K: int, N: int, which: int) -> int:
    return lib().moe_forward_workspace_offset(M, E, k, K, N, which)


def forward(logits, x, w_q, w_scales, k: int, softcap: float, out, workspace,
            chunk_rows: int = 0, flags: int = 0, stream=None):
    M, E = logits.shape
    K = x.shape[1]
    N = w_q.shape[1]
    _call("moe_forward_ex", _ptr(logits), _ptr(x), _ptr(w_q), _ptr(w_scales), M, E, k, K, N,
          softcap, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
          chunk_rows, flags, _stream(stream))


def router_logits(x, w_gate, logits, stream=None):
    """logits f32 [M][E] = x bf16 [M][H] . w_gate bf16 [E][H]^T (moe_router_logits)."""
    M, H = x.shape
    E = w_gate.shape[0]
    _call("moe_router_logits", _ptr(x), M, H, _ptr(w_gate), E, _ptr(logits), _stream(stream))


def forward_noalloc(logits, x, w_q, w_scales, k: int, softcap: float, out, stream=None):
    M, E = logits.shape
    K = x.shape[1]
    N = w_q.shape[1]
    _call("moe_forward_noalloc", _ptr(logits), _ptr(x), _ptr(w_q), _ptr(w_scales), M, E, k, K,
          N, softcap, _ptr(out), _stream(stream))


def sort_gather_bf16(x, topk_ids, E: int, cursors, sorted_route_ids, a, route_slots=None,
                     stream=None):
    M, K = x.shape
    k = topk_ids.shape[1]
    _call("moe_sort_gather_bf16", _ptr(x), M, K, _ptr(topk_ids), k, E, _ptr(cursors),
          _ptr(sorted_route_ids), _ptr(route_slots), _ptr(a), _stream(stream))


def ffn_workspace_bytes(M: int, E: int, k: int, H: int, F: int) -> int:
    v = lib().moe_ffn_workspace_bytes(M, E, k, H, F)
    if v == 0:
        raise MoeError("moe_ffn_workspace_bytes", MOE_E_INVAL)
    return v


def ffn_workspace_offset(M: int, E: int, k: int, H: int, F: int, which: int) -> int:
    return lib().moe_ffn_workspace_offset(M, E, k, H, F, which)


def ffn_forward(logits, x, w_up, w_down, k: int, softcap: float, out, workspace,
                chunk_rows: int = 0, flags: int = 0, stream=None):
    M, E = logits.shape
    H = x.shape[1]
    F = w_down.shape[2]
    _call("moe_ffn_forward", _ptr(logits), _ptr(x), _ptr(w_up), _ptr(w_down), M, E, k, H, F,
          softcap, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
          chunk_rows, flags, _stream(stream))


def swiglu_quant(h, a_q, a_scales, stream=None):
    """h f32 [rows][2I] -> a_q uint8 [rows][I], a_scales f32 [I/128][rows]."""
    rows, I2 = h.shape
    _call("moe_swiglu_quant", _ptr(h), rows, I2 // 2, _ptr(a_q), _ptr(a_scales),
          _stream(stream))


def mlp_workspace_bytes(M: int, E: int, k: int, H: int, I: int) -> int:
    v = lib().moe_mlp_workspace_bytes(M, E, k, H, I)
    if v == 0:
        raise MoeError("moe_mlp_workspace_bytes", MOE_E_INVAL)
    return v


def mlp_forward_kernels(M: int, E: int, k: int, H: int, I: int, chunk_rows: int = 0) -> int:
    v = lib().moe_mlp_forward_kernels(M, E, k, H, I, chunk_rows)
    if v < 0:
        raise MoeError("moe_mlp_forward_kernels", v)
    return v


def mlp_workspace_offset(M: int, E: int, k: int, H: int, I: int, which: int) -> int:
    return lib().moe_mlp_workspace_offset(M, E, k, H, I, which)


def mlp_forward(logits, x, w1_q, w1_scales, w2_q, w2_scales, k: int, softcap: float, out,
                workspace, chunk_rows: int = 0, stream=None):
    M, E = logits.shape
    H = x.shape[1]
    I = w2_q.shape[2]
    _call("moe_mlp_forward", _ptr(logits), _ptr(x), _ptr(w1_q), _ptr(w1_scales), _ptr(w2_q),
          _ptr(w2_scales), M, E, k, H, I, softcap, _ptr(out), _ptr(workspace),
          workspace.numel() * workspace.element_size(), chunk_rows, _stream(stream))
