"""ctypes front end of the plain C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only users.  The product path never imports this module, and this
module never imports the product package: inputs arrive as numpy arrays.

Every function takes and returns numpy arrays with the layouts documented in ``oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

# Single-threaded, IEEE arithmetic: no fast-math and no FMA contraction.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc and return its path."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        F = ctypes.c_float
        sig = {
            "orc_e4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_e4m3_encode": (ctypes.c_uint8, [F]),
            "orc_e4m3_encode_bruteforce": (ctypes.c_uint8, [F]),
            "orc_bf16_from_double": (ctypes.c_uint16, [ctypes.c_double]),
            "orc_bf16_value": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_route": (I, [P, I, I, I, F, P, P]),
            "orc_layout": (I, [P, I, I, I, P, P]),
            "orc_tasks": (I, [P, P, I, I, I, P, I]),
            "orc_quant_act": (I, [P, I, I, P, P]),
            "orc_quant_weights": (I, [P, I, I, I, P, P]),
            "orc_sort_gather": (I, [P, I, I, I, P, P, P, I, P, P, P]),
            "orc_gemm_fp8": (I, [P, P, I, P, P, P, I, I, I, P]),
            "orc_scatter": (I, [P, P, I, P, I, I, I, P, P]),
            "orc_forward": (I, [P, P, P, P, I, I, I, I, I, F, P, P, P, P, P, P, P, P, P, P]),
            "orc_forward_tokens": (I, [P, P, P, P, I, I, I, I, I, F, P, I, P, P]),
            "orc_gemm_bf16": (I, [P, I, I, P, I, P, I, P, I, P, P]),
            "orc_router_logits": (I, [P, I, I, P, I, P, P]),
            "orc_ffn_tokens": (I, [P, P, P, P, I, I, I, I, I, F, P, I, P, P]),
            "orc_swiglu_f32": (I, [P, I, I, P]),
            "orc_quant_rows_f32": (I, [P, I, I, P, P]),
            "orc_mlp_tokens": (I, [P, P, P, P, P, P, I, I, I, I, I, F, P, I, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (rc={rc})")


# ---- number formats -------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def e4m3_encode(y: float) -> int:
    return lib().orc_e4m3_encode(y)


def e4m3_encode_bruteforce(y: float) -> int:
    return lib().orc_e4m3_encode_bruteforce(y)


def e4m3_encode_array(y: np.ndarray) -> np.ndarray:
    f = lib().orc_e4m3_encode
    return np.array([f(float(v)) for v in np.asarray(y, np.float32).ravel()], np.uint8)


def e4m3_decode_table() -> np.ndarray:
    return np.array([lib().orc_e4m3_value(c) for c in range(256)], np.float64)


def bf16_from_double(v: float) -> int:
    return lib().orc_bf16_from_double(v)


def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(bits)


# ---- path steps -----------------------------------------------------------------------

def route(logits: np.ndarray, k: int, cap: float):
    logits = _c(logits, np.float32)
    M, E = logits.shape
    ids = np.zeros((M, k), np.int32)
    w = np.zeros((M, k), np.float32)
    _check(lib().orc_route(_p(logits), M, E, k, cap, _p(ids), _p(w)), "orc_route")
    return ids, w


def layout(ids: np.ndarray, E: int):
    ids = _c(ids, np.int32)
    M, k = ids.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    _check(lib().orc_layout(_p(ids), M, k, E, _p(counts), _p(offsets)), "orc_layout")
    return counts, offsets


def tasks(counts: np.ndarray, offsets: np.ndarray, n_blocks: int, chunk_rows: int) -> np.ndarray:
    counts = _c(counts, np.int32)
    offsets = _c(offsets, np.int32)
    E = counts.shape[0]
    cap = int(sum((int(c) + chunk_rows - 1) // chunk_rows for c in counts)) * n_blocks + 1
    out = np.zeros((cap, 4), np.int32)
    n = lib().orc_tasks(_p(counts), _p(offsets), E, n_blocks, chunk_rows, _p(out), cap)
    if n < 0:
        raise ValueError("orc_tasks failed")
    return out[:n].copy()


def quant_act(x_bf16: np.ndarray):
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    q = np.zeros((M, K), np.uint8)
    s = np.zeros((M, K // 128), np.float32)
    _check(lib().orc_quant_act(_p(x), M, K, _p(q), _p(s)), "orc_quant_act")
    return q, s


def quant_weights(w: np.ndarray):
    w = _c(w, np.float32)
    E, N, K = w.shape
    q = np.zeros((E, N, K), np.uint8)
    s = np.zeros((E, N // 128, K // 128), np.float32)
    _check(lib().orc_quant_weights(_p(w), E, N, K, _p(q), _p(s)), "orc_quant_weights")
    return q, s


def sort_gather(ids, offsets, q, scales):
    ids = _c(ids, np.int32)
    offsets = _c(offsets, np.int32)
    q = _c(q, np.uint8)
    scales = _c(scales, np.float32)
    M, k = ids.shape
    E = offsets.shape[0] - 1
    K = q.shape[1]
    R = M * k
    sorted_ids = np.zeros(R, np.int32)
    a_q = np.zeros((R, K), np.uint8)
    a_s = np.zeros((K // 128, R), np.float32)
    _check(lib().orc_sort_gather(_p(ids), M, k, E, _p(offsets), _p(q), _p(scales), K,
                                 _p(sorted_ids), _p(a_q), _p(a_s)), "orc_sort_gather")
    return sorted_ids, a_q, a_s


def gemm_fp8(a_q, a_scales, w_q, w_scales, offsets) -> np.ndarray:
    a_q = _c(a_q, np.uint8)
    a_scales = _c(a_scales, np.float32)
    w_q = _c(w_q, np.uint8)
    w_scales = _c(w_scales, np.float32)
    offsets = _c(offsets, np.int32)
    rows, K = a_q.shape
    E, N, _ = w_q.shape
    C = np.zeros((rows, N), np.float64)
    _check(lib().orc_gemm_fp8(_p(a_q), _p(a_scales), rows, _p(w_q), _p(w_scales),
                              _p(offsets), E, N, K, _p(C)), "orc_gemm_fp8")
    return C


def scatter(C, sorted_ids, weights, M: int):
    C = _c(C, np.float64)
    sorted_ids = _c(sorted_ids, np.int32)
    weights = _c(weights, np.float32)
    rows, N = C.shape
    k = weights.shape[1]
    y64 = np.zeros((M, N), np.float64)
    y = np.zeros((M, N), np.uint16)
    _check(lib().orc_scatter(_p(C), _p(sorted_ids), rows, _p(weights), M, k, N, _p(y64), _p(y)),
           "orc_scatter")
    return y, y64


def forward(logits, x_bf16, w_q, w_scales, k: int, cap: float, intermediates: bool = False):
    logits = _c(logits, np.float32)
    x = _c(x_bf16, np.uint16)
    w_q = _c(w_q, np.uint8)
    w_scales = _c(w_scales, np.float32)
    M, E = logits.shape
    K = x.shape[1]
    N = w_q.shape[1]
    R = M * k
    y = np.zeros((M, N), np.uint16)
    y64 = np.zeros((M, N), np.float64)
    out = {}
    if intermediates:
        out = dict(ids=np.zeros((M, k), np.int32), weights=np.zeros((M, k), np.float32),
                   counts=np.zeros(E, np.int32), offsets=np.zeros(E + 1, np.int32),
                   sorted_route_ids=np.zeros(R, np.int32), a_q=np.zeros((R, K), np.uint8),
                   a_scales=np.zeros((K // 128, R), np.float32),
                   C=np.zeros((R, N), np.float64))
    g = out.get
    _check(lib().orc_forward(_p(logits), _p(x), _p(w_q), _p(w_scales), M, E, k, K, N, cap,
                             _p(y), _p(y64), _p(g("ids")), _p(g("weights")), _p(g("counts")),
                             _p(g("offsets")), _p(g("sorted_route_ids")), _p(g("a_q")),
                             _p(g("a_scales")), _p(g("C"))), "orc_forward")
    out["y"] = y
    out["y64"] = y64
    return out


def forward_tokens(logits, x_bf16, w_q, w_scales, k: int, cap: float, tokens):
    logits = _c(logits, np.float32)
    x = _c(x_bf16, np.uint16)
    w_q = _c(w_q, np.uint8)
    w_scales = _c(w_scales, np.float32)
    tokens = _c(tokens, np.int32)
    M, E = logits.shape
    K = x.shape[1]
    N = w_q.shape[1]
    n = tokens.shape[0]
    y = np.zeros((n, N), np.uint16)
    y64 = np.zeros((n, N), np.float64)
    _check(lib().orc_forward_tokens(_p(logits), _p(x), _p(w_q), _p(w_scales), M, E, k, K, N,
                                    cap, _p(tokens), n, _p(y), _p(y64)), "orc_forward_tokens")
    return y, y64


def gemm_bf16(A, W, offsets, rows_list=None):
    A = _c(A, np.uint16)
    W = _c(W, np.uint16)
    offsets = _c(offsets, np.int32)
    rows, K = A.shape
    E, N, _ = W.shape
    rl = None if rows_list is None else _c(rows_list, np.int32)
    n = rows if rl is None else rl.shape[0]
    out = np.zeros((n, N), np.uint16)
    out64 = np.zeros((n, N), np.float64)
    _check(lib().orc_gemm_bf16(_p(A), rows, K, _p(W), N, _p(offsets), E, _p(rl),
                               0 if rl is None else n, _p(out), _p(out64)), "orc_gemm_bf16")
    return out, out64


def router_logits(x_bf16, w_gate_bf16):
    """Router projection: logits f32 [M][E] and their double sums for x [M][H], w_gate [E][H]
    (both bf16 bits)."""
    x = _c(x_bf16, np.uint16)
    wg = _c(w_gate_bf16, np.uint16)
    M, H = x.shape
    E = wg.shape[0]
    logits = np.zeros((M, E), np.float32)
    logits64 = np.zeros((M, E), np.float64)
    _check(lib().orc_router_logits(_p(x), M, H, _p(wg), E, _p(logits), _p(logits64)),
           "orc_router_logits")
    return logits, logits64


def ffn_tokens(logits, x_bf16, w_up, w_down, k: int, cap: float, tokens=None):
    logits = _c(logits, np.float32)
    x = _c(x_bf16, np.uint16)
    w_up = _c(w_up, np.uint16)
    w_down = _c(w_down, np.uint16)
    M, E = logits.shape
    H = x.shape[1]
    F = w_down.shape[2]
    tl = None if tokens is None else _c(tokens, np.int32)
    n = M if tl is None else tl.shape[0]
    y = np.zeros((n, H), np.uint16)
    y64 = np.zeros((n, H), np.float64)
    _check(lib().orc_ffn_tokens(_p(logits), _p(x), _p(w_up), _p(w_down), M, E, k, H, F, cap,
                                _p(tl), 0 if tl is None else n, _p(y), _p(y64)),
           "orc_ffn_tokens")
    return y, y64


def swiglu_f32(h: np.ndarray) -> np.ndarray:
    """act = fp32(silu(g) * u) for h [rows][2I] (gate columns first)."""
    h = _c(h, np.float64)
    rows, I2 = h.shape
    act = np.zeros((rows, I2 // 2), np.float32)
    _check(lib().orc_swiglu_f32(_p(h), rows, I2 // 2, _p(act)), "orc_swiglu_f32")
    return act


def quant_rows_f32(v: np.ndarray):
    v = _c(v, np.float32)
    rows, K = v.shape
    q = np.zeros((rows, K), np.uint8)
    s = np.zeros((rows, K // 128), np.float32)
    _check(lib().orc_quant_rows_f32(_p(v), rows, K, _p(q), _p(s)), "orc_quant_rows_f32")
    return q, s


def mlp_tokens(logits, x_bf16, w1_q, w1_scales, w2_q, w2_scales, k: int, cap: float,
               tokens=None):
    logits = _c(logits, np.float32)
    x = _c(x_bf16, np.uint16)
    w1_q = _c(w1_q, np.uint8)
    w1_scales = _c(w1_scales, np.float32)
    w2_q = _c(w2_q, np.uint8)
    w2_scales = _c(w2_scales, np.float32)
    M, E = logits.shape
    H = x.shape[1]
    I = w2_q.shape[2]
    tl = None if tokens is None else _c(tokens, np.int32)
    n = M if tl is None else tl.shape[0]
    y = np.zeros((n, H), np.uint16)
    y64 = np.zeros((n, H), np.float64)
    _check(lib().orc_mlp_tokens(_p(logits), _p(x), _p(w1_q), _p(w1_scales), _p(w2_q),
                                _p(w2_scales), M, E, k, H, I, cap, _p(tl),
                                0 if tl is None else n, _p(y), _p(y64)), "orc_mlp_tokens")
    return y, y64
