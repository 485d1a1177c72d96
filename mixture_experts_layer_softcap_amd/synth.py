"""Seeded synthetic inputs for the fused MoE forward and the grouped GEMMs.

This module only draws random numbers and lays them out; it holds none of the forward's
arithmetic (no routing, quantisation, layout or GEMM).  Both the HIP path's tests and
benchmark and the CPU oracle's tests take their inputs from here.

Generator: ``numpy.random.Generator(PCG64(seed))``, drawing in a fixed order:
logits (float32 N(0,1)), then activations x (float32 N(0,1) rounded to bf16), then the
expert weights (0.02 * float32 N(0,1)), then any draws for the row distribution.

Workload shapes come from the pages: the Qwen3.5-35B-A3B-shaped layer of the Fused MoE FP8
tutorial's problem table (M=128 tokens, 256 experts, top-8, K=2048, N=512); the H200
grouped-GEMM notes' benchmark design (H=3072, I=1536, 16 experts, top-8, random /
balanced / skewed expert-row distributions); and the Weave blog's Mixtral-like layer
(8 experts, top-2, hidden 4096, FFN 1024, skewed expert loads).
"""
from __future__ import annotations

import numpy as np

SOFTCAP = 30.0


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even, via torch's cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- expert-load biases added to the router logits ------------------------------------

def zipf_bias(E: int, amplitude: float = 2.0, s: float = 1.2) -> np.ndarray:
    """b_e = amplitude * (e+1)^-s: a Zipf(s) tilt over the expert index."""
    e = np.arange(E, dtype=np.float64)
    return (amplitude * (e + 1.0) ** (-s)).astype(np.float32)


def log_bias(E: int, slope: float = 1.1) -> np.ndarray:
    """b_e = -slope * ln(e+1): about a 15x max/min expert load at E=8, top-2."""
    e = np.arange(E, dtype=np.float64)
    return (-slope * np.log(e + 1.0)).astype(np.float32)


# ---- fused FP8 forward inputs ---------------------------------------------------------

FUSED_WORKLOADS = {
    # small correctness case: 8 tokens, 16 experts, top-2, K=N=256
    "fused_fp8_M8_E16_k2_K256_N256": dict(M=8, E=16, k=2, K=256, N=256, bias=None),
    # Qwen3.5-35B-A3B-shaped layer, uniform routing (about 4 rows per expert)
    "fused_fp8_M128_E256_k8_K2048_N512": dict(M=128, E=256, k=8, K=2048, N=512, bias=None),
    # same layer, more tokens, Zipf-skewed routing
    "fused_fp8_M1024_E256_k8_K2048_N512_zipf": dict(M=1024, E=256, k=8, K=2048, N=512,
                                                    bias="zipf"),
    "fused_fp8_M4096_E256_k8_K2048_N512_zipf": dict(M=4096, E=256, k=8, K=2048, N=512,
                                                    bias="zipf"),
}


def fused_inputs(M: int, E: int, k: int, K: int, N: int, seed: int = 0, bias=None,
                 weights: bool = True):
    """Return dict(logits f32 [M,E], x bf16 bits [M,K], w f32 [E,N,K] or None)."""
    g = rng(seed)
    logits = g.standard_normal((M, E), dtype=np.float32)
    if isinstance(bias, str):
        b = {"zipf": zipf_bias, "log": log_bias}[bias](E)
        logits = (logits + b[None, :]).astype(np.float32)
    elif bias is not None:
        logits = (logits + np.asarray(bias, np.float32)[None, :]).astype(np.float32)
    x = bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    w = None
    if weights:
        w = g.standard_normal((E, N, K), dtype=np.float32)
        w *= np.float32(0.02)
    return dict(logits=logits, x=x, w=w)


def workload_inputs(name: str, seed: int = 0, weights: bool = True):
    cfg = dict(FUSED_WORKLOADS[name])
    bias = cfg.pop("bias")
    d = fused_inputs(seed=seed, bias=bias, weights=weights, **cfg)
    d.update(cfg)
    d["cap"] = SOFTCAP
    return d


# ---- FP8 expert MLP inputs ---------------------------------------------------------------

# exponent fields 8..15 of the E4M3 weight codes, weighted like |N(0, 1)| * 112 (4 sigma near
# the largest finite value 448): counts out of 256 per field
_E4M3_EXP_COUNTS = [(8, 5), (9, 10), (10, 20), (11, 41), (12, 64), (13, 64), (14, 39), (15, 13)]
_E4M3_EXP_EDGES = np.cumsum([c for _, c in _E4M3_EXP_COUNTS])[:-1]   # 7 thresholds in 0..255


def fp8_weight_codes(shape, g: np.random.Generator) -> np.ndarray:
    """Seeded E4M3 codes from one random 16-bit draw each: bits 0-7 pick the exponent field
    8 + #(edges <= byte), bits 8-10 the mantissa, bit 11 the sign (the NaN pattern 0x7F is
    moved to 0x7E).  Drawn one leading-axis slice at a time (small temporaries)."""
    out = np.empty(shape, np.uint8)
    for i in range(shape[0]):
        r = g.integers(0, 1 << 16, size=shape[1:], dtype=np.uint16)
        b = r.view(np.uint8).reshape(*shape[1:], 2)
        lo, hi = b[..., 0], b[..., 1]                 # little-endian: bits 0-7, 8-15
        field = np.full(shape[1:], 8, np.uint8)
        for edge in _E4M3_EXP_EDGES:
            field += lo >= np.uint8(edge)
        code = (field << np.uint8(3)) | (hi & np.uint8(7))
        code[code == 0x7F] = 0x7E
        code |= (hi & np.uint8(8)) << np.uint8(4)
        out[i] = code
    return out


def fp8_block_scales(shape, g: np.random.Generator, base: float = 0.02 / 112) -> np.ndarray:
    """Per 128x128-block scales around `base` (a factor 2^U(-0.5, 0.5) per block)."""
    return (base * np.exp2(g.uniform(-0.5, 0.5, size=shape))).astype(np.float32)


MLP_WORKLOADS = {
    "mlp_fp8_M128_E256_k8_H2048_I512": dict(M=128, E=256, k=8, H=2048, I=512),
}


def mlp_inputs(M: int, E: int, k: int, H: int, I: int, seed: int = 0):
    """Return dict(logits f32 [M,E], x bf16 bits [M,H], w1_q uint8 [E,2I,H] (gate rows then
    up rows), w1_s f32 [E,2I/128,H/128], w2_q uint8 [E,H,I], w2_s f32 [E,H/128,I/128])."""
    g = rng(seed)
    logits = g.standard_normal((M, E), dtype=np.float32)
    x = bf16_bits(g.standard_normal((M, H), dtype=np.float32))
    w1_q = fp8_weight_codes((E, 2 * I, H), g)
    w1_s = fp8_block_scales((E, 2 * I // 128, H // 128), g)
    w2_q = fp8_weight_codes((E, H, I), g)
    w2_s = fp8_block_scales((E, H // 128, I // 128), g)
    return dict(logits=logits, x=x, w1_q=w1_q, w1_s=w1_s, w2_q=w2_q, w2_s=w2_s, M=M, E=E,
                k=k, H=H, I=I, cap=SOFTCAP)


# ---- grouped BF16 GEMM inputs ----------------------------------------------------------

def row_counts(rows: int, E: int, dist: str, g: np.random.Generator) -> np.ndarray:
    """Per-expert row counts summing to `rows`.

    balanced: floor(rows/E) each, the remainder to the lowest experts;
    random:   Dirichlet(alpha=1) shares;  skewed: Dirichlet(alpha=0.3) shares;
    shares are turned into integers by largest-remainder rounding (zero rows can occur).
    """
    if dist == "balanced":
        c = np.full(E, rows // E, np.int64)
        c[: rows % E] += 1
        return c.astype(np.int32)
    alpha = {"random": 1.0, "skewed": 0.3}[dist]
    p = g.dirichlet(np.full(E, alpha))
    raw = p * rows
    c = np.floor(raw).astype(np.int64)
    short = rows - int(c.sum())
    order = np.argsort(-(raw - c), kind="stable")
    c[order[:short]] += 1
    return c.astype(np.int32)


def grouped_gemm_inputs(rows: int, E: int, N: int, K: int, dist: str, seed: int = 0):
    """A bf16 [rows,K] ~N(0,1); W bf16 [E,N,K] ~0.02 N(0,1); expert-contiguous rows."""
    g = rng(seed)
    A = bf16_bits(g.standard_normal((rows, K), dtype=np.float32))
    W = g.standard_normal((E, N, K), dtype=np.float32)
    W *= np.float32(0.02)
    W = bf16_bits(W)
    counts = row_counts(rows, E, dist, g)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return dict(A=A, W=W, counts=counts, offsets=offsets)


def ffn_inputs(T: int, E: int, H: int, F: int, seed: int = 0, skewed: bool = True,
               weights: bool = True):
    """Mixtral-like layer inputs: logits [T,E] (+ -1.1 ln(e+1) when skewed), x bf16 [T,H],
    w_up bf16 [E,2F,H] (gate rows then up rows), w_down bf16 [E,H,F]."""
    g = rng(seed)
    logits = g.standard_normal((T, E), dtype=np.float32)
    if skewed:
        logits = (logits + log_bias(E)[None, :]).astype(np.float32)
    x = bf16_bits(g.standard_normal((T, H), dtype=np.float32))
    w_up = w_down = None
    if weights:
        w_up = g.standard_normal((E, 2 * F, H), dtype=np.float32)
        w_up *= np.float32(0.02)
        w_up = bf16_bits(w_up)
        w_down = g.standard_normal((E, H, F), dtype=np.float32)
        w_down *= np.float32(0.02)
        w_down = bf16_bits(w_down)
    return dict(logits=logits, x=x, w_up=w_up, w_down=w_down)




def router_inputs(M: int, H: int, E: int, seed: int = 0):
    """Hidden states and gate weights of the router projection: x bf16 [M,H] ~ N(0,1) and
    w_gate bf16 [E,H] ~ N(0, 1/H), so the logits x . w_gate^T have about unit variance like
    the directly drawn logits of the other workloads."""
    g = rng(seed)
    x = bf16_bits(g.standard_normal((M, H), dtype=np.float32))
    wg = g.standard_normal((E, H), dtype=np.float32)
    wg *= np.float32(1.0 / np.sqrt(H))
    return dict(x=x, w_gate=bf16_bits(wg))
