"""Helpers shared by the GPU parity tests: numpy <-> device tensors, the tolerance rule,
segment canonicalisation, cached full-size workloads."""
from __future__ import annotations

import functools

import numpy as np
import torch

from mixture_experts_layer_softcap_amd import synth

DEV = "cuda:0"

# Tolerances: the BF16 output bar (relative Frobenius error and per-element error against
# the rms of the reference); routing weights are fp32 transcendentals.
REL_FRO = 5e-3
ELEM_RMS = 2e-2
WEIGHT_RTOL = 1e-5
# fp32 rows of the FP8 grouped GEMM against the exact (double) oracle.  The matrix core sums
# the 128 products of one scale block at reduced precision (about 2^-13 of the block's
# magnitude was measured); the kernel promotes every block to fp32, so the error stays one
# block's rounding per block.
GEMM_F32_REL_FRO = 1e-4
GEMM_F32_ELEM_RMS = 5e-4


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_np(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def zeros(shape, dtype) -> torch.Tensor:
    return torch.zeros(shape, dtype=dtype, device=DEV)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(np.asarray(bits).view(np.uint16)).astype(np.float64)


def assert_bf16_close(y_bits: np.ndarray, ref64: np.ndarray, what: str = ""):
    y = bf16_f64(y_bits)
    ref = np.asarray(ref64, np.float64)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    fro = float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))
    worst = float(np.abs(y - ref).max()) if y.size else 0.0
    assert fro <= REL_FRO, f"{what}: relative Frobenius error {fro:.3e} > {REL_FRO}"
    assert worst <= ELEM_RMS * rms, f"{what}: max |d| {worst:.3e} > {ELEM_RMS}*rms ({rms:.3e})"


def assert_gemm_f32_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    ref = np.asarray(ref, np.float64)
    d = np.asarray(got, np.float64) - ref
    rms = float(np.sqrt(np.mean(ref ** 2)))
    fro = float(np.linalg.norm(d) / np.linalg.norm(ref))
    assert fro <= GEMM_F32_REL_FRO, f"{what}: relative Frobenius {fro:.3e}"
    assert np.abs(d).max() <= GEMM_F32_ELEM_RMS * rms, f"{what}: max |d| {np.abs(d).max():.3e}"


def canonical_segments(sorted_ids: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Permutation that sorts each expert segment by route id (the oracle's order)."""
    perm = np.arange(sorted_ids.shape[0])
    for e in range(offsets.shape[0] - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        perm[a:b] = a + np.argsort(sorted_ids[a:b], kind="stable")
    return perm


@functools.lru_cache(maxsize=None)
def workload(name: str):
    """Full-size seeded inputs plus the oracle-quantised weights (computed once)."""
    import oracle

    d = synth.workload_inputs(name)
    w_q, w_s = oracle.quant_weights(d["w"])
    d["w_q"], d["w_s"] = w_q, w_s
    return d
