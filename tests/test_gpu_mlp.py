"""GPU parity of the FP8 expert MLP (moe_swiglu_quant, moe_mlp_forward) against the oracle.

The activation requantiser is bit-exact where silu(g) * u is exact in fp32 (gates far in
silu's identity range, products of E4M3 values and powers of two, all-zero blocks).  On
random rows the device forms silu(g) * u in fp32 (two roundings and expf) and the oracle in
double (one rounding), so a code may land one E4M3 step away where the value sits on a
rounding boundary: scales are held to a few fp32 ulps and the dequantised values to one E4M3
step, with at most 1 % of codes differing.

The layer output is held to the BF16 output bar in aggregate (relative Frobenius 5e-3), but not
element by element: the first GEMM's fp32 rows carry the matrix core's ~2^-13 per-block
error, so about 0.2 % of the activation codes land one E4M3 step (<= 2^-3 of the value) away
from the oracle's, and each such flip moves every output of its route by that step times the
weight.  One flip changes an output by at most 2^-3 * (|a|/rms a) * (|w|/rms w) / sqrt(I) of
its rms: with |a| <= 8 rms, |w| <= 448/123 rms and I >= 256 that is <= 0.23, and 0.15 covers
the combine over k routes of unit-sum weights in practice.  So elements are held to 2e-2 rms
for all but 0.5 % of them and to 0.15 rms everywhere (MLP_*).
"""
import numpy as np
import pytest
import torch

import oracle as orc
from mixture_experts_layer_softcap_amd import moe, synth

from gpu_util import (REL_FRO, assert_bf16_close, bf16_f64, oracle_gemm_rows_by_expert,
                      oracle_rows_parallel, to_dev, to_np, zeros)

pytestmark = pytest.mark.gpu

CAP = synth.SOFTCAP
MLP_ELEM_RMS = 2e-2          # per-element bar for all but MLP_OUTLIER_FRAC of the elements
MLP_OUTLIER_FRAC = 5e-3
MLP_MAX_RMS = 0.15           # every element


def assert_mlp_close(y_bits, ref64, what=""):
    assert_bf16_close_fro(y_bits, ref64, what)
    y = bf16_f64(y_bits)
    ref = np.asarray(ref64, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    d = np.abs(y - ref)
    frac = float((d > MLP_ELEM_RMS * rms).mean())
    assert frac <= MLP_OUTLIER_FRAC, f"{what}: {frac:.4f} of elements beyond {MLP_ELEM_RMS} rms"
    assert d.max() <= MLP_MAX_RMS * rms, f"{what}: max |d| {d.max():.3e} vs rms {rms:.3e}"


def assert_bf16_close_fro(y_bits, ref64, what=""):
    y = bf16_f64(y_bits)
    ref = np.asarray(ref64, np.float64)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    fro = float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))
    assert fro <= REL_FRO, f"{what}: relative Frobenius error {fro:.3e} > {REL_FRO}"


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    orc.build(force=False)
    assert moe.device_check() == moe.MOE_OK


def gpu_swiglu_quant(h):
    rows, I2 = h.shape
    I = I2 // 2
    a_q = zeros((rows, I), torch.uint8)
    a_s = zeros((I // 128, rows), torch.float32)
    moe.swiglu_quant(to_dev(h.astype(np.float32)), a_q, a_s)
    torch.cuda.synchronize()
    return to_np(a_q), to_np(a_s)


def oracle_swiglu_quant(h):
    act = orc.swiglu_f32(h.astype(np.float64))
    return orc.quant_rows_f32(act)


@pytest.mark.parametrize("I", [128, 384, 640])
def test_swiglu_quant_exact_rows(I):
    g = np.random.default_rng(I)
    rows = 37
    vals = np.array([0.0, 1.0, 0.5, 0.25, 0.75, 1.5, 3.0, 0.125, 0.0625, 448.0], np.float32)
    gate = g.choice(np.array([64.0, 128.0, 256.0, 1024.0], np.float32), (rows, I))
    up = g.choice(vals, (rows, I)) * g.choice(np.array([-1, 1], np.float32), (rows, I))
    up *= np.exp2(g.integers(-6, 4, (rows, 1))).astype(np.float32)
    gate[3, :] = 0.0                                  # act = +-0: scale 0, signed zero codes
    up[3, :] = np.where(np.arange(I) % 2, -1.0, 2.0)
    gate[5, 128:256 if I > 128 else 128] = 0.0        # one zero block inside a live row
    h = np.concatenate([gate, up], axis=1)
    q, s = gpu_swiglu_quant(h)
    rq, rs = oracle_swiglu_quant(h)
    np.testing.assert_array_equal(s.T.view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(q, rq)
    assert rs[3].tolist() == [0.0] * (I // 128)
    assert set(np.unique(q[3]).tolist()) <= {0x00, 0x80}


@pytest.mark.parametrize("rows,I", [(1, 128), (53, 512), (200, 1536)])
def test_swiglu_quant_random_rows(rows, I):
    g = np.random.default_rng(rows + I)
    h = (g.standard_normal((rows, 2 * I)) * 2.0).astype(np.float32)
    q, s = gpu_swiglu_quant(h)
    rq, rs = oracle_swiglu_quant(h)
    s = s.T
    np.testing.assert_allclose(s, rs, rtol=5e-7, atol=0)
    dq = orc.e4m3_decode_table()
    got = dq[q] * np.repeat(s.astype(np.float64), 128, 1)
    ref = dq[rq] * np.repeat(rs.astype(np.float64), 128, 1)
    step = 2.0 ** -3 * np.abs(ref) + 2.0 ** -9 * np.repeat(rs.astype(np.float64), 128, 1)
    assert (np.abs(got - ref) <= step * 1.0001).all()
    assert (q != rq).mean() <= 0.01


def test_swiglu_quant_zero_rows_is_a_no_op():
    a_q = zeros((1, 128), torch.uint8)
    a_s = zeros((1, 1), torch.float32)
    h = zeros((0, 256), torch.float32)
    moe.swiglu_quant(h, a_q, a_s)
    torch.cuda.synchronize()
    assert int(a_q.sum()) == 0 and float(a_s.sum()) == 0.0


def gpu_mlp(d, chunk=0, reps=1):
    M, H = d["x"].shape
    E, k, I = d["E"], d["k"], d["I"]
    args = [to_dev(d[n]) for n in ("logits", "x", "w1_q", "w1_s", "w2_q", "w2_s")]
    ws = zeros(moe.mlp_workspace_bytes(M, E, k, H, I), torch.uint8)
    outs = []
    for _ in range(reps):
        out = zeros((M, H), torch.int16)
        moe.mlp_forward(*args, k, CAP, out, ws, chunk_rows=chunk)
        torch.cuda.synchronize()
        outs.append(to_np(out, np.uint16))
    return outs, ws


def ws_part(ws, d, which, dtype, n):
    M, H = d["x"].shape
    off = moe.mlp_workspace_offset(M, d["E"], d["k"], H, d["I"], which)
    size = np.dtype(dtype).itemsize * n
    return to_np(ws[off:off + size]).view(dtype)


@pytest.mark.parametrize("M,E,k,H,I,chunk,kernels", [
    (8, 16, 2, 256, 256, 0, 3),       # the correctness-sized layer (both GEMMs at K = 256)
    (8, 16, 2, 256, 256, 64, 7),      # the same with 64-row chunks: general GEMM for both
    (37, 5, 3, 384, 384, 64, 7),      # ragged segments, 64-row chunks
    (64, 8, 2, 2048, 512, 16, 3),     # small batch: gate+up from the routed ids with the
                                      # route inside, down GEMM from the same ids forming and
                                      # requantising the activations of its rows itself
    (64, 8, 2, 2048, 512, 128, 7),    # LDS-tiled GEMM for both projections
    (64, 8, 2, 1024, 512, 16, 3),     # small batch at hidden width 1024
    (40, 16, 3, 512, 1024, 0, 3),     # ... and 512, expert width 1024
    (24, 12, 2, 2048, 256, 0, 3),     # expert width 256 (the down GEMM at K = 256)
])
def test_mlp_forward_matches_oracle(M, E, k, H, I, chunk, kernels):
    assert moe.mlp_forward_kernels(M, E, k, H, I, chunk) == kernels
    d = synth.mlp_inputs(M, E, k, H, I, seed=M + H)
    outs, ws = gpu_mlp(d, chunk=chunk, reps=2)
    _, y64 = orc.mlp_tokens(d["logits"], d["x"], d["w1_q"], d["w1_s"], d["w2_q"], d["w2_s"],
                            k, CAP)
    assert_mlp_close(outs[0], y64, f"mlp M={M} H={H} I={I} chunk={chunk}")
    np.testing.assert_array_equal(outs[1], outs[0])
    ids, _ = orc.route(d["logits"], k, CAP)
    counts, offsets = orc.layout(ids, E)
    np.testing.assert_array_equal(ws_part(ws, d, 0, np.int32, M * k).reshape(M, k), ids)
    if kernels == 7:                            # (the small-batch path builds no layout)
        np.testing.assert_array_equal(ws_part(ws, d, 2, np.int32, E), counts)
        np.testing.assert_array_equal(ws_part(ws, d, 3, np.int32, E + 1), offsets)


def random_mlp_shapes(n=10, seed=2028):
    """Seeded MLP layer shapes (M, E, k, H, I, chunk): 8 to a few hundred tokens, one to 40
    experts, k up to min(E, 8), hidden width 2048 (the small-batch path's depth) or one to
    eight 128-column tiles, expert width one to eight tiles, chunk 0 (the default) or 16 / 64
    / 128 rows; every third shape in the small-batch regime; at least 2048 output elements, so that the share of elements the per-element
    bar lets through is a share of many; shapes whose oracle would take more than about a
    second are drawn again."""
    g = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        if len(shapes) % 3 == 2:
            # the small-batch regime: hidden 2048, expert width 512 or 1024, at most 16
            # routes per expert on average
            E = int(g.integers(8, 65))
            k = int(g.integers(1, 9))
            M = int(g.integers(1, 16 * E // k + 1))
            H, I, chunk = 2048, 512 * int(g.integers(1, 3)), int(g.choice([0, 16]))
        else:
            M = int(np.exp(g.uniform(np.log(8), np.log(400))))
            E = int(g.integers(1, 41))
            k = int(g.integers(1, min(E, 8) + 1))
            H = 2048 if g.random() < 0.4 else 128 * int(g.integers(1, 9))
            I = 128 * int(g.integers(1, 9))
            chunk = int(g.choice([0, 16, 64, 128]))
        if M * H < 2048 or M * k * 3 * I * H > 6e8:
            continue
        shapes.append((M, E, k, H, I, chunk))
    return shapes


@pytest.mark.parametrize("M,E,k,H,I,chunk", random_mlp_shapes())
def test_mlp_forward_random_shapes(M, E, k, H, I, chunk):
    # whole layer against the oracle on seeded shapes no hand-picked case names (one expert,
    # k = E, ragged widths, every chunk size), in whichever launch form the shape takes; the
    # kernels are deterministic, so a repeated call gives the same bits
    d = synth.mlp_inputs(M, E, k, H, I, seed=M * 131 + E * 17 + k + H + I)
    n = moe.mlp_forward_kernels(M, E, k, H, I, chunk)
    print(f"mlp M={M} E={E} k={k} H={H} I={I} chunk={chunk}: {n} kernels", flush=True)
    outs, _ = gpu_mlp(d, chunk=chunk, reps=2)
    np.testing.assert_array_equal(outs[1], outs[0])
    _, y64 = orc.mlp_tokens(d["logits"], d["x"], d["w1_q"], d["w1_s"], d["w2_q"], d["w2_s"],
                            k, CAP)
    assert_mlp_close(outs[0], y64, f"mlp M={M} E={E} k={k} H={H} I={I} chunk={chunk}")


def e4m3_rank(codes):
    """Position of an E4M3FN code on the number line (codes of one sign are monotone in their
    low 7 bits; -0 and +0 share rank 0), so one rounding step apart is a rank difference 1."""
    c = codes.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def test_mlp_forward_full_size():
    # the FP8 tutorial's layer as a full expert MLP: M=128, 256 experts, top-8, hidden 2048,
    # expert width 512 (gate+up 1024 columns).  Every token against the oracle, then the
    # reason for the relaxed per-element bar made visible:
    #  1. the device's activation codes differ from the oracle's only by single E4M3 rounding
    #     steps, on a small fraction of codes (the gate+up rows carry the matrix core's error);
    #  2. fed the device's own activation codes and scales, the oracle's down projection and
    #     combine reproduce the device output to the strict BF16 bar (5e-3 relative Frobenius
    #     and 2e-2 rms for every element), so nothing but those flips separates the two.
    d = synth.mlp_inputs(**{kk: v for kk, v in
                            synth.MLP_WORKLOADS["mlp_fp8_M128_E256_k8_H2048_I512"].items()})
    M, E, k, H, I = d["M"], d["E"], d["k"], d["H"], d["I"]
    assert moe.mlp_forward_kernels(M, E, k, H, I) == 3
    outs, ws = gpu_mlp(d, reps=2)
    np.testing.assert_array_equal(outs[1], outs[0])
    toks = np.arange(M, dtype=np.int32)
    _, y64 = oracle_rows_parallel(orc.mlp_tokens, toks, d["logits"], d["x"], d["w1_q"],
                                  d["w1_s"], d["w2_q"], d["w2_s"], k, CAP)
    assert_mlp_close(outs[0], y64, "mlp full size")

    R = M * k
    ids, wts = orc.route(d["logits"], k, CAP)
    counts, offsets = orc.layout(ids, E)
    q, sc = orc.quant_act(d["x"])
    r_ids, xq_s, xs_s = orc.sort_gather(ids, offsets, q, sc)
    h = oracle_gemm_rows_by_expert(xq_s, xs_s, d["w1_q"], d["w1_s"], offsets)  # sorted order
    act = orc.swiglu_f32(h)
    r_codes, r_scales = orc.quant_rows_f32(act)                 # [R][I], [R][I/128]
    # the device's activations are in route order (small-batch path)
    g_codes = ws_part(ws, d, 13, np.uint8, R * I).reshape(R, I)[r_ids]
    g_scales = ws_part(ws, d, 14, np.float32, (I // 128) * R).reshape(I // 128, R)[:, r_ids]
    np.testing.assert_allclose(g_scales.T, r_scales, rtol=2.0 ** -10, atol=0)
    # Codes differ only by rounding: the dequantised activations differ by at most one E4M3
    # step of the oracle's value plus the gate+up rows' own error, which the matrix core
    # bounds relative to sum |x_i w_i| rather than to the value: near zero that spans several
    # of the small steps, but stays far below the block's amax (2^-9 of it).
    table = orc.e4m3_decode_table()
    mag = r_codes & 0x7F
    spacing = np.where(mag < 0x7E, np.abs(table[np.minimum(mag + 1, 0x7E)] - table[mag]),
                       table[0x7E] - table[0x7D])
    sg = np.repeat(g_scales.T, 128, axis=1)
    sr = np.repeat(r_scales, 128, axis=1)
    excess = np.abs(table[g_codes] * sg - table[r_codes] * sr) - spacing * sr
    amax = 448.0 * sr
    worst = float(np.max(excess / np.where(amax > 0, amax, 1.0)))
    step = np.abs(e4m3_rank(g_codes) - e4m3_rank(r_codes))
    flips = float((step > 0).mean())
    print(f"activation codes: {flips:.5f} differ, {float((step > 1).mean()):.6f} by more than "
          f"one step; worst excess over one step 2^{np.log2(max(worst, 2.0 ** -60)):.1f} of "
          f"the block amax")
    assert worst <= 2.0 ** -9, "an activation code beyond rounding of the oracle's value"
    assert flips <= 1e-2, f"{flips:.4f} of the activation codes differ"
    C2 = oracle_gemm_rows_by_expert(g_codes, g_scales, d["w2_q"], d["w2_s"], offsets)
    _, y_dev_act = orc.scatter(C2, r_ids, wts, M)
    assert_bf16_close(outs[0], y_dev_act, "mlp with the device's activation codes")
