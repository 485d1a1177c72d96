"""Pins of the oracle's blockwise FP8 quantiser, block-scaled grouped GEMM, scatter,
whole forward, BF16 grouped GEMM and the SiLU-gated expert FFN.

GEMM pins reduce the method to exact integer matmuls (numpy int64), to dense float64
matmuls of the dequantised operands (E=1, k=1), and to sums over every expert (k=E).
"""
import numpy as np
import scipy.special
import pytest
import torch

from mixture_experts_layer_softcap_amd import synth


def _f32_bits(v):
    return int(np.float32(v).view(np.uint32))


# ---- quantiser ------------------------------------------------------------------------

def test_quant_block_with_amax_448_is_the_plain_encoding(orc):
    g = np.random.default_rng(0)
    row = (g.standard_normal(256) * 100).astype(np.float32)
    row[3] = 448.0
    row[200] = -448.0
    x = synth.bf16_bits(row)[None, :]
    q, s = orc.quant_act(x)
    assert s.tolist() == [[1.0, 1.0]]
    vals = synth.bf16_to_f32(x[0])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q[0], ref)


def test_quant_block_amax_one(orc):
    # scale = fp32(1/448) = 0x3B124925, its fp32 reciprocal is 447.99997 (0x43DFFFFF), and
    # 1.0 * 447.99997 encodes to 448 (0x7E)
    row = np.zeros(128, np.float32)
    row[0] = 1.0
    row[1] = -0.5
    q, s = orc.quant_act(synth.bf16_bits(row)[None, :])
    assert _f32_bits(s[0, 0]) == 0x3B124925
    assert _f32_bits(np.float32(1.0) / s[0, 0]) == 0x43DFFFFF
    assert q[0, 0] == 0x7E and q[0, 1] == 0xF6 and q[0, 2] == 0x00


def test_quant_all_zero_block_keeps_signs(orc):
    row = np.zeros(128, np.float32)
    row[5] = -0.0
    q, s = orc.quant_act(synth.bf16_bits(row)[None, :])
    assert s[0, 0] == 0.0
    assert q[0, 5] == 0x80 and (np.delete(q[0], 5) == 0).all()


def test_quant_every_nonzero_block_holds_the_top_code(orc):
    d = synth.workload_inputs("fused_fp8_M128_E256_k8_K2048_N512", weights=False)
    q, s = orc.quant_act(d["x"])
    blocks = (q & 0x7F).reshape(128, 16, 128)
    assert (blocks.max(axis=2) == 0x7E).all()
    assert (s > 0).all()


def test_quant_error_bound(orc):
    d = synth.workload_inputs("fused_fp8_M8_E16_k2_K256_N256", weights=False)
    q, s = orc.quant_act(d["x"])
    x = synth.bf16_to_f32(d["x"]).astype(np.float64)
    dq = orc.e4m3_decode_table()[q] * np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(x - dq)
    scale = np.repeat(s.astype(np.float64), 128, axis=1)
    normal = np.abs(x) >= scale * 2.0 ** -6
    # half an ulp of a 3-bit mantissa (2^-4 relative), half the subnormal spacing 2^-10
    # (times the scale), plus the rounding of the fp32 reciprocal
    assert (err[normal] <= np.abs(x[normal]) * (2.0 ** -4 + 2.0 ** -20)).all()
    assert (err[~normal] <= scale[~normal] * 2.0 ** -10 + np.abs(x[~normal]) * 2.0 ** -20).all()


@pytest.mark.parametrize("p", [-7, -1, 1, 5])
def test_quant_power_of_two_scaling_invariance(orc, p):
    d = synth.workload_inputs("fused_fp8_M8_E16_k2_K256_N256", weights=False)
    x = synth.bf16_to_f32(d["x"])
    q0, s0 = orc.quant_act(d["x"])
    q1, s1 = orc.quant_act(synth.bf16_bits(x * np.float32(2.0 ** p)))
    np.testing.assert_array_equal(q0, q1)
    np.testing.assert_array_equal(s1, s0 * np.float32(2.0 ** p))


def test_quant_weights_blocks_are_128_by_128(orc):
    g = np.random.default_rng(4)
    w = (g.standard_normal((2, 256, 384)) * 0.02).astype(np.float32)
    w[1, 130, 300] = 7.0           # lives in block (e=1, nb=1, kb=2) only
    q, s = orc.quant_weights(w)
    assert s.shape == (2, 2, 3)
    np.testing.assert_allclose(s[1, 1, 2], np.float32(7.0) / np.float32(448.0), rtol=0)
    assert q[1, 130, 300] == 0x7E
    amax = np.abs(w).reshape(2, 2, 128, 3, 128).max(axis=(2, 4))
    np.testing.assert_array_equal(s, (amax / np.float32(448.0)).astype(np.float32))
    # codes of a block equal the activation quantiser's codes when every row of the block is
    # forced to share the block amax (each row then has the block's scale); the values are
    # made bf16-exact first so that both quantisers see the same numbers
    blk = synth.bf16_to_f32(synth.bf16_bits(w[0, :128, :128]))
    blk[:, 0] = np.abs(blk).max()
    qb, sb = orc.quant_weights(np.ascontiguousarray(blk)[None])
    qa, sa = orc.quant_act(synth.bf16_bits(blk))
    assert sa.shape == (128, 1) and (sa[:, 0] == sb[0, 0, 0]).all()
    np.testing.assert_array_equal(qb[0], qa)
    assert (qb[0] & 0x7F).max() == 0x7E


# ---- grouped GEMM ---------------------------------------------------------------------

_INT_CODES = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48,
              -1: 0xB8, -2: 0xC0, -3: 0xC4, -4: 0xC8}


def _int_codes(a):
    out = np.zeros(a.shape, np.uint8)
    for v, c in _INT_CODES.items():
        out[a == v] = c
    return out


def test_gemm_fp8_is_an_exact_integer_matmul_with_power_of_two_scales(orc):
    g = np.random.default_rng(9)
    E, N, K, rows = 3, 256, 384, 11
    counts = np.array([4, 0, 7], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    Ai = g.integers(-4, 5, (rows, K))
    Wi = g.integers(-4, 5, (E, N, K))
    sa = np.exp2(g.integers(-3, 4, (K // 128, rows))).astype(np.float32)
    sb = np.exp2(g.integers(-3, 4, (E, N // 128, K // 128))).astype(np.float32)
    C = orc.gemm_fp8(_int_codes(Ai), sa, _int_codes(Wi), sb, offsets)
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1]):
            ref = np.zeros(N)
            for b in range(K // 128):
                part = Wi[e, :, b * 128:(b + 1) * 128] @ Ai[r, b * 128:(b + 1) * 128]
                ref += part * sa[b, r] * np.repeat(sb[e, :, b], 128)
            np.testing.assert_array_equal(C[r], ref)


def _dequant_w(orc, wq, ws):
    E, N, K = wq.shape
    t = orc.e4m3_decode_table()
    return t[wq] * np.repeat(np.repeat(ws.astype(np.float64), 128, 1), 128, 2)


def test_forward_single_expert_is_a_dense_blockwise_gemm(orc):
    g = np.random.default_rng(21)
    M, K, N = 5, 256, 384
    logits = g.standard_normal((M, 1)).astype(np.float32)
    x = synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    wq, ws = orc.quant_weights((g.standard_normal((1, N, K)) * 0.02).astype(np.float32))
    out = orc.forward(logits, x, wq, ws, 1, 30.0)
    q, s = orc.quant_act(x)
    A = orc.e4m3_decode_table()[q] * np.repeat(s.astype(np.float64), 128, 1)
    ref = A @ _dequant_w(orc, wq, ws)[0].T
    np.testing.assert_allclose(out["y64"], ref, rtol=1e-12, atol=1e-15)
    ref_bf16 = np.vectorize(orc.bf16_from_double)(ref).astype(np.uint16)
    np.testing.assert_array_equal(out["y"], ref_bf16)


def test_forward_with_all_experts_sums_every_expert(orc):
    g = np.random.default_rng(22)
    M, E, K, N = 6, 4, 128, 256
    logits = g.standard_normal((M, E)).astype(np.float32)
    x = synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    wq, ws = orc.quant_weights((g.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    out = orc.forward(logits, x, wq, ws, E, 30.0, intermediates=True)
    q, s = orc.quant_act(x)
    A = orc.e4m3_decode_table()[q] * np.repeat(s.astype(np.float64), 128, 1)
    Wd = _dequant_w(orc, wq, ws)
    ref = np.zeros((M, N))
    for t in range(M):
        for j in range(E):
            e = out["ids"][t, j]
            ref[t] += float(out["weights"][t, j]) * (Wd[e] @ A[t])
    np.testing.assert_allclose(out["y64"], ref, rtol=1e-12, atol=1e-15)


def test_forward_tokens_matches_forward(orc):
    d = synth.workload_inputs("fused_fp8_M8_E16_k2_K256_N256")
    wq, ws = orc.quant_weights(d["w"])
    full = orc.forward(d["logits"], d["x"], wq, ws, d["k"], d["cap"])
    toks = np.array([7, 0, 3], np.int32)
    y, y64 = orc.forward_tokens(d["logits"], d["x"], wq, ws, d["k"], d["cap"], toks)
    np.testing.assert_array_equal(y, full["y"][toks])
    np.testing.assert_allclose(y64, full["y64"][toks], rtol=1e-13, atol=1e-16)


def test_scatter_weights_each_route(orc):
    M, k, N = 3, 2, 4
    C = np.arange(M * k * N, dtype=np.float64).reshape(M * k, N)
    sorted_ids = np.array([5, 0, 3, 1, 2, 4], np.int32)
    w = np.array([[0.5, 0.25], [1.0, -1.0], [2.0, 0.0]], np.float32)
    _, y64 = orc.scatter(C, sorted_ids, w, M)
    ref = np.zeros((M, N))
    for s, r in enumerate(sorted_ids):
        ref[r // k] += w.ravel()[r] * C[s]
    np.testing.assert_array_equal(y64, ref)
    assert y64[0, 0] == 0.5 * C[1, 0] + 0.25 * C[3, 0]


# ---- BF16 grouped GEMM and the gated FFN ------------------------------------------------

def test_gemm_bf16_segments_use_their_expert(orc):
    d = synth.grouped_gemm_inputs(rows=40, E=3, N=48, K=64, dist="skewed", seed=3)
    out, out64 = orc.gemm_bf16(d["A"], d["W"], d["offsets"])
    A = synth.bf16_to_f32(d["A"]).astype(np.float64)
    W = synth.bf16_to_f32(d["W"]).astype(np.float64)
    for e in range(3):
        a, b = d["offsets"][e], d["offsets"][e + 1]
        np.testing.assert_allclose(out64[a:b], A[a:b] @ W[e].T, rtol=1e-12, atol=1e-12)
    ref = torch.from_numpy(out64.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    # bf16(float32(v)) can differ from bf16(v) only by double rounding: at most one code
    diff = np.abs(out.astype(np.int32) - ref.numpy().view(np.uint16).astype(np.int32))
    assert diff.max() <= 1
    sub, _ = orc.gemm_bf16(d["A"], d["W"], d["offsets"], rows_list=np.array([39, 0, 17]))
    np.testing.assert_array_equal(sub, out[[39, 0, 17]])


def test_ffn_single_expert_matches_torch_composition(orc):
    T, E, H, F = 4, 1, 64, 32
    d = synth.ffn_inputs(T, E, H, F, seed=5, skewed=False)
    y, y64 = orc.ffn_tokens(d["logits"], d["x"], d["w_up"], d["w_down"], 1, 30.0)
    x = torch.from_numpy(synth.bf16_to_f32(d["x"]).astype(np.float64))
    wu = torch.from_numpy(synth.bf16_to_f32(d["w_up"][0]).astype(np.float64))
    wd = torch.from_numpy(synth.bf16_to_f32(d["w_down"][0]).astype(np.float64))
    h = x @ wu.T
    act = torch.nn.functional.silu(h[:, :F]) * h[:, F:]
    act_b = act.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    ref = act_b @ wd.T
    # the oracle rounds act to bf16 directly from double; torch goes via fp32, which can
    # move a rare tie by one bf16 ulp, so compare with a bound of one ulp per term
    np.testing.assert_allclose(y64, ref.numpy(), rtol=2e-2, atol=1e-3)
    np.testing.assert_allclose(y64, ref.numpy(), rtol=0, atol=np.abs(ref.numpy()).max() * 1e-2)


def test_ffn_activation_is_rounded_to_bf16_before_the_down_projection(orc):
    # One token, one expert (k = 1, weight exactly 1), x = e_0, so g_f and u_f are single
    # bf16 weights; the down projection is the identity on the first F outputs.  Then
    # y64[f] is the activation the layer feeds the down GEMM: it must be a bf16 value (the
    # intermediate rounding of the Mixtral-like layer) within half a bf16 ulp of
    # silu(g)*u, which scipy's logistic gives independently.  None of the chosen products is
    # a bf16 value, so an oracle that dropped the rounding would fail the bf16-value checks.
    H, F = 8, 4
    g = np.array([0.5, 1.25, -2.0, 3.0], np.float32)
    u = np.array([1.0, 0.75, 1.5, -0.625], np.float32)
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    w_up = np.zeros((1, 2 * F, H), np.float32)
    w_up[0, :F, 0] = g
    w_up[0, F:, 0] = u
    w_down = np.zeros((1, H, F), np.float32)
    w_down[0, np.arange(F), np.arange(F)] = 1.0
    logits = np.zeros((1, 1), np.float32)
    y, y64 = orc.ffn_tokens(logits, synth.bf16_bits(x), synth.bf16_bits(w_up),
                            synth.bf16_bits(w_down), 1, 30.0)
    exact = g.astype(np.float64) * scipy.special.expit(g.astype(np.float64)) * u
    act = y64[0, :F]
    assert (y64[0, F:] == 0).all()
    # a bf16 value: exact in fp32 with the low 16 bits of its fp32 image clear
    assert (act.astype(np.float32).astype(np.float64) == act).all()
    assert (act.astype(np.float32).view(np.uint32) & 0xFFFF == 0).all()
    assert (np.abs(act - exact) <= 2.0 ** -8 * np.abs(exact)).all()   # half an ulp (p = 8)
    # the unrounded products are not bf16 values, so the rounding is what the checks see
    assert (exact.astype(np.float32).view(np.uint32) & 0xFFFF != 0).all()
    assert (np.abs(act - exact) > 2.0 ** -20 * np.abs(exact)).all()


def test_ffn_k2_weights_combine_two_experts(orc):
    T, E, H, F = 3, 4, 32, 16
    d = synth.ffn_inputs(T, E, H, F, seed=6)
    y, y64 = orc.ffn_tokens(d["logits"], d["x"], d["w_up"], d["w_down"], 2, 30.0)
    ids, w = orc.route(d["logits"], 2, 30.0)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(2):
            one_hot = np.full((1, E), -100.0, np.float32)
            one_hot[0, ids[t, j]] = 0.0
            _, yj = orc.ffn_tokens(one_hot, d["x"][t:t + 1], d["w_up"], d["w_down"], 1, 30.0)
            acc += float(w[t, j]) * yj[0]
        np.testing.assert_allclose(y64[t], acc, rtol=1e-12, atol=1e-14)
