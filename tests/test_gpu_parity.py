"""GPU parity of every stage and of the whole forward against the CPU oracle.

Integer results (ids, counts, offsets, task sets, segment contents, E4M3 codes, scales) are
compared bit for bit; routing weights to 1e-5 relative; BF16 outputs with the relative
Frobenius <= 5e-3 and per-element <= 2e-2*rms rule.  Rows inside one expert segment come in
atomic arrival order from the one-workgroup layout and the QSG stage, so there segments are
sorted by route id before comparing; the layout over many workgroups keeps route-id order.
"""
import concurrent.futures as cf
import functools

import numpy as np
import pytest
import torch

import oracle as orc
from mixture_experts_layer_softcap_amd import moe, synth

from gpu_util import (DEV, WEIGHT_RTOL, assert_bf16_close, assert_gemm_f32_close, bf16_f64,
                      bf16_ulp,
                      canonical_segments, oracle_gemm_rows_by_expert, oracle_rows_parallel,
                      oracle_threads, to_dev, to_np, workload, zeros)

pytestmark = pytest.mark.gpu

CAP = 30.0
TINY = "fused_fp8_M8_E16_k2_K256_N256"
QWEN = "fused_fp8_M128_E256_k8_K2048_N512"
ZIPF1K = "fused_fp8_M1024_E256_k8_K2048_N512_zipf"
ZIPF4K = "fused_fp8_M4096_E256_k8_K2048_N512_zipf"
TINY_K2048 = "M24_E40_k3_K2048_N256"


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    orc.build(force=False)
    assert moe.device_check() == moe.MOE_OK, "current device is not gfx950"


def sync():
    torch.cuda.synchronize()


# ---- stage 1: route --------------------------------------------------------------------

def gpu_route(logits, k, cap=CAP):
    M, E = logits.shape
    ids, w = zeros((M, k), torch.int32), zeros((M, k), torch.float32)
    moe.route(to_dev(logits), k, cap, ids, w)
    sync()
    return to_np(ids), to_np(w)


def check_route(logits, k, cap=CAP):
    ids, w = gpu_route(logits, k, cap)
    rids, rw = orc.route(logits, k, cap)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=WEIGHT_RTOL, atol=0)


@pytest.mark.parametrize("name", [TINY, QWEN, ZIPF1K, ZIPF4K])
def test_route_workloads(name):
    d = synth.workload_inputs(name, weights=False)
    check_route(d["logits"], d["k"])


@pytest.mark.parametrize("M,E,k", [(1, 16, 1), (5, 16, 16), (33, 64, 8), (7, 1024, 8),
                                   (9, 100, 3), (3, 1000, 64), (130, 256, 8)])
def test_route_shapes(M, E, k):
    g = np.random.default_rng(M * 7 + E + k)
    logits = g.standard_normal((M, E)).astype(np.float32)
    logits[:, ::3] = np.round(logits[:, ::3], 1)        # exact ties
    check_route(logits, k)
    check_route(logits, k, cap=0.0)


def test_route_ties_and_signed_zero():
    logits = np.zeros((4, 64), np.float32)
    logits[1, [5, 9, 40]] = 1.0
    logits[2, 7] = -0.0
    logits[3] = -1.0
    logits[3, [63, 0]] = -0.0
    check_route(logits, 3)
    ids, w = gpu_route(np.full((2, 16), 0.5, np.float32), 8)
    assert (ids == np.arange(8)).all() and (w == np.float32(0.125)).all()


def test_route_nan_and_infinite_logits():
    # NaN ranks below every number (-inf included), NaNs tie by the lower index; +-inf rank as
    # numbers.  The ids are compared bit for bit; weights only where they are finite.
    g = np.random.default_rng(12)
    logits = g.standard_normal((6, 256)).astype(np.float32)
    logits[0, [2, 9, 200]] = np.nan
    logits[1, :] = np.nan
    logits[2, 3] = -np.inf
    logits[2, [0, 5, 6, 100]] = np.nan
    logits[3, ::2] = np.nan
    logits[4, 1:] = np.nan
    logits[5, 7] = np.inf
    logits[5, 8] = np.nan
    for k in (1, 8):
        ids, w = gpu_route(logits, k)
        rids, rw = orc.route(logits, k, CAP)
        np.testing.assert_array_equal(ids, rids)
        fin = np.isfinite(rw).all(1)
        np.testing.assert_allclose(w[fin], rw[fin], rtol=WEIGHT_RTOL, atol=0)


@pytest.mark.parametrize("name", [TINY, QWEN, ZIPF1K])
def test_route_quantize_matches_oracle(name):
    # the route and, per token, the activation quantiser of the sort/gather stage: codes and
    # scales bit-exact, token-major ([M][K] codes, [K/128][M] scales)
    d = synth.workload_inputs(name, weights=False)
    M, E, k, K = d["M"], d["E"], d["k"], d["K"]
    ids, w = zeros((M, k), torch.int32), zeros((M, k), torch.float32)
    x_q = torch.full((M, K), 0x55, dtype=torch.uint8, device=DEV)
    x_s = torch.full((K // 128, M), -1.0, dtype=torch.float32, device=DEV)
    moe.route_quantize(to_dev(d["logits"]), to_dev(d["x"]), k, CAP, ids, w, x_q, x_s)
    sync()
    rids, rw = orc.route(d["logits"], k, CAP)
    np.testing.assert_array_equal(to_np(ids), rids)
    np.testing.assert_allclose(to_np(w), rw, rtol=WEIGHT_RTOL, atol=0)
    q, sc = orc.quant_act(d["x"])
    np.testing.assert_array_equal(to_np(x_q), q)
    np.testing.assert_array_equal(to_np(x_s).view(np.uint32), sc.T.copy().view(np.uint32))


def test_route_quantize_edge_rows():
    # K = 128 (one block: only the first 16 lanes of a pass hold data), a zero row, signed
    # zeros and values that saturate; E = 16 with one token
    g = np.random.default_rng(11)
    for M, E, k, K in ((1, 16, 1, 128), (5, 64, 4, 640), (9, 300, 3, 1152)):
        logits = g.standard_normal((M, E)).astype(np.float32)
        xf = g.standard_normal((M, K)).astype(np.float32) * 3.0
        xf[0, :128] = 0.0
        xf[0, 1] = -0.0
        if M > 1:
            xf[1, 5] = 448.0 * 4
        x = synth.bf16_bits(xf)
        ids, w = zeros((M, k), torch.int32), zeros((M, k), torch.float32)
        x_q = zeros((M, K), torch.uint8)
        x_s = zeros((K // 128, M), torch.float32)
        moe.route_quantize(to_dev(logits), to_dev(x), k, CAP, ids, w, x_q, x_s)
        sync()
        q, sc = orc.quant_act(x)
        np.testing.assert_array_equal(to_np(x_q), q)
        np.testing.assert_array_equal(to_np(x_s).view(np.uint32), sc.T.copy().view(np.uint32))
        np.testing.assert_array_equal(to_np(ids), orc.route(logits, k, CAP)[0])


# ---- stage 2: layout -------------------------------------------------------------------

def gpu_layout(ids, E, n_blocks, chunk):
    M, k = ids.shape
    mt = moe.max_tasks(M, k, E, n_blocks, chunk)
    counts, offsets, cursors = zeros(E, torch.int32), zeros(E + 1, torch.int32), zeros(E, torch.int32)
    tasks = torch.full((max(mt, 1), 4), -7, dtype=torch.int32, device=DEV)
    ntasks = zeros(1, torch.int32)
    queue = torch.full((moe.MOE_QUEUE_WORDS,), 5, dtype=torch.int32, device=DEV)
    moe.build_layout(to_dev(ids), E, n_blocks, chunk, counts, offsets, cursors, tasks, ntasks,
                     queue)
    sync()
    n = int(to_np(ntasks)[0])
    return dict(counts=to_np(counts), offsets=to_np(offsets), cursors=to_np(cursors),
                tasks=to_np(tasks)[:n], queue=to_np(queue), max_tasks=mt)


def check_layout(ids, E, n_blocks, chunk):
    g = gpu_layout(ids, E, n_blocks, chunk)
    counts, offsets = orc.layout(ids, E)
    np.testing.assert_array_equal(g["counts"], counts)
    np.testing.assert_array_equal(g["offsets"], offsets)
    np.testing.assert_array_equal(g["cursors"], offsets[:-1])
    assert (g["queue"] == 0).all()
    ref = orc.tasks(counts, offsets, n_blocks, chunk)
    key = lambda t: sorted(map(tuple, t.tolist()))
    assert key(g["tasks"]) == key(ref)
    assert len(g["tasks"]) <= g["max_tasks"]
    # order: every n_block of one chunk adjacent; full chunks first, then partial chunks by
    # non-increasing row count
    t = g["tasks"]
    if len(t):
        chunks = t.reshape(-1, n_blocks, 4)
        assert (chunks[:, :, 3] == np.arange(n_blocks)).all()
        assert (chunks[:, :, :3] == chunks[:, :1, :3]).all()
        rc = chunks[:, 0, 2]
        assert (np.diff(rc) <= 0).all()
    return g


@pytest.mark.parametrize("name,chunk", [(TINY, 16), (QWEN, 16), (ZIPF1K, 32), (ZIPF4K, 64),
                                        (ZIPF4K, 1), (QWEN, 1024)])
def test_layout_workloads(name, chunk):
    d = synth.workload_inputs(name, weights=False)
    ids, _ = orc.route(d["logits"], d["k"], CAP)
    check_layout(ids, d["E"], d["N"] // 128, chunk)


@pytest.mark.parametrize("name,chunk", [(TINY, 128), (QWEN, 128), (ZIPF1K, 128), (ZIPF4K, 256)])
def test_layout_sorted_routes(name, chunk):
    # the layout's own sort: every segment holds exactly its expert's routes (order free),
    # route_slots is the inverse permutation; counts/offsets/tasks as without the sort
    d = synth.workload_inputs(name, weights=False)
    ids, _ = orc.route(d["logits"], d["k"], CAP)
    E = d["E"]
    M, k = ids.shape
    nb = d["N"] // 128
    mt = moe.max_tasks(M, k, E, nb, chunk)
    counts, offsets, cursors = zeros(E, torch.int32), zeros(E + 1, torch.int32), zeros(E, torch.int32)
    tasks = zeros((mt, 4), torch.int32)
    ntasks, queue = zeros(1, torch.int32), zeros(moe.MOE_QUEUE_WORDS, torch.int32)
    srt = torch.full((M * k,), -5, dtype=torch.int32, device=DEV)
    slots = torch.full((M * k,), -5, dtype=torch.int32, device=DEV)
    moe.build_layout(to_dev(ids), E, nb, chunk, counts, offsets, cursors, tasks, ntasks, queue,
                     sorted_route_ids=srt, route_slots=slots)
    sync()
    rcounts, roffsets = orc.layout(ids, E)
    np.testing.assert_array_equal(to_np(offsets), roffsets)
    s_ids, sl = to_np(srt), to_np(slots)
    r_ids, _, _ = orc.sort_gather(ids, roffsets, np.zeros((M, 128), np.uint8),
                                  np.zeros((M, 1), np.float32))
    perm = canonical_segments(s_ids, roffsets)
    np.testing.assert_array_equal(s_ids[perm], r_ids)
    np.testing.assert_array_equal(s_ids[sl], np.arange(M * k))
    n = int(to_np(ntasks)[0])
    ref_tasks = orc.tasks(rcounts, roffsets, nb, chunk)
    assert n == len(ref_tasks)


def test_layout_edge_cases():
    # every route on one expert; empty experts; a single token; E = 1024
    check_layout(np.full((40, 1), 3, np.int32), 8, 2, 16)
    check_layout(np.array([[0]], np.int32), 1, 1, 1)
    g = np.random.default_rng(3)
    check_layout(g.integers(0, 1024, (300, 8)).astype(np.int32), 1024, 4, 7)
    check_layout(g.integers(0, 5, (64, 2)).astype(np.int32), 300, 1, 16)


# ---- stage 3: quantise + sort + gather -------------------------------------------------

def gpu_qsg(x, ids, E, K):
    M, k = ids.shape
    lay = gpu_layout(ids, E, 1, 16)
    cursors = to_dev(lay["offsets"][:-1].copy())
    R = M * k
    sorted_ids = torch.full((R,), -1, dtype=torch.int32, device=DEV)
    a_q = zeros((R, K), torch.uint8)
    a_s = zeros((K // 128, R), torch.float32)
    moe.quant_sort_gather(to_dev(x), to_dev(ids), E, cursors, sorted_ids, a_q, a_s)
    sync()
    return to_np(sorted_ids), to_np(a_q), to_np(a_s), to_np(cursors), lay


def check_qsg(x, ids, E):
    K = x.shape[1]
    s_ids, a_q, a_s, cursors, lay = gpu_qsg(x, ids, E, K)
    counts, offsets = orc.layout(ids, E)
    np.testing.assert_array_equal(cursors, offsets[1:])
    q, s = orc.quant_act(x)
    r_ids, r_aq, r_as = orc.sort_gather(ids, offsets, q, s)
    perm = canonical_segments(s_ids, offsets)
    np.testing.assert_array_equal(s_ids[perm], r_ids)
    np.testing.assert_array_equal(a_q[perm], r_aq)
    np.testing.assert_array_equal(a_s[:, perm].view(np.uint32), r_as.view(np.uint32))


@pytest.mark.parametrize("name", [TINY, QWEN, ZIPF1K])
def test_qsg_workloads(name):
    d = synth.workload_inputs(name, weights=False)
    ids, _ = orc.route(d["logits"], d["k"], CAP)
    check_qsg(d["x"], ids, d["E"])


def test_qsg_edge_values():
    # zero blocks, signed zeros, blocks whose amax is a power of two, tiny and huge values,
    # odd K (3 blocks), K larger than one 2048-wide pass
    g = np.random.default_rng(12)
    for K in (384, 4096 + 128):
        x = g.standard_normal((6, K)).astype(np.float32)
        x[0, :128] = 0.0
        x[0, 5] = -0.0
        x[1, :128] *= np.float32(2.0 ** -60)
        x[2, 128:256] = np.float32(448.0) * np.sign(x[2, 128:256])
        x[3] *= np.float32(2.0 ** 40)
        x[4, :] = np.float32(1.0)
        xb = synth.bf16_bits(x)
        ids = g.integers(0, 5, (6, 3)).astype(np.int32)
        check_qsg(xb, ids, 5)


# ---- weight preparation ------------------------------------------------------------------

def gpu_wquant(w):
    E, N, K = w.shape
    w_q = zeros((E, N, K), torch.uint8)
    w_s = zeros((E, N // 128, K // 128), torch.float32)
    moe.quantize_weights(to_dev(w), w_q, w_s)
    sync()
    return to_np(w_q), to_np(w_s)


def test_quantize_weights_full_qwen_layer():
    d = workload(QWEN)
    w_q, w_s = gpu_wquant(d["w"])
    np.testing.assert_array_equal(w_s.view(np.uint32), d["w_s"].view(np.uint32))
    np.testing.assert_array_equal(w_q, d["w_q"])


def wquant_vs_oracle(w):
    """The device's weight quantiser against the oracle's on blocks w [nblk][128][128]: codes
    and scales bit for bit (the oracle's side in threads over disjoint blocks)."""
    nblk = w.shape[0]
    w_q, w_s = gpu_wquant(w)
    parts = [p for p in np.array_split(np.arange(nblk), oracle_threads()) if p.size]
    with cf.ThreadPoolExecutor(max_workers=len(parts)) as ex:
        refs = list(ex.map(lambda p: orc.quant_weights(w[p[0]:p[-1] + 1]), parts))
    np.testing.assert_array_equal(w_q, np.concatenate([r[0] for r in refs]))
    np.testing.assert_array_equal(w_s.view(np.uint32),
                                  np.concatenate([r[1] for r in refs]).view(np.uint32))
    return w_q, w_s


def test_e4m3_encoder_exhaustive():
    # Every fp32 bit pattern with |y| <= 448 (0x43E00000), both signs: 2.27e9 encoder inputs.
    # Blocks whose amax is exactly 448 have scale 1 and multiplier 1, so their codes are the
    # plain encoding of the values; each 128x128 weight block holds 448 and 16383 swept
    # values, and the device's quantiser is compared bit for bit with the oracle's.
    limit = 0x43E00000
    per_block = 128 * 128 - 1
    chunk = per_block * 8192                     # 134M values per pass
    total = 0
    for sign in (0, 0x80000000):
        for start in range(0, limit + 1, chunk):
            bits = np.arange(start, min(start + chunk, limit + 1), dtype=np.uint32) | sign
            n = bits.size
            nblk = -(-n // per_block)
            vals = np.zeros(nblk * per_block, np.float32)
            vals[:n] = bits.view(np.float32)
            buf = np.empty((nblk, 128 * 128), np.float32)
            buf[:, 0] = 448.0
            buf[:, 1:] = vals.reshape(nblk, per_block)
            w_q, w_s = wquant_vs_oracle(buf.reshape(nblk, 128, 128))
            assert (w_s == 1.0).all()
            total += n
    assert total == 2 * (limit + 1)


def test_e4m3_saturation_above_448():
    # Encoder inputs above 448 arise only at a block's amax A, where A * fl(1/fl(A/448)) can
    # round past 448 (then the code saturates to 0x7E, never NaN), and for values within an
    # ulp of it.  Blocks with amax every 64th fp32 value in (448, 465] (and 465 itself, up to
    # where fp32 -> E4M3 rounding would leave the finite range), holding the 16383 fp32
    # values just below A and their negatives.
    A = np.arange(0x43E00001, 0x43E88001, 64, dtype=np.uint32)
    A = np.unique(np.append(A, np.uint32(0x43E88000))).view(np.float32)
    near = np.arange(1, 128 * 128, dtype=np.uint32)
    bits = A.view(np.uint32)[:, None] - (near[None, :] >> 1)
    vals = bits.view(np.float32) * np.where(near[None, :] & 1, -1.0, 1.0).astype(np.float32)
    w = np.concatenate([A[:, None], vals], axis=1).reshape(-1, 128, 128)
    w_q, w_s = wquant_vs_oracle(w)
    assert (w_q.reshape(A.size, -1)[:, 0] == 0x7E).all()
    assert ((w_q & 0x7F) != 0x7F).all()


# ---- stage 4: grouped GEMM ---------------------------------------------------------------

INT_CODES = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, -1: 0xB8, -2: 0xC0, -3: 0xC4,
             -4: 0xC8}


def int_codes(a):
    out = np.zeros(a.shape, np.uint8)
    for v, c in INT_CODES.items():
        out[a == v] = c
    return out


def gpu_gemm(a_q, a_s, w_q, w_s, offsets, chunk, epilogue, sorted_ids=None, queue=True,
             out_rows=None, repeat=1):
    rows, K = a_q.shape
    E, N, _ = w_q.shape
    counts = np.diff(offsets).astype(np.int32)
    tasks = orc.tasks(counts, offsets, N // 128, chunk)
    tasks_d = to_dev(tasks if len(tasks) else np.zeros((1, 4), np.int32))
    ntasks = to_dev(np.array([len(tasks)], np.int32))
    q = zeros(moe.MOE_QUEUE_WORDS, torch.int32) if queue else None
    n_out = rows if out_rows is None else out_rows
    dt = torch.int16 if epilogue == moe.MOE_EPI_STORE_BF16 else torch.float32
    out = torch.full((n_out, N), -3, dtype=dt, device=DEV)
    args = (to_dev(a_q), to_dev(a_s), to_dev(w_q), to_dev(w_s))
    sid = None if sorted_ids is None else to_dev(sorted_ids)
    for _ in range(repeat):
        moe.grouped_gemm(moe.MOE_GEMM_FP8_B128, *args, tasks_d, ntasks, chunk, out, epilogue,
                         queue=q, sorted_route_ids=sid)
    sync()
    if q is not None:
        assert (to_np(q) == 0).all(), "queue not reset by the last workgroup"
    return to_np(out)


@pytest.mark.parametrize("chunk,queue,K", [(16, True, 512), (16, False, 512), (32, True, 512),
                                           (64, True, 512), (5, True, 512), (16, True, 2048),
                                           (16, False, 2048), (7, False, 4096),
                                           (3, True, 4096), (64, False, 2048),
                                           (128, True, 512), (256, False, 2048),
                                           (200, True, 4096), (256, True, 128),
                                           (16, True, 1024), (16, True, 640),
                                           (9, False, 768)])
def test_gemm_integer_exact(chunk, queue, K):
    # K in {512, 1024, 2048} with chunk <= 16 takes the streaming range kernel, chunks of
    # 65..256 rows the LDS-tiled kernel, the rest (K = 640, 768, 4096 at small chunks, and
    # chunks of 17..64 rows) the general one
    g = np.random.default_rng(chunk + K)
    E, N = 4, 256
    counts = np.array([3, 0, 37, 70], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    Ai = g.integers(-4, 5, (rows, K))
    Wi = g.integers(-4, 5, (E, N, K))
    # power-of-two scales in [1/2, 2]: every partial sum stays an integer multiple of 2^-2
    # below 2^15, so fp32 accumulation is exact in any order
    sa = np.exp2(g.integers(-1, 2, (K // 128, rows))).astype(np.float32)
    sb = np.exp2(g.integers(-1, 2, (E, N // 128, K // 128))).astype(np.float32)
    ref = orc.gemm_fp8(int_codes(Ai), sa, int_codes(Wi), sb, offsets)
    got = gpu_gemm(int_codes(Ai), sa, int_codes(Wi), sb, offsets, chunk,
                   moe.MOE_EPI_STORE_F32, queue=queue, repeat=2)
    np.testing.assert_array_equal(got, ref.astype(np.float32))


def finite_e4m3_codes(g, shape):
    c = g.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)   # no NaN codes


def test_fp8_block_sum_error_of_the_matrix_core():
    # One 128-wide scale block per output (E=1, K=128, unit scales), random finite E4M3 codes
    # on both sides: the oracle's block sum is exact, so the device's deviation is the matrix
    # core's own arithmetic.  Measured: its error stays below 2^-11 of the block's absolute
    # sum T = sum |a_i w_i| (typically ~2^-14); exact whenever the products are integers of
    # like magnitude (the integer tests).  This bound is what the fp32-row tolerance of the
    # FP8 GEMM rests on: per output, sum_b s_b * 2^-11 * T_b over the K/128 blocks.
    g = np.random.default_rng(2024)
    rows, N, K = 512, 128, 128
    ratios = []
    for mode in ("all", "positive", "narrow"):
        a = finite_e4m3_codes(g, (rows, K))
        w = finite_e4m3_codes(g, (1, N, K))
        if mode == "positive":               # no cancellation: T equals |sum|
            a &= 0x7F
            w &= 0x7F
        if mode == "narrow":                 # exponents within a factor 4 of each other
            a = ((a & 0x80) | (0x38 + (a & 0x0F))).astype(np.uint8)
            w = ((w & 0x80) | (0x38 + (w & 0x0F))).astype(np.uint8)
        a_s = np.ones((1, rows), np.float32)
        w_s = np.ones((1, 1, 1), np.float32)
        off = np.array([0, rows], np.int32)
        got = gpu_gemm(a, a_s, w, w_s, off, 16, moe.MOE_EPI_STORE_F32).astype(np.float64)
        exact = orc.gemm_fp8(a, a_s, w, w_s, off)
        T = orc.gemm_fp8(a & 0x7F, a_s, w & 0x7F, w_s, off)
        nz = T > 0
        r = np.abs(got - exact)[nz] / T[nz]
        ratios.append(r)
        print(f"{mode}: max |err|/T = 2^{np.log2(r.max() + 1e-300):.2f}, "
              f"median 2^{np.log2(np.median(r) + 1e-300):.2f}, exact {np.mean(r == 0):.3f}")
    assert max(float(r.max()) for r in ratios) <= 2.0 ** -11


@pytest.mark.parametrize("chunk", [80, 256])
def test_gemm_tiled_multi_chunk_epilogues(chunk):
    # experts of 0, 1, 255, 256, 257 and 600 rows: full 256-row tiles, a one-row tile, ragged
    # tails inside 16- and 8-row groups; integer data with power-of-two scales is exact
    g = np.random.default_rng(chunk)
    E, N, K = 6, 384, 640
    counts = np.array([0, 1, 255, 256, 257, 600], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    Ai = g.integers(-4, 5, (rows, K))
    Wi = g.integers(-4, 5, (E, N, K))
    sa = np.exp2(g.integers(-1, 2, (K // 128, rows))).astype(np.float32)
    sb = np.exp2(g.integers(-1, 2, (E, N // 128, K // 128))).astype(np.float32)
    ref = orc.gemm_fp8(int_codes(Ai), sa, int_codes(Wi), sb, offsets).astype(np.float32)
    a_q, w_q = int_codes(Ai), int_codes(Wi)
    got = gpu_gemm(a_q, sa, w_q, sb, offsets, chunk, moe.MOE_EPI_STORE_F32, repeat=2)
    np.testing.assert_array_equal(got, ref)
    b16 = gpu_gemm(a_q, sa, w_q, sb, offsets, chunk, moe.MOE_EPI_STORE_BF16).view(np.uint16)
    np.testing.assert_array_equal(b16, synth.bf16_bits(ref))
    perm = g.permutation(rows).astype(np.int32)     # a route id per sorted row
    rt = gpu_gemm(a_q, sa, w_q, sb, offsets, chunk, moe.MOE_EPI_ROUTE_F32, sorted_ids=perm)
    np.testing.assert_array_equal(rt[perm], ref)


SCHEDS = (moe.MOE_SCHED_DISPATCH, moe.MOE_SCHED_STATIC, moe.MOE_SCHED_QUEUE,
          moe.MOE_SCHED_QUEUE_XCD)


def gpu_gemm_gather(x_q, x_s, ids, w_q, w_s, chunk, sched=moe.MOE_SCHED_AUTO, repeat=1):
    """moe_build_layout (sorted) + moe_grouped_gemm_gather on device; rows at route ids.  The
    task counters must come back zeroed (and the iteration-cap word clear)."""
    M, k = ids.shape
    E, N, K = w_q.shape
    nb = N // 128
    mt = moe.max_tasks(M, k, E, nb, chunk)
    counts, offsets, cursors = zeros(E, torch.int32), zeros(E + 1, torch.int32), zeros(E, torch.int32)
    tasks = zeros((mt, 4), torch.int32)
    ntasks, queue = zeros(1, torch.int32), zeros(moe.MOE_QUEUE_WORDS, torch.int32)
    srt = zeros(M * k, torch.int32)
    ids_d = to_dev(ids)
    moe.build_layout(ids_d, E, nb, chunk, counts, offsets, cursors, tasks, ntasks, queue,
                     sorted_route_ids=srt)
    rows = torch.full((M * k, N), -3.0, dtype=torch.float32, device=DEV)
    args = (to_dev(x_q), to_dev(x_s), k, to_dev(w_q), to_dev(w_s), tasks, ntasks, chunk, srt,
            rows)
    for _ in range(repeat):
        moe.grouped_gemm_gather(*args, queue=queue, sched=sched)
    sync()
    assert (to_np(queue) == 0).all(), "task counters not left zeroed"
    return to_np(rows)


@pytest.mark.parametrize("chunk", [96, 128, 256])
def test_gemm_gather_integer_exact(chunk):
    # token-major integer codes with power-of-two scales: the GEMM is exact in fp32; experts of
    # 0 .. 300 routes exercise full, ragged and one-row tiles
    g = np.random.default_rng(chunk)
    M, k, E, N, K = 160, 3, 5, 384, 640
    bias = np.array([3.0, 2.0, 0.0, -9.0, 1.0], np.float32)
    logits = (g.standard_normal((M, E)) + bias).astype(np.float32)
    ids, _ = orc.route(logits, k, CAP)
    Ai = g.integers(-4, 5, (M, K))
    Wi = g.integers(-4, 5, (E, N, K))
    sa = np.exp2(g.integers(-1, 2, (M, K // 128))).astype(np.float32)
    sb = np.exp2(g.integers(-1, 2, (E, N // 128, K // 128))).astype(np.float32)
    counts, offsets = orc.layout(ids, E)
    r_ids, a_q, a_s = orc.sort_gather(ids, offsets, int_codes(Ai), sa)
    C = orc.gemm_fp8(a_q, a_s, int_codes(Wi), sb, offsets).astype(np.float32)
    got = gpu_gemm_gather(int_codes(Ai), sa.T.copy(), ids, int_codes(Wi), sb, chunk)
    np.testing.assert_array_equal(got[r_ids], C)


@functools.lru_cache(maxsize=None)
def skewed_reference(name):
    """Oracle of a full-size skewed layer: ids, layout, every fp32 GEMM row (sorted order) and
    every output token (threads over disjoint token and expert sets)."""
    d = workload(name)
    ids, _ = orc.route(d["logits"], d["k"], CAP)
    counts, offsets = orc.layout(ids, d["E"])
    q, sc = orc.quant_act(d["x"])
    r_ids, a_q, a_s = orc.sort_gather(ids, offsets, q, sc)
    C = oracle_gemm_rows_by_expert(a_q, a_s, d["w_q"], d["w_s"], offsets)
    toks = np.arange(d["M"], dtype=np.int32)
    _, y64 = oracle_rows_parallel(orc.forward_tokens, toks, d["logits"], d["x"], d["w_q"],
                                  d["w_s"], d["k"], CAP)
    return dict(ids=ids, counts=counts, offsets=offsets, q=q, sc=sc, sorted=r_ids, C=C, y64=y64)


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("chunk", [96, 128])
def test_gemm_gather_schedules_integer_exact(chunk, sched):
    # every task schedule (hardware dispatch, static walk, one queue, per-XCD queues) on
    # integer codes with power-of-two scales: exact, and repeated launches reuse the counters
    g = np.random.default_rng(chunk + 7)
    M, k, E, N, K = 700, 3, 9, 512, 640
    bias = np.linspace(3.0, -3.0, E).astype(np.float32)
    logits = (g.standard_normal((M, E)) + bias).astype(np.float32)
    ids, _ = orc.route(logits, k, CAP)
    Ai = g.integers(-4, 5, (M, K))
    Wi = g.integers(-4, 5, (E, N, K))
    sa = np.exp2(g.integers(-1, 2, (M, K // 128))).astype(np.float32)
    sb = np.exp2(g.integers(-1, 2, (E, N // 128, K // 128))).astype(np.float32)
    counts, offsets = orc.layout(ids, E)
    r_ids, a_q, a_s = orc.sort_gather(ids, offsets, int_codes(Ai), sa)
    C = orc.gemm_fp8(a_q, a_s, int_codes(Wi), sb, offsets).astype(np.float32)
    got = gpu_gemm_gather(int_codes(Ai), sa.T.copy(), ids, int_codes(Wi), sb, chunk,
                          sched=sched, repeat=3)
    np.testing.assert_array_equal(got[r_ids], C)


@pytest.mark.parametrize("name", [ZIPF1K, ZIPF4K])
def test_gemm_gather_schedules_agree_on_skewed_layers(name):
    # the schedules only decide which workgroup runs a tile, so the rows are bit-identical
    d = workload(name)
    ref = skewed_reference(name)
    outs = [gpu_gemm_gather(ref["q"], ref["sc"].T.copy(), ref["ids"], d["w_q"], d["w_s"], 128,
                            sched=s, repeat=2) for s in SCHEDS]
    assert_gemm_f32_close(outs[0][ref["sorted"]], ref["C"], name)
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


def test_gemm_gather_persistent_schedules_refuse_256_row_chunks():
    d = workload(ZIPF1K)
    ref = skewed_reference(ZIPF1K)
    for s in SCHEDS[1:]:
        with pytest.raises(moe.MoeError):
            gpu_gemm_gather(ref["q"], ref["sc"].T.copy(), ref["ids"], d["w_q"], d["w_s"], 256,
                            sched=s)


@pytest.mark.parametrize("chunk", [128, 256])
@pytest.mark.parametrize("name", [ZIPF1K, ZIPF4K])
def test_gemm_gather_workload_rows(name, chunk):
    # full-size skewed layers: every fp32 row against the exact oracle row
    d = workload(name)
    ref = skewed_reference(name)
    got = gpu_gemm_gather(ref["q"], ref["sc"].T.copy(), ref["ids"], d["w_q"], d["w_s"], chunk)
    assert_gemm_f32_close(got[ref["sorted"]], ref["C"], f"{name} chunk={chunk}")


def test_gemm_random_store_modes():
    d = workload(TINY)
    ids, _ = orc.route(d["logits"], d["k"], CAP)
    counts, offsets = orc.layout(ids, d["E"])
    q, s = orc.quant_act(d["x"])
    sorted_ids, a_q, a_s = orc.sort_gather(ids, offsets, q, s)
    C = orc.gemm_fp8(a_q, a_s, d["w_q"], d["w_s"], offsets)
    f32 = gpu_gemm(a_q, a_s, d["w_q"], d["w_s"], offsets, 16, moe.MOE_EPI_STORE_F32)
    assert_gemm_f32_close(f32, C, "store f32")
    b16 = gpu_gemm(a_q, a_s, d["w_q"], d["w_s"], offsets, 16, moe.MOE_EPI_STORE_BF16)
    assert_bf16_close(b16.view(np.uint16), C, "store bf16")
    R = ids.size
    rt = gpu_gemm(a_q, a_s, d["w_q"], d["w_s"], offsets, 16, moe.MOE_EPI_ROUTE_F32,
                  sorted_ids=sorted_ids, out_rows=R)
    np.testing.assert_array_equal(rt[sorted_ids], f32)


def test_gemm_qwen_layer_rows():
    d = workload(QWEN)
    ids, _ = orc.route(d["logits"], d["k"], CAP)
    counts, offsets = orc.layout(ids, d["E"])
    q, s = orc.quant_act(d["x"])
    sorted_ids, a_q, a_s = orc.sort_gather(ids, offsets, q, s)
    C = orc.gemm_fp8(a_q, a_s, d["w_q"], d["w_s"], offsets)
    for chunk, queue in ((16, True), (16, False), (64, True), (256, True)):
        got = gpu_gemm(a_q, a_s, d["w_q"], d["w_s"], offsets, chunk, moe.MOE_EPI_STORE_F32,
                       queue=queue)
        assert_gemm_f32_close(got, C, f"chunk={chunk} queue={queue}")


def routed_case(name):
    """Inputs of the fused small-batch GEMM: a named workload, or (M, E, k, N, bias) at K=2048."""
    if isinstance(name, str):
        return workload(name)
    M, E, k, N, bias = name
    d = synth.fused_inputs(M, E, k, 2048, N, seed=M + E, bias=bias)
    d.update(M=M, E=E, k=k, K=2048, N=N)
    d["w_q"], d["w_s"] = orc.quant_weights(d["w"])
    return d


@pytest.mark.parametrize("name", [
    QWEN,
    (24, 40, 3, 256, None),     # 1.8 rows per expert; workgroup ranges cross expert boundaries
    (256, 16, 8, 256, None),    # 128 rows per expert: 8 tiles, two rounds of resident tiles
    (200, 64, 6, 384, "zipf"),  # skewed: a hot expert with several tiles, many with one
    (300, 600, 2, 128, None),   # more experts than CUs: ranges of several experts
    (1024, 64, 2, 256, None),   # 2048 routed rows, the most the kernel takes
])
def test_gemm_routed_matches_staged_oracle(name):
    # the fused small-batch GEMM: layout, sort/gather and quantisation inside the kernel; its
    # rows sit at route ids, so the oracle's sorted rows are permuted back before comparing
    d = routed_case(name)
    M, E, k, K, N = d["M"], d["E"], d["k"], d["K"], d["N"]
    ids, _ = orc.route(d["logits"], k, CAP)
    counts, offsets = orc.layout(ids, E)
    q, s = orc.quant_act(d["x"])
    sorted_ids, a_q, a_s = orc.sort_gather(ids, offsets, q, s)
    C = orc.gemm_fp8(a_q, a_s, d["w_q"], d["w_s"], offsets)
    ref = np.zeros_like(C)
    ref[sorted_ids] = C
    rows = zeros((M * k, N), torch.float32)
    cnt, off = zeros((E,), torch.int32), zeros((E + 1,), torch.int32)
    moe.grouped_gemm_routed(to_dev(d["x"]), to_dev(ids), E, to_dev(d["w_q"]), to_dev(d["w_s"]),
                            rows, cnt, off)
    sync()
    np.testing.assert_array_equal(to_np(cnt), counts)
    np.testing.assert_array_equal(to_np(off), offsets)
    assert_gemm_f32_close(to_np(rows), ref, f"routed {name}")


def test_gemm_routed_invalid_ids_and_repeat():
    # ids outside [0, E) route nowhere: their rows stay untouched; a second call on the same
    # buffers gives the same bits (no state kept between calls); counts/offsets may be NULL
    M, E, k, N = 40, 24, 4, 256
    d = routed_case((M, E, k, N, None))
    ids, _ = orc.route(d["logits"], k, CAP)
    bad = ids.copy()
    bad[3, 1], bad[17, 0], bad[39, 3] = -1, E, 1 << 20
    valid = (bad >= 0) & (bad < E)
    # a route's row depends only on its token and expert: the reference of the clean ids
    # holds every row the kernel must write
    counts, offsets = orc.layout(ids, E)
    q, s = orc.quant_act(d["x"])
    sorted_ids, a_q, a_s = orc.sort_gather(ids, offsets, q, s)
    C = orc.gemm_fp8(a_q, a_s, d["w_q"], d["w_s"], offsets)
    ref = np.zeros_like(C)
    ref[sorted_ids] = C
    flat = valid.reshape(-1)
    outs = []
    for _ in range(2):
        rows = torch.full((M * k, N), 7.0, dtype=torch.float32, device="cuda")
        moe.grouped_gemm_routed(to_dev(d["x"]), to_dev(bad), E, to_dev(d["w_q"]),
                                to_dev(d["w_s"]), rows)
        sync()
        outs.append(to_np(rows))
    np.testing.assert_array_equal(outs[0], outs[1])
    assert (outs[0][~flat] == 7.0).all()
    assert_gemm_f32_close(outs[0][flat], ref[flat], "routed, invalid ids")


# ---- stage 5: scatter --------------------------------------------------------------------

def test_scatter_matches_oracle():
    g = np.random.default_rng(8)
    M, k, E, N = 37, 8, 64, 384
    ids = np.stack([g.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
    w = g.random((M, k)).astype(np.float32)
    rows = g.standard_normal((M * k, N)).astype(np.float32)
    out = zeros((M, N), torch.int16)
    moe.scatter(to_dev(rows), to_dev(w), to_dev(ids), E, out)
    sync()
    y, y64 = orc.scatter(rows.astype(np.float64), np.arange(M * k, dtype=np.int32), w, M)
    got = to_np(out).view(np.uint16)
    assert_bf16_close(got, y64, "scatter")
    # fp32 sum of 8 terms, then one rounding: at most one bf16 ulp from the exact rounding
    diff = np.abs(got.astype(np.int32) - y.astype(np.int32))
    assert diff.max() <= 1


# ---- whole forward -----------------------------------------------------------------------

def gpu_forward(d, flags=0, chunk=0, reps=1, keep_ws=False):
    M, E, k, K, N = d["M"], d["E"], d["k"], d["K"], d["N"]
    ws = zeros(moe.forward_workspace_bytes(M, E, k, K, N), torch.uint8)
    out = zeros((M, N), torch.int16)
    args = [to_dev(d["logits"]), to_dev(d["x"]), to_dev(d["w_q"]), to_dev(d["w_s"])]
    outs = []
    for _ in range(reps):
        out.fill_(0)
        moe.forward(*args, k, CAP, out, ws, chunk_rows=chunk, flags=flags)
        sync()
        outs.append(to_np(out).view(np.uint16).copy())
    return (outs, ws) if keep_ws else outs


def ws_part(ws, d, which, dtype, count):
    off = moe.forward_workspace_offset(d["M"], d["E"], d["k"], d["K"], d["N"], which)
    nbytes = count * np.dtype(dtype).itemsize
    return to_np(ws[off:off + nbytes]).view(dtype)


@pytest.mark.parametrize("flags", [0, moe.MOE_FWD_GRAPH, moe.MOE_FWD_STATIC_GRID,
                                   moe.MOE_FWD_STAGED, moe.MOE_FWD_ROUTE_KERNEL])
@pytest.mark.parametrize("name", [TINY, QWEN])
def test_forward_full(name, flags):
    d = workload(name)
    ref = orc.forward(d["logits"], d["x"], d["w_q"], d["w_s"], d["k"], CAP,
                      intermediates=True)
    (outs, ws) = gpu_forward(d, flags=flags, reps=3, keep_ws=True)
    for y in outs:
        assert_bf16_close(y, ref["y64"], f"{name} flags={flags}")
        np.testing.assert_array_equal(y, outs[0])     # replays are bit-identical
    R = d["M"] * d["k"]
    np.testing.assert_array_equal(ws_part(ws, d, 0, np.int32, R).reshape(d["M"], d["k"]),
                                  ref["ids"])
    M, E, k, K, N = d["M"], d["E"], d["k"], d["K"], d["N"]
    if moe.forward_kernels(M, E, k, K, N, 0, flags) in (4, 5):  # (the small-batch path has none)
        np.testing.assert_array_equal(ws_part(ws, d, 2, np.int32, d["E"]), ref["counts"])
        np.testing.assert_array_equal(ws_part(ws, d, 3, np.int32, d["E"] + 1), ref["offsets"])
    else:
        assert not flags & moe.MOE_FWD_STAGED


@pytest.mark.parametrize("chunk", [0, 64, 256])
@pytest.mark.parametrize("name", [ZIPF1K, ZIPF4K])
def test_forward_skewed_full(name, chunk):
    # the whole output of the Zipf-skewed layers against the oracle, for the default chunk
    # (the gathering tiled path), 64-row chunks (staged, general GEMM) and 256-row tiles
    d = workload(name)
    ref = skewed_reference(name)
    counts = ref["counts"]
    assert counts.min() >= 1 and counts.max() / counts.min() >= 10
    outs, ws = gpu_forward(d, reps=2, chunk=chunk, keep_ws=True)
    R = d["M"] * d["k"]
    np.testing.assert_array_equal(ws_part(ws, d, 0, np.int32, R).reshape(d["M"], d["k"]),
                                  ref["ids"])
    np.testing.assert_array_equal(ws_part(ws, d, 2, np.int32, d["E"]), counts)
    np.testing.assert_array_equal(ws_part(ws, d, 3, np.int32, d["E"] + 1), ref["offsets"])
    s_ids = ws_part(ws, d, 8, np.int32, R)
    if moe.forward_kernels(d["M"], d["E"], d["k"], d["K"], d["N"], chunk) == 4:
        # the layout over many workgroups keeps each segment in ascending route id, the
        # oracle's counting-sort order
        np.testing.assert_array_equal(s_ids, ref["sorted"])
    else:
        np.testing.assert_array_equal(s_ids[canonical_segments(s_ids, ref["offsets"])],
                                      ref["sorted"])
    for o in outs:
        assert_bf16_close(o, ref["y64"], f"{name} chunk={chunk}")
        np.testing.assert_array_equal(o, outs[0])


@pytest.mark.parametrize("name", [ZIPF1K, ZIPF4K])
def test_forward_skewed_schedules(name):
    # the whole layer under each task schedule of its tiled GEMM: bit-identical outputs
    d = workload(name)
    ref = skewed_reference(name)
    base = None
    for s in SCHEDS:
        outs, ws = gpu_forward(d, reps=2, flags=moe.MOE_FWD_SCHED(s), keep_ws=True)
        assert (ws_part(ws, d, 7, np.uint32, moe.MOE_QUEUE_WORDS) == 0).all()
        if base is None:
            base = outs[0]
            assert_bf16_close(base, ref["y64"], f"{name} sched={s}")
        for o in outs:
            np.testing.assert_array_equal(o, base)


@pytest.mark.parametrize("chunk", [0, 256])
@pytest.mark.parametrize("name", [ZIPF1K, ZIPF4K])
def test_forward_skewed_atomic_combine(name, chunk):
    # the pages' scatter-add combine (fp32 atomics into token rows, then bf16): the whole
    # output against the oracle; the fp32 sums follow arrival order, so repeats may differ in
    # the last bit but stay within the bar; repeated calls reuse the accumulator rows
    d = workload(name)
    ref = skewed_reference(name)
    outs = gpu_forward(d, reps=3, chunk=chunk, flags=moe.MOE_FWD_ATOMIC_COMBINE)
    for o in outs:
        assert_bf16_close(o, ref["y64"], f"{name} atomic combine chunk={chunk}")
    # against the gather-sum: one bf16 step, plus the fp32 summation-order difference near
    # zero (k terms of magnitude ~rms in either order differ by a few fp32 ulps of rms)
    plain = bf16_f64(gpu_forward(d, chunk=chunk)[0])
    rms = float(np.sqrt(np.mean(plain ** 2)))
    diff = np.abs(bf16_f64(outs[0]) - plain)
    assert (diff <= bf16_ulp(plain) + 2.0 ** -18 * rms).all()


def test_forward_atomic_combine_only_on_the_gathering_path():
    d = workload(QWEN)                               # the small-batch path
    with pytest.raises(moe.MoeError):
        gpu_forward(d, flags=moe.MOE_FWD_ATOMIC_COMBINE)


@pytest.mark.parametrize("M,E,k", [(700, 1024, 3), (1500, 1000, 2), (345, 64, 8)])
def test_forward_wide_layout_edges(M, E, k):
    # the layout over many workgroups at its limits: up to 1024 experts (11-bit ballot match,
    # a 16 x 1024 table of wave counts), route counts that leave the last 1024-route chunk
    # ragged, and many empty experts; counts, offsets and the sorted route ids equal the
    # oracle's exactly, and the whole output passes the oracle's bar
    K, N = 256, 128
    d = synth.fused_inputs(M, E, k, K, N, seed=M + E)
    d.update(M=M, E=E, k=k, K=K, N=N)
    d["w_q"], d["w_s"] = orc.quant_weights(d["w"])
    assert moe.forward_kernels(M, E, k, K, N, 128) == 4
    outs, ws = gpu_forward(d, chunk=128, reps=2, keep_ws=True)
    ref = orc.forward(d["logits"], d["x"], d["w_q"], d["w_s"], k, CAP, intermediates=True)
    R = M * k
    np.testing.assert_array_equal(ws_part(ws, d, 2, np.int32, E), ref["counts"])
    np.testing.assert_array_equal(ws_part(ws, d, 3, np.int32, E + 1), ref["offsets"])
    np.testing.assert_array_equal(ws_part(ws, d, 8, np.int32, R), ref["sorted_route_ids"])
    for o in outs:
        assert_bf16_close(o, ref["y64"], f"wide layout M={M} E={E} k={k}")
        np.testing.assert_array_equal(o, outs[0])


@pytest.mark.parametrize("name", [ZIPF1K, ZIPF4K])
def test_forward_skewed_layout_repeats(name):
    # across repeated forwards the integer outputs (ids, counts, offsets, the set of tasks,
    # the sorted route ids) stay identical and every output is bit-identical.  (Partial chunks
    # of equal size are placed by LDS atomics, so their order in the task list is one of
    # several correct orders.)
    d = workload(name)
    ref = skewed_reference(name)
    R, E = d["M"] * d["k"], d["E"]
    mt = moe.max_tasks(d["M"], d["k"], E, d["N"] // 128, 128)
    first = None
    for _ in range(5):
        outs, ws = gpu_forward(d, reps=1, keep_ws=True)
        nt = int(ws_part(ws, d, 6, np.int32, 1)[0])
        tasks = ws_part(ws, d, 5, np.int32, 4 * nt).reshape(nt, 4)
        tasks = tasks[np.lexsort(tasks.T[::-1])]                 # as a set
        s_ids = ws_part(ws, d, 8, np.int32, R)
        cur = (ws_part(ws, d, 2, np.int32, E), ws_part(ws, d, 3, np.int32, E + 1), tasks,
               s_ids, outs[0])
        if first is None:
            first = cur
            assert 0 < nt <= mt
            np.testing.assert_array_equal(cur[3], ref["sorted"])
            r_tasks = orc.tasks(ref["counts"], ref["offsets"], d["N"] // 128, 128)
            np.testing.assert_array_equal(tasks, r_tasks[np.lexsort(r_tasks.T[::-1])])
        for a, b in zip(cur, first):
            np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("M,E,k,K,N,bias", [
    (1, 16, 1, 128, 128, None),        # one token, one expert, smallest tiles
    (3, 8, 8, 256, 256, None),         # k = E: every expert
    (64, 8, 1, 384, 256, "one"),       # every route on one expert -> several chunks
    (200, 300, 3, 128, 384, None),     # E not a multiple of 64, empty experts
    (17, 64, 4, 2176, 128, None),      # K over one 2048 pass, ragged
    (100, 300, 3, 2048, 384, None),    # fused small-batch path: E not a multiple of 64, Nb=3
    (512, 512, 4, 2048, 128, None),    # fused path at its limits (2048 routes, 512 experts,
                                       # one panel): ranges span several tile rounds
])
def test_forward_edge_shapes(M, E, k, K, N, bias):
    b = None
    if bias == "one":
        b = np.zeros(E, np.float32)
        b[3] = 50.0
    d = synth.fused_inputs(M, E, k, K, N, seed=M + E, bias=b)
    d.update(M=M, E=E, k=k, K=K, N=N)
    d["w_q"], d["w_s"] = orc.quant_weights(d["w"])
    ref = orc.forward(d["logits"], d["x"], d["w_q"], d["w_s"], k, CAP)
    for flags, chunk in ((0, 0), (moe.MOE_FWD_STATIC_GRID, 0), (moe.MOE_FWD_STAGED, 0),
                        (0, 256), (0, 100)):
        y = gpu_forward(d, flags=flags, chunk=chunk)[0]
        assert_bf16_close(y, ref["y64"], f"edge M={M} E={E} k={k} K={K} N={N} chunk={chunk}")


def random_layer_shapes(n=24, seed=2026):
    """Seeded layer shapes (M, E, k, K, N) spread over every path the forward can take: one
    to several hundred tokens, one to a few hundred experts, k up to E, K a multiple of 128
    (half of them 2048, the small-batch GEMM's depth) and one to four 128-column panels;
    shapes whose oracle or weight quantisation would take more than about a second are
    drawn again."""
    g = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        M = int(np.exp(g.uniform(0, np.log(700))))
        E = int(np.exp(g.uniform(0, np.log(400))))
        k = int(g.integers(1, min(E, 10) + 1))
        K = 2048 if g.random() < 0.5 else 128 * int(g.integers(1, 17))
        N = 128 * int(g.integers(1, 5))
        if E * N * K > 48 * 2 ** 20 or M * k * K * N > 1.2e9:
            continue
        shapes.append((M, E, k, K, N))
    return shapes


@pytest.mark.parametrize("M,E,k,K,N", random_layer_shapes())
def test_forward_random_shapes(M, E, k, K, N):
    # whole output against the oracle on seeded shapes that no hand-picked case names
    # (E = 1, k = E, a token or two, hundreds of routes per expert, ragged K), in the default
    # launch form and in the staged one
    d = synth.fused_inputs(M, E, k, K, N, seed=M * 1009 + E * 31 + k * 7 + K + N)
    d.update(M=M, E=E, k=k, K=K, N=N)
    d["w_q"], d["w_s"] = orc.quant_weights(d["w"])
    ref = orc.forward(d["logits"], d["x"], d["w_q"], d["w_s"], k, CAP)
    for flags in (0, moe.MOE_FWD_STAGED):
        n = moe.forward_kernels(M, E, k, K, N, 0, flags)
        print(f"shape M={M} E={E} k={k} K={K} N={N} flags={flags}: {n} kernels", flush=True)
        y = gpu_forward(d, flags=flags)[0]
        assert_bf16_close(y, ref["y64"], f"M={M} E={E} k={k} K={K} N={N} flags={flags}")


@pytest.mark.parametrize("mode", ["handoff", "handoff_graph", "self"])
@pytest.mark.parametrize("M,E,k,N", [
    (128, 256, 8, 512),     # the M=128, E=256, top-8 layer
    (1, 16, 1, 128),        # one token: one routing wave; 128 workgroups without slices exit
    (8, 16, 2, 256),        # the tiny layer's routing at K = 2048
    (300, 128, 4, 128),     # more tokens than workgroups: second waves route as well
    (2048, 128, 1, 128),    # every wave of every workgroup routes a token
])
def test_forward_fused_route_matches_three_kernels(M, E, k, N, mode):
    # the two-kernel step (the default: route inside the small-batch GEMM, routes handed over
    # through tagged words in the workspace) against the three-kernel step: the same ids,
    # weights and output bits, call after call, starting from a workspace full of old bytes;
    # the combine leaves the words cleared.  "self": no handoff, every wave routes the tokens
    # it reads itself (the path a wave takes when its routing wave is late), which sets the
    # handoff status word; the handoff leaves it untouched.
    K = 2048
    d = synth.fused_inputs(M, E, k, K, N, seed=M + 7 * E)
    d.update(M=M, E=E, k=k, K=K, N=N)
    d["w_q"], d["w_s"] = orc.quant_weights(d["w"])
    flags = {"handoff": 0, "handoff_graph": moe.MOE_FWD_GRAPH,
             "self": moe.MOE_FWD_ROUTE_SELF}[mode]
    assert moe.forward_kernels(M, E, k, K, N, 0, flags) == 2
    assert moe.forward_kernels(M, E, k, K, N, 0, flags | moe.MOE_FWD_ROUTE_KERNEL) == 3
    (base, ws3) = gpu_forward(d, reps=1, keep_ws=True, flags=moe.MOE_FWD_ROUTE_KERNEL)
    ws = zeros(moe.forward_workspace_bytes(M, E, k, K, N), torch.uint8)
    ws.fill_(0xA5)
    out = zeros((M, N), torch.int16)
    args = [to_dev(d["logits"]), to_dev(d["x"]), to_dev(d["w_q"]), to_dev(d["w_s"])]
    R = M * k
    for rep in range(4):
        out.fill_(0)
        moe.forward(*args, k, CAP, out, ws, flags=flags)
        sync()
        np.testing.assert_array_equal(to_np(out).view(np.uint16), base[0], f"call {rep}")
        for part, dt in ((0, np.int32), (1, np.float32)):
            np.testing.assert_array_equal(ws_part(ws, d, part, dt, R), ws_part(ws3, d, part, dt, R))
        assert (ws_part(ws, d, 12, np.uint32, R) == 0).all(), "route words left set"
        status = ws_part(ws, d, 7, np.uint32, moe.MOE_QUEUE_WORDS)[moe.MOE_QUEUE_HANDOFF_STATUS]
        assert status == (1 if mode == "self" else 0xA5A5A5A5), hex(status)
    ref = orc.forward(d["logits"], d["x"], d["w_q"], d["w_s"], k, CAP)
    assert_bf16_close(base[0], ref["y64"], f"fused route M={M} E={E} k={k} N={N}")


@pytest.mark.parametrize("K", [256, 512, 1024])
@pytest.mark.parametrize("M,E,k,N", [
    (8, 16, 2, 256),        # the tiny layer
    (120, 64, 8, 128),      # 960 routes, 15 per expert
    (33, 40, 5, 384),       # E not a multiple of 64, three panels
])
def test_forward_small_batch_depths(M, E, k, N, K):
    # the small-batch GEMM at the depths below 2048: the route inside (two kernels) and as a
    # kernel of its own (three) give the same bits, and both match the oracle; the staged
    # step (five kernels) matches it too
    d = synth.fused_inputs(M, E, k, K, N, seed=M + E + K)
    d.update(M=M, E=E, k=k, K=K, N=N)
    d["w_q"], d["w_s"] = orc.quant_weights(d["w"])
    ref = orc.forward(d["logits"], d["x"], d["w_q"], d["w_s"], k, CAP)
    assert moe.forward_kernels(M, E, k, K, N, 0, 0) == 2
    assert moe.forward_kernels(M, E, k, K, N, 0, moe.MOE_FWD_ROUTE_KERNEL) == 3
    two = gpu_forward(d, reps=2)
    three = gpu_forward(d, flags=moe.MOE_FWD_ROUTE_KERNEL)[0]
    staged = gpu_forward(d, flags=moe.MOE_FWD_STAGED)[0]
    for y in two:
        np.testing.assert_array_equal(y, three)
    assert_bf16_close(three, ref["y64"], f"small batch M={M} E={E} k={k} K={K} N={N}")
    assert_bf16_close(staged, ref["y64"], f"staged M={M} E={E} k={k} K={K} N={N}")


@pytest.mark.parametrize("flags", [0, 256])
def test_forward_fused_route_ties_and_non_finite_logits(flags):
    # the route inside the GEMM (handed over, or taken by every wave itself: flags 256 =
    # MOE_FWD_ROUTE_SELF) follows the route's order on crafted rows: all tied, ten tied above
    # the rest (the k/k+1 boundary), NaN (below every number) and +inf logits; ids against the
    # oracle's route, output bits against the three-kernel step
    M, E, k, K, N = 16, 64, 4, 2048, 128
    d = synth.fused_inputs(M, E, k, K, N, seed=5)
    lg = d["logits"]
    lg[0, :] = 1.0
    lg[1, 10:20] = 3.0
    lg[2, :] = np.nan
    lg[2, 7] = -5.0
    lg[3, ::2] = np.nan
    lg[4, 60:] = np.inf
    d.update(M=M, E=E, k=k, K=K, N=N)
    d["w_q"], d["w_s"] = orc.quant_weights(d["w"])
    assert moe.forward_kernels(M, E, k, K, N, 0, flags) == 2
    (base, ws3) = gpu_forward(d, reps=1, keep_ws=True, flags=moe.MOE_FWD_ROUTE_KERNEL)
    (got, ws2) = gpu_forward(d, flags=flags, reps=2, keep_ws=True)
    R = M * k
    r_ids, _ = orc.route(lg, k, CAP)
    np.testing.assert_array_equal(ws_part(ws2, d, 0, np.int32, R).reshape(M, k), r_ids)
    np.testing.assert_array_equal(ws_part(ws3, d, 0, np.int32, R).reshape(M, k), r_ids)
    for y in got:
        np.testing.assert_array_equal(y, base[0])


def test_forward_fused_route_only_where_it_applies():
    # the route moves into the GEMM by default on the small-batch path (K = 256, 512, 1024 or
    # 2048) with E <= 256; E above 256, a batch outside that path, another K, the staged flag
    # or MOE_FWD_ROUTE_KERNEL keep the route kernel
    assert moe.forward_kernels(128, 256, 8, 2048, 512, 0, 0) == 2
    assert moe.forward_kernels(128, 256, 8, 2048, 512, 0, moe.MOE_FWD_ROUTE_KERNEL) == 3
    assert moe.forward_kernels(100, 300, 3, 2048, 384, 0, 0) == 3
    assert moe.forward_kernels(8, 16, 2, 256, 256, 0, 0) == 2
    assert moe.forward_kernels(8, 16, 2, 256, 256, 0, moe.MOE_FWD_ROUTE_KERNEL) == 3
    assert moe.forward_kernels(8, 16, 2, 384, 256, 0, 0) == 5
    assert moe.forward_kernels(8, 16, 2, 4096, 256, 0, 0) == 5
    assert moe.forward_kernels(1024, 256, 8, 2048, 512, 0, 0) == 4
    # the edge of the small-batch path: 2048 routed rows stay on it; 2056 (9 per expert,
    # 16-row chunks) take the staged form
    assert moe.forward_kernels(256, 256, 8, 2048, 512, 0, 0) == 2
    assert moe.forward_kernels(257, 256, 8, 2048, 512, 0, 0) == 5
    assert moe.forward_kernels(128, 256, 8, 2048, 512, 0, moe.MOE_FWD_STAGED) == 5


def test_forward_repeat_determinism():
    d = workload(QWEN)
    outs = gpu_forward(d, reps=20)
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
