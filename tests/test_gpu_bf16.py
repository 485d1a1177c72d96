"""GPU parity of the BF16 grouped GEMM (large routed-row counts) against the CPU oracle.

The oracle computes every output in double from the bf16 operands.  fp32 outputs are held to
a tolerance derived from the arithmetic: bf16 x bf16 products are exact in fp32 and the matrix
core accumulates in fp32, so the error is a few fp32 roundings per 16-wide k step
(GEMM_BF16_F32_*).  bf16 stores use the BF16 output bar and lie within one bf16 ulp of the
oracle's own bf16 rounding; SwiGLU outputs are held to their bf16 rounding per element.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from mixture_experts_layer_softcap_amd import moe, synth

from gpu_util import (assert_bf16_close, bf16_f64, oracle_rows_parallel, to_dev, to_np,
                      zeros)

pytestmark = pytest.mark.gpu

# fp32 rows against the double oracle: K/16 fp32 accumulations of exact products
GEMM_BF16_F32_REL_FRO = 2e-5
GEMM_BF16_F32_ELEM_RMS = 2e-4
CHUNK = 256


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    orc.build(force=False)
    assert moe.device_check() == moe.MOE_OK


def layout_for_counts(counts, n_blocks, chunk=CHUNK):
    """Task list for expert-contiguous rows with these per-expert counts (k = 1 routing)."""
    counts = np.asarray(counts, np.int32)
    E = counts.shape[0]
    rows = int(counts.sum())
    ids = np.repeat(np.arange(E, dtype=np.int32), counts).reshape(rows, 1)
    mt = moe.max_tasks(rows, 1, E, n_blocks, chunk)
    dev = dict(counts=zeros((E,), torch.int32), offsets=zeros((E + 1,), torch.int32),
               cursors=zeros((E,), torch.int32), tasks=zeros((max(mt, 1), 4), torch.int32),
               ntasks=zeros((1,), torch.int32), queue=zeros((moe.MOE_QUEUE_WORDS,), torch.int32))
    moe.build_layout(to_dev(ids), E, n_blocks, chunk, dev["counts"], dev["offsets"],
                     dev["cursors"], dev["tasks"], dev["ntasks"], dev["queue"])
    return dev


SCHEDS = (moe.MOE_SCHED_DISPATCH, moe.MOE_SCHED_STATIC, moe.MOE_SCHED_QUEUE,
          moe.MOE_SCHED_QUEUE_XCD)


def run_gemm(A, W, counts, epilogue, out_cols=None, sched=moe.MOE_SCHED_AUTO, repeat=1):
    rows, K = A.shape
    E, N, _ = W.shape
    lay = layout_for_counts(counts, N // moe.gemm_n_tile(moe.MOE_GEMM_BF16))
    cols = N if out_cols is None else out_cols
    dt = torch.float32 if epilogue == moe.MOE_EPI_STORE_F32 else torch.int16
    out = zeros((rows, cols), dt)
    args = (to_dev(A), None, to_dev(W), None, lay["tasks"], lay["ntasks"], CHUNK, out, epilogue)
    for _ in range(repeat):
        moe.grouped_gemm(moe.MOE_GEMM_BF16, *args, queue=lay["queue"], sched=sched)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(lay["counts"]), counts)
    assert (to_np(lay["queue"]) == 0).all(), "task counters not left zeroed"
    return to_np(out, None if dt == torch.float32 else np.uint16)


def assert_f32_close(y, ref, what=""):
    ref = np.asarray(ref, np.float64)
    y = np.asarray(y, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    fro = float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))
    worst = float(np.abs(y - ref).max())
    assert fro <= GEMM_BF16_F32_REL_FRO, f"{what}: rel Frobenius {fro:.3e}"
    assert worst <= GEMM_BF16_F32_ELEM_RMS * rms, f"{what}: max |d| {worst:.3e} vs rms {rms:.3e}"


def inputs(rows, E, N, K, dist, seed=0, counts=None):
    d = synth.grouped_gemm_inputs(rows, E, N, K, dist, seed=seed)
    if counts is not None:
        d["counts"] = np.asarray(counts, np.int32)
        d["offsets"] = np.concatenate([[0], np.cumsum(d["counts"])]).astype(np.int32)
    return d


@pytest.mark.parametrize("rows,E,N,K,dist", [
    (700, 5, 512, 192, "random"),      # chunks of 256 + partial chunks, K of 3 steps
    (513, 3, 256, 64, "skewed"),       # one k step; a 1-row tail chunk likely
    (300, 4, 768, 1024, "balanced"),   # 16 k steps, three column panels
])
def test_bf16_gemm_f32_matches_oracle(rows, E, N, K, dist):
    d = inputs(rows, E, N, K, dist, seed=rows)
    y = run_gemm(d["A"], d["W"], d["counts"], moe.MOE_EPI_STORE_F32)
    _, ref = orc.gemm_bf16(d["A"], d["W"], d["offsets"])
    assert_f32_close(y, ref, f"rows={rows}")


def test_bf16_gemm_bf16_store_and_edge_counts():
    # an empty expert, a single-row expert, a 31-row expert and one just over a chunk
    counts = [0, 1, 31, 257]
    d = inputs(sum(counts), 4, 512, 128, "balanced", seed=3, counts=counts)
    y = run_gemm(d["A"], d["W"], d["counts"], moe.MOE_EPI_STORE_BF16)
    bits, ref = orc.gemm_bf16(d["A"], d["W"], d["offsets"])
    assert_bf16_close(y, ref, "bf16 store")
    # bf16 of the fp32 accumulation lies within one bf16 ulp of the oracle's bf16(double)
    diff = np.abs(bf16_f64(y) - bf16_f64(bits))
    ulp = np.abs(bf16_f64(bits)) * 2.0 ** -7 + 1e-30
    assert (diff <= ulp).all()


def test_bf16_gemm_swiglu_epilogue():
    rows, E, N, K = 600, 3, 512, 256       # gate rows [0, 256), up rows [256, 512)
    d = inputs(rows, E, N, K, "random", seed=11)
    y = run_gemm(d["A"], d["W"], d["counts"], moe.MOE_EPI_SWIGLU_BF16, out_cols=N // 2)
    _, h = orc.gemm_bf16(d["A"], d["W"], d["offsets"])
    g, u = h[:, : N // 2], h[:, N // 2:]
    ref = g / (1.0 + np.exp(-g)) * u
    # The product is heavy-tailed (its largest entries are tens of rms), so the bound per
    # element is the bf16 rounding itself (RNE: 2^-9 relative; 2^-8 leaves room for the fp32
    # accumulation and fp32 silu) plus a small absolute term for entries near zero, and the
    # Frobenius part of the BF16 output bar.
    yv = bf16_f64(y)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bad = np.abs(yv - ref) > 2.0 ** -8 * np.abs(ref) + 1e-5 * rms
    assert not bad.any(), f"swiglu: {int(bad.sum())} entries beyond bf16 rounding"
    fro = float(np.linalg.norm(yv - ref) / np.linalg.norm(ref))
    assert fro <= 5e-3, f"swiglu: relative Frobenius {fro:.3e}"


def test_bf16_gemm_full_up_projection_sampled():
    # the gated-up projection at 4096 routed rows, E=16, H=3072, I=1536 (Dirichlet(1) rows);
    # the oracle checks every expert's first and last row plus a seeded sample
    rows, E, N, K = 4096, 16, 3072, 3072
    d = inputs(rows, E, N, K, "random", seed=0)
    y = run_gemm(d["A"], d["W"], d["counts"], moe.MOE_EPI_STORE_F32)
    off = d["offsets"]
    pick = set()
    for e in range(E):
        if d["counts"][e]:
            pick.update((int(off[e]), int(off[e + 1]) - 1))
    pick.update(np.random.default_rng(5).choice(rows, 32, replace=False).tolist())
    rl = np.array(sorted(pick), np.int32)
    _, ref = orc.gemm_bf16(d["A"], d["W"], off, rows_list=rl)
    assert_f32_close(y[rl], ref, "up projection sample")


def test_bf16_gemm_five_panels_ragged_tile_groups():
    # N = 1280 is five 256-column panels, so a tile group of 4 panels leaves a 1-panel group
    # per chunk run; 9 chunks are not a multiple of the 8-chunk groups either.  Full output.
    counts = [700, 0, 1100, 1]          # 3 + 0 + 5 + 1 chunks of up to 256 rows
    rows, E, N, K = sum(counts), 4, 1280, 256
    d = inputs(rows, E, N, K, "balanced", seed=21, counts=counts)
    y = run_gemm(d["A"], d["W"], d["counts"], moe.MOE_EPI_STORE_F32)
    _, ref = oracle_rows_parallel(orc.gemm_bf16, np.arange(rows, dtype=np.int32), d["A"],
                                  d["W"], d["offsets"])
    assert_f32_close(y, ref, "N=1280")


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("epilogue", [moe.MOE_EPI_STORE_F32, moe.MOE_EPI_STORE_BF16,
                                      moe.MOE_EPI_SWIGLU_BF16])
def test_bf16_gemm_schedules(epilogue, sched):
    # each task schedule and epilogue on a skewed split with an empty expert, ragged chunks and
    # ten k steps (one pass of the six stage phases plus four): the schedule only decides which
    # workgroup runs a tile, so outputs are bit-identical to hardware dispatch; fp32 rows are
    # also checked against the oracle; repeated launches reuse the counters
    counts = [900, 0, 37, 1300, 257]
    rows, E, N, K = sum(counts), 5, 1024, 640
    d = inputs(rows, E, N, K, "balanced", seed=31, counts=counts)
    cols = N // 2 if epilogue == moe.MOE_EPI_SWIGLU_BF16 else None
    y = run_gemm(d["A"], d["W"], d["counts"], epilogue, out_cols=cols, sched=sched, repeat=2)
    y0 = run_gemm(d["A"], d["W"], d["counts"], epilogue, out_cols=cols,
                  sched=moe.MOE_SCHED_DISPATCH)
    np.testing.assert_array_equal(y, y0)
    if epilogue == moe.MOE_EPI_STORE_F32:
        _, ref = oracle_rows_parallel(orc.gemm_bf16, np.arange(rows, dtype=np.int32), d["A"],
                                      d["W"], d["offsets"])
        assert_f32_close(y, ref, f"sched={sched}")


def chunk_edge_rows(counts, chunk=CHUNK):
    """Sorted rows at every chunk's first and last row (which covers every expert's first
    and last row): every task and every tile group of the launch is touched."""
    off = np.concatenate([[0], np.cumsum(counts)])
    pick = []
    for e, c in enumerate(counts):
        for b in range(0, int(c), chunk):
            pick += [int(off[e]) + b, int(off[e]) + min(b + chunk, int(c)) - 1]
    return np.unique(np.array(pick, np.int32))


@pytest.mark.parametrize("proj", ["up", "down"])
@pytest.mark.parametrize("rows,dist", [(29446, "random"), (65536, "skewed")])
def test_bf16_gemm_bench_sizes(rows, dist, proj):
    # the timed shapes (E=16, H=3072, I=1536): gated-up [rows,3072]x[3072,3072] and down
    # [rows,1536]x[1536,3072]; fp32 rows at every chunk boundary against the oracle
    N, K = (3072, 3072) if proj == "up" else (3072, 1536)
    d = inputs(rows, 16, N, K, dist, seed=0)
    y = run_gemm(d["A"], d["W"], d["counts"], moe.MOE_EPI_STORE_F32)
    rl = chunk_edge_rows(d["counts"])
    _, ref = oracle_rows_parallel(orc.gemm_bf16, rl, d["A"], d["W"], d["offsets"])
    assert_f32_close(y[rl], ref, f"{proj} rows={rows} {dist}")
    assert np.isfinite(y).all()
    if rows == 29446:
        for sched in SCHEDS[1:]:
            yq = run_gemm(d["A"], d["W"], d["counts"], moe.MOE_EPI_STORE_F32, sched=sched)
            np.testing.assert_array_equal(yq, y)


# ---- the Mixtral-like expert FFN layer ------------------------------------------------

def test_sort_gather_bf16_copies_rows_into_segments():
    T, E, k, H = 333, 8, 2, 512
    d = synth.ffn_inputs(T, E, H, 256, seed=4, weights=False)
    ids, _ = orc.route(d["logits"], k, 30.0)
    counts, offsets = orc.layout(ids, E)
    R = T * k
    cur = to_dev(offsets[:E].copy())
    srt, slots = zeros((R,), torch.int32), zeros((R,), torch.int32)
    a = zeros((R, H), torch.int16)
    moe.sort_gather_bf16(to_dev(d["x"]), to_dev(ids), E, cur, srt, a, route_slots=slots)
    torch.cuda.synchronize()
    srt, slots, a = to_np(srt), to_np(slots), to_np(a, np.uint16)
    np.testing.assert_array_equal(to_np(cur), offsets[1:])
    r = np.arange(R)
    np.testing.assert_array_equal(srt[slots], r)                  # slots are a permutation
    np.testing.assert_array_equal(a[slots], d["x"][r // k])      # rows copied bit for bit
    for e in range(E):                                            # segment membership
        seg = np.sort(srt[offsets[e]:offsets[e + 1]])
        np.testing.assert_array_equal(seg, np.flatnonzero(ids.reshape(-1) == e))


def run_ffn(d, k, chunk=0):
    logits, x, wu, wd = d["logits"], d["x"], d["w_up"], d["w_down"]
    T, E = logits.shape
    H, F = x.shape[1], wd.shape[2]
    ws = torch.empty(moe.ffn_workspace_bytes(T, E, k, H, F), dtype=torch.uint8, device="cuda")
    out = zeros((T, H), torch.int16)
    moe.ffn_forward(to_dev(logits), to_dev(x), to_dev(wu), to_dev(wd), k, 30.0, out, ws,
                    chunk_rows=chunk)
    torch.cuda.synchronize()
    return to_np(out, np.uint16)


@pytest.mark.parametrize("chunk", [0, 64])
def test_ffn_layer_small_full(chunk):
    T, E, k, H, F = 300, 8, 2, 512, 256
    d = synth.ffn_inputs(T, E, H, F, seed=7)
    y = run_ffn(d, k, chunk)
    _, ref = orc.ffn_tokens(d["logits"], d["x"], d["w_up"], d["w_down"], k, 30.0)
    assert_bf16_close(y, ref, f"ffn chunk={chunk}")


def random_ffn_shapes(n=10, seed=2027):
    """Seeded FFN layer shapes (T, E, k, H, F, chunk): one token to several hundred, one to 24
    experts, k up to min(E, 4), hidden and FFN widths of one to four tiles, chunk 0 (the
    default) or 64 / 128 / 256 rows; shapes whose oracle would take more than about a second
    are drawn again."""
    g = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        T = int(np.exp(g.uniform(0, np.log(600))))
        E = int(g.integers(1, 25))
        k = int(g.integers(1, min(E, 4) + 1))
        H = 256 * int(g.integers(1, 5))
        F = 128 * int(g.integers(1, 5))
        chunk = int(g.choice([0, 64, 128, 256]))
        if T * k * 3 * F * H > 6e8:
            continue
        shapes.append((T, E, k, H, F, chunk))
    return shapes


@pytest.mark.parametrize("T,E,k,H,F,chunk", random_ffn_shapes())
def test_ffn_layer_random_shapes(T, E, k, H, F, chunk):
    # whole layer against the oracle on seeded shapes no hand-picked case names (one expert,
    # k = E, a single token, ragged last chunks at every chunk size)
    d = synth.ffn_inputs(T, E, H, F, seed=T * 131 + E * 17 + k + H + F)
    print(f"ffn T={T} E={E} k={k} H={H} F={F} chunk={chunk}", flush=True)
    y = run_ffn(d, k, chunk)
    _, ref = orc.ffn_tokens(d["logits"], d["x"], d["w_up"], d["w_down"], k, 30.0)
    assert_bf16_close(y, ref, f"ffn T={T} E={E} k={k} H={H} F={F} chunk={chunk}")


def ffn_ws_part(ws, T, E, k, H, F, which, dtype, n):
    off = moe.ffn_workspace_offset(T, E, k, H, F, which)
    return to_np(ws[off:off + n * np.dtype(dtype).itemsize]).view(dtype)


@pytest.mark.parametrize("T", [8192, 32768])
def test_ffn_layer_mixtral_shape_chunk_edges(T):
    # E=8, top-2, hidden 4096, FFN 1024, skewed router (-1.1 ln(e+1) bias): every token whose
    # route sits at a chunk's first or last sorted row (both GEMMs' tasks cut the same
    # chunks), plus a seeded spread, against the oracle
    E, k, H, F = 8, 2, 4096, 1024
    d = synth.ffn_inputs(T, E, H, F, seed=0)
    logits, x, wu, wd = d["logits"], d["x"], d["w_up"], d["w_down"]
    ws = torch.empty(moe.ffn_workspace_bytes(T, E, k, H, F), dtype=torch.uint8, device="cuda")
    out = zeros((T, H), torch.int16)
    moe.ffn_forward(to_dev(logits), to_dev(x), to_dev(wu), to_dev(wd), k, 30.0, out, ws)
    torch.cuda.synchronize()
    y = to_np(out, np.uint16)
    for sched in SCHEDS[1:]:              # every schedule gives the same bits
        out2 = zeros((T, H), torch.int16)
        moe.ffn_forward(to_dev(logits), to_dev(x), to_dev(wu), to_dev(wd), k, 30.0, out2, ws,
                        flags=moe.MOE_FWD_SCHED(sched))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(out2, np.uint16), y)
        q = ffn_ws_part(ws, T, E, k, H, F, 12, np.uint32, 2 * moe.MOE_QUEUE_WORDS)
        assert (q == 0).all()
    ids, _ = orc.route(logits, k, 30.0)
    counts, offsets = orc.layout(ids, E)
    np.testing.assert_array_equal(ffn_ws_part(ws, T, E, k, H, F, 2, np.int32, E), counts)
    np.testing.assert_array_equal(ffn_ws_part(ws, T, E, k, H, F, 3, np.int32, E + 1), offsets)
    srt = ffn_ws_part(ws, T, E, k, H, F, 8, np.int32, T * k)
    # the layout's segments hold their routes in ascending route id: a stable sort by expert
    np.testing.assert_array_equal(srt, np.argsort(ids.ravel(), kind="stable"))
    edges = chunk_edge_rows(counts)
    tok = np.unique(np.concatenate([srt[edges] // k,
                                    np.random.default_rng(1).choice(T, 32, replace=False)]))
    tok = tok.astype(np.int32)
    _, ref = oracle_rows_parallel(orc.ffn_tokens, tok, logits, x, wu, wd, k, 30.0)
    assert_bf16_close(y[tok], ref, f"ffn T={T} ({tok.size} tokens)")
