"""Benchmark of the fused FP8 MoE forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole forward (route -> layout -> QSG -> FP8 grouped GEMM -> combine), enqueued
as plain kernel launches (--graph replays the library's cached HIP graph instead), on the
Qwen3.5-35B-A3B-shaped layer of the Fused MoE
FP8 tutorial's problem table: M=128 tokens, 256 experts, top-8, K=2048, N=512.  Inputs are
seeded synthetic data resident in HBM before timing; the weights are rotated over enough
copies (>= 1 GiB) that every step streams them from HBM rather than from the 256 MB
Infinity Cache.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
SCHEDS = {"auto": -1, "dispatch": 0, "static": 1, "queue": 2, "queue_xcd": 3}
WEIGHT_BYTES_ROTATION = 1 << 30


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="fused_fp8_M128_E256_k8_K2048_N512")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--staged", action="store_true",
                   help="run the five staged kernels even where the fused small-batch path "
                        "(route, fused GEMM, combine) applies")
    p.add_argument("--static-grid", action="store_true",
                   help="walk the task list with a fixed stride instead of the atomic queue")
    p.add_argument("--chunk-rows", type=int, default=0)
    p.add_argument("--sched", default="auto", choices=list(SCHEDS),
                   help="task schedule of the LDS-tiled grouped GEMMs: hardware dispatch of one "
                        "workgroup per task, a static persistent walk, one atomic queue, or "
                        "per-XCD atomic queues (auto: the library's default)")
    p.add_argument("--atomic-combine", action="store_true",
                   help="gathering path: the scatter-add combine (fp32 atomics into token rows, "
                        "then bf16) instead of fp32 routed rows and a gather-sum kernel")
    p.add_argument("--route-kernel", action="store_true",
                   help="small-batch path: the route as a kernel of its own (three kernels) "
                        "instead of inside the grouped GEMM (two, the default)")
    p.add_argument("--graph", action="store_true",
                   help="replay the cached HIP graph of the step instead of launching its kernels")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run ten device-to-device copies of MIB MiB (a kernel of known "
                        "traffic for scaling the HBM byte counters) and exit")
    return p.parse_args()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of the timed grouped GEMM from the committed rocprofv3 counter
    record (FETCH_SIZE + WRITE_SIZE, copy-calibrated) for this workload and kernel, or None
    when there is none or the kernel's source has changed since the counters were taken."""
    import glob
    import hashlib

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_bytes.json"))):
        with open(path) as f:
            rec = json.load(f)
        if rec.get("workload") != workload or not rec.get("kernel", "").startswith(kernel):
            continue
        # every source file the kernel is built from must be unchanged since the counters
        srcs = rec.get("sources") or {rec["source"]: rec["source_sha256"]}
        same = True
        for rel, sha in srcs.items():
            path = os.path.join(ROOT, rel)
            if not os.path.exists(path):
                same = False
                break
            with open(path, "rb") as f:
                same &= hashlib.sha256(f.read()).hexdigest() == sha
        if same:
            return rec["traffic_bytes"]
    return None


def gemm_algorithmic_bytes(counts, M, k, K, N, fused=False, gather=False, E=0):
    """Bytes the grouped GEMM must move: each non-empty expert's FP8 weights and scales once,
    the fp32 routed output rows once, and its inputs once: the routed FP8 rows, their scales
    and sorted ids (staged), the token-major FP8 rows, their scales and the sorted ids
    (gather), or the bf16 token rows and the routed ids (fused: layout, gather and
    quantisation inside the GEMM).  With E > 0 the route runs inside as well: the logits
    [M][E] in place of the routed ids, and the ids and weights written."""
    nonempty = int((counts > 0).sum())
    R = M * k
    Nb, Kb = N // 128, K // 128
    weights = nonempty * (N * K + Nb * Kb * 4)
    if fused and E:
        return weights + M * K * 2 + M * E * 4 + R * N * 4 + R * 8
    if fused:
        acts = M * K * 2 + R * 4
    elif gather:
        acts = M * K + Kb * M * 4 + R * 4
    else:
        acts = R * K + Kb * R * 4 + R * 4
    out = R * N * 4
    return weights + acts + out


def layer_algorithmic_bytes(counts, M, E, k, K, N):
    """Bytes the whole layer must move: used expert weights + scales, logits, x, output."""
    nonempty = int((counts > 0).sum())
    return nonempty * (N * K + (N // 128) * (K // 128) * 4) + M * E * 4 + M * K * 2 + M * N * 2


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), for the CPU baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, k, cap, budget_s=12.0):
    import oracle

    oracle.build(force=not os.path.exists(oracle.LIB_PATH))
    w_q, w_s = oracle.quant_weights(d["w"])          # input preparation, not timed
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or len(times) < 3:
        t0 = time.perf_counter()
        oracle.forward(d["logits"], d["x"], w_q, w_s, k, cap)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {"value": med * 1e6, "unit": "us/layer", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"whole layer ({d['M']} tokens, fp64 single-threaded C oracle), "
                      f"median of {len(times)} runs; host has {os.cpu_count()} cores"}


# BF16 grouped GEMMs of the gated-up and down projections over compact routed rows (E=16,
# H=3072, I=1536: up [rows,3072] x [3072,3072], down [rows,1536] x [1536,3072]).
BF16_GEMMS = {"up": (3072, 3072), "down": (3072, 1536)}   # N, K
BF16_DENSE_PEAK_TFLOPS = 2500.0                          # MI355X dense BF16 MFMA, published


def bench_bf16_gemm(args, moe, synth, torch, np):
    """--workload bf16_grouped_gemm_<up|down>_rows<R>_<balanced|random|skewed>: one grouped
    GEMM per step (tasks built once, outside timing), fp32 accumulate, bf16 out."""
    _, _, _, proj, rows_s, dist = args.workload.split("_")
    N, K = BF16_GEMMS[proj]
    rows, E, chunk = int(rows_s[4:]), 16, 256
    d = synth.grouped_gemm_inputs(rows, E, N, K, dist, seed=0)
    dev = torch.device("cuda:0")
    a = torch.from_numpy(d["A"].view(np.int16)).to(dev)
    w0 = torch.from_numpy(d["W"].view(np.int16)).to(dev)
    copies = max(1, -(-WEIGHT_BYTES_ROTATION // (w0.numel() * 2)))
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    counts = d["counts"]
    ids = torch.from_numpy(np.repeat(np.arange(E, dtype=np.int32), counts).reshape(rows, 1)).to(dev)
    nb = N // moe.gemm_n_tile(moe.MOE_GEMM_BF16)
    mt = moe.max_tasks(rows, 1, E, nb, chunk)
    z = lambda n: torch.zeros(n, dtype=torch.int32, device=dev)
    cnt, off, cur, ntasks, queue = z(E), z(E + 1), z(E), z(1), z(moe.MOE_QUEUE_WORDS)
    tasks = z(mt * 4).view(mt, 4)
    moe.build_layout(ids, E, nb, chunk, cnt, off, cur, tasks, ntasks, queue)
    out = torch.empty((rows, N), dtype=torch.int16, device=dev)

    def step(i):
        moe.grouped_gemm(moe.MOE_GEMM_BF16, a, None, ws[i % copies], None, tasks, ntasks, chunk,
                         out, moe.MOE_EPI_STORE_BF16, queue=queue, sched=SCHEDS[args.sched])

    for i in range(max(args.warmup, copies)):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)]
    us = evs[0].elapsed_time(evs[-1]) * 1e3 / args.steps
    flops = 2.0 * rows * N * K
    tflops = flops / (us * 1e-6) / 1e12
    nonempty = int((counts > 0).sum())
    gbytes = rows * K * 2 + nonempty * N * K * 2 + rows * N * 2
    result = {
        "metric": "µs per BF16 grouped GEMM + TFLOPS & %MFMA peak",
        "value": round(us, 3), "unit": "us/gemm", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": rows, "E": E, "N": N, "K": K,
                   "row_distribution": dist, "nonempty_experts": nonempty, "chunk_rows": chunk,
                   "sched": args.sched,
                   "max_expert_rows": int(counts.max()), "weight_copies_rotated": copies},
        "effective_tflops": round(tflops, 2),
        "us_p10_p50_p90": [round(float(np.percentile(per, q)), 2) for q in (10, 50, 90)],
        "roofline": {"bound": "mfma", "kernel": "gemm_bf16_kernel (STORE_BF16)",
                     "achieved": round(tflops, 2), "peak": BF16_DENSE_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_DENSE_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload, "gemm_bf16_kernel"),
                     "algorithmic_bytes_per_launch": gbytes,
                     "hbm_frac": round(gbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(us, 3)},
    }
    print(json.dumps(result))


def bench_dense_library(args, synth, torch, np):
    """--workload bf16_dense_library_<up|down>_rows<R>: context for the grouped GEMM, never a
    path of this library.  The same compact rows as ONE dense bf16 GEMM [rows,K] x [K,N]
    (expert 0's weights as the right operand, contiguous) through torch.mm, i.e. the vendor
    GEMM library, with fp32 accumulation: the best case a library reaches on this shape with
    no grouping, no partial chunks and no gather."""
    _, _, _, proj, rows_s = args.workload.split("_")
    N, K = BF16_GEMMS[proj]
    rows = int(rows_s[4:])
    d = synth.grouped_gemm_inputs(rows, 1, N, K, "balanced", seed=0)
    dev = torch.device("cuda:0")
    a = torch.from_numpy(d["A"].view(np.int16)).to(dev).view(torch.bfloat16)
    b = torch.from_numpy(d["W"][0].view(np.int16)).to(dev).view(torch.bfloat16).t().contiguous()
    out = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)
    for _ in range(args.warmup):
        torch.mm(a, b, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        torch.mm(a, b, out=out)
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / args.steps
    tflops = 2.0 * rows * N * K / (us * 1e-6) / 1e12
    print(json.dumps({
        "metric": "µs per dense BF16 GEMM through torch.mm (library reference, context only)",
        "value": round(us, 3), "unit": "us/gemm", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": rows, "N": N, "K": K,
                   "library": f"torch {torch.__version__} mm"},
        "effective_tflops": round(tflops, 2),
        "roofline": {"bound": "mfma", "kernel": "library GEMM", "achieved": round(tflops, 2),
                     "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_DENSE_PEAK_TFLOPS, 4), "traffic": None,
                     "avg_launch_us": round(us, 3)},
    }))


def bench_ffn(args, moe, synth, torch, np):
    """--workload ffn_mixtral_T<T>[_uniform]: the whole Mixtral-like expert FFN layer (E=8,
    top-2, hidden 4096, FFN 1024, bf16), router logits skewed by -1.1 ln(e+1) unless
    _uniform; --chunk-rows picks the task chunk (0 = 256)."""
    parts = args.workload.split("_")
    T = int(parts[2][1:])
    skewed = not (len(parts) > 3 and parts[3] == "uniform")
    E, k, H, F = 8, 2, 4096, 1024
    d = synth.ffn_inputs(T, E, H, F, seed=0, skewed=skewed)
    dev = torch.device("cuda:0")
    tl = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    logits, x, wu, wd = tl(d["logits"]), tl(d["x"]), tl(d["w_up"]), tl(d["w_down"])
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    ws = torch.empty(moe.ffn_workspace_bytes(T, E, k, H, F), dtype=torch.uint8, device=dev)
    sched = SCHEDS[args.sched]

    def step(i):
        moe.ffn_forward(logits, x, wu, wd, k, synth.SOFTCAP, out, ws, chunk_rows=args.chunk_rows,
                        flags=moe.MOE_FWD_SCHED(sched) if sched >= 0 else 0)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)]
    us = evs[0].elapsed_time(evs[-1]) * 1e3 / args.steps
    off = moe.ffn_workspace_offset(T, E, k, H, F, 2)
    counts = ws[off:off + 4 * E].view(torch.int32).cpu().numpy()
    rows = T * k
    flops = 2.0 * rows * (2 * F * H + H * F)
    tflops = flops / (us * 1e-6) / 1e12
    result = {
        "metric": "µs per Mixtral-like FFN layer + TFLOPS & %MFMA peak",
        "value": round(us, 3), "unit": "us/layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "E": E, "top_k": k, "hidden": H,
                   "ffn": F, "chunk_rows": args.chunk_rows or 256, "skewed_router": skewed,
                   "sched": args.sched,
                   "rows_per_expert_max_min": [int(counts.max()), int(counts.min())]},
        "effective_tflops": round(tflops, 2),
        "us_p10_p50_p90": [round(float(np.percentile(per, q)), 2) for q in (10, 50, 90)],
        "roofline": {"bound": "mfma", "kernel": "whole layer (gemm_bf16_kernel x2 + glue)",
                     "achieved": round(tflops, 2), "peak": BF16_DENSE_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_DENSE_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload, "whole layer"),
                     "avg_launch_us": round(us, 3)},
    }
    print(json.dumps(result))


def bench_router(args, moe, synth, torch, np):
    """--workload router_M<M>_H<H>_E<E>: the router projection (moe_router_logits) alone,
    logits f32 [M,E] = x bf16 [M,H] . w_gate bf16 [E,H]^T; HBM-bound (x and w_gate read once)."""
    _, ms, hs, es = args.workload.split("_")
    M, H, E = int(ms[1:]), int(hs[1:]), int(es[1:])
    d = synth.router_inputs(M, H, E, seed=0)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
    wg = torch.from_numpy(d["w_gate"].view(np.int16)).to(dev)
    out = torch.empty((M, E), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        moe.router_logits(x, wg, out)
    torch.cuda.synchronize()
    eager = out.clone()
    # one call is a few microseconds of GPU work, less than a ctypes call costs on the host, so
    # the timed steps are one captured graph of K back-to-back calls (the kernel launches only;
    # the projection allocates and clears nothing), replayed once warm and once timed
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for i in range(args.steps):
                moe.router_logits(x, wg, out)
    torch.cuda.current_stream().wait_stream(cs)
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, eager):
        raise SystemExit("router graph replay differs from the eager call")
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    # plain launches from Python, for the host-bound figure
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        moe.router_logits(x, wg, out)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)]
    us_plain = evs[0].elapsed_time(evs[-1]) * 1e3 / args.steps
    nbytes = M * H * 2 + E * H * 2 + M * E * 4
    achieved = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "µs per router projection + %HBM roofline",
        "value": round(us, 3), "unit": "us/call", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (fp32 accumulate, fp32 out)",
        "data": "synthetic", "config": {"workload": args.workload, "M": M, "H": H, "E": E},
        "effective_tflops": round(2.0 * M * H * E / (us * 1e-6) / 1e12, 3),
        "timing": "one graph of K back-to-back calls",
        "us_per_call_plain_launches": round(us_plain, 3),
        "plain_us_p10_p50_p90": [round(float(np.percentile(per, q)), 2) for q in (10, 50, 90)],
        "roofline": {"bound": "hbm", "kernel": "router_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, "router_kernel"),
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": round(us, 3)}}))


def bench_mlp(args, moe, synth, torch, np):
    """--workload mlp_fp8_M<M>_E<E>_k<k>_H<H>_I<I>: the whole FP8 expert MLP layer per step
    (route, layouts, QSG, gate+up FP8 GEMM, silu(g)*u requantise, down FP8 GEMM, combine);
    the dominant kernel, the gate+up GEMM, is also timed alone on the step's own inputs."""
    d = synth.mlp_inputs(**synth.MLP_WORKLOADS[args.workload])
    M, E, k, H, I, cap = d["M"], d["E"], d["k"], d["H"], d["I"], d["cap"]
    dev = torch.device("cuda:0")
    tl = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    logits, x = tl(d["logits"]), tl(d["x"])
    w1 = (tl(d["w1_q"]), tl(d["w1_s"]))
    w2 = (tl(d["w2_q"]), tl(d["w2_s"]))
    wbytes = w1[0].numel() + w2[0].numel()
    copies = max(1, -(-WEIGHT_BYTES_ROTATION // wbytes))
    w1s = [w1] + [(w1[0].clone(), w1[1].clone()) for _ in range(copies - 1)]
    w2s = [w2] + [(w2[0].clone(), w2[1].clone()) for _ in range(copies - 1)]
    out = torch.empty((M, H), dtype=torch.int16, device=dev)
    ws = torch.empty(moe.mlp_workspace_bytes(M, E, k, H, I), dtype=torch.uint8, device=dev)

    def step(i):
        a, b = w1s[i % copies], w2s[i % copies]
        moe.mlp_forward(logits, x, a[0], a[1], b[0], b[1], k, cap, out, ws,
                        chunk_rows=args.chunk_rows)

    for i in range(max(args.warmup, copies)):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)]
    us = evs[0].elapsed_time(evs[-1]) * 1e3 / args.steps

    def wsp(i, dtype, n):
        o = moe.mlp_workspace_offset(M, E, k, H, I, i)
        return ws[o:o + n * torch.tensor([], dtype=dtype).element_size()].view(dtype)

    R = M * k
    chunk = args.chunk_rows or (16 if -(-R // E) <= 16 else (128 if H <= 8192 else 64))
    nkern = moe.mlp_forward_kernels(M, E, k, H, I, args.chunk_rows)
    fused = nkern in (3, 4)
    h1 = torch.empty((R, 2 * I), dtype=torch.float32, device=dev)
    if nkern == 3:
        # the gate+up GEMM alone with the route inside, as the step runs it
        ids_b = torch.empty((M, k), dtype=torch.int32, device=dev)
        wts_b = torch.empty((M, k), dtype=torch.float32, device=dev)
        words = torch.zeros(R, dtype=torch.int32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)

        def gemm(i):
            a = w1s[i % copies]
            moe.route_grouped_gemm(logits, x, k, cap, a[0], a[1], ids_b, wts_b, words, status,
                                   h1)
    elif fused:
        # the gate+up GEMM alone, straight from the routed ids the last step left (part 0)
        ids_ws = wsp(0, torch.int32, R).view(M, k)

        def gemm(i):
            a = w1s[i % copies]
            moe.grouped_gemm_routed(x, ids_ws, E, a[0], a[1], h1)
    else:
        # the gate+up GEMM alone on the sorted FP8 rows, tasks and ids the last step left
        mtu = moe.max_tasks(M, k, E, 2 * I // 128, chunk)
        a_q = wsp(10, torch.uint8, R * H).view(R, H)
        a_s = wsp(11, torch.float32, (H // 128) * R)
        tasks = wsp(5, torch.int32, 4 * mtu).view(mtu, 4)
        nt = wsp(7, torch.int32, 1)
        o7 = moe.mlp_workspace_offset(M, E, k, H, I, 7)
        queue = ws[o7 + 64:o7 + 64 + 4 * moe.MOE_QUEUE_WORDS].view(torch.int32)
        sorted_ids = wsp(8, torch.int32, R)

        def gemm(i):
            a = w1s[i % copies]
            moe.grouped_gemm(moe.MOE_GEMM_FP8_B128, a_q, a_s, a[0], a[1], tasks, nt, chunk,
                             h1, moe.MOE_EPI_STORE_F32, queue=queue,
                             sorted_route_ids=sorted_ids)

    for i in range(2 * copies):
        gemm(i)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for i in range(args.steps):
        gemm(i)
    g1.record(stream)
    torch.cuda.synchronize()
    gemm_us = g0.elapsed_time(g1) * 1e3 / args.steps

    ids_np = wsp(0, torch.int32, R).cpu().numpy()
    counts = np.bincount(ids_np, minlength=E)
    nonempty = int((counts > 0).sum())
    N1 = 2 * I
    acts = (M * H * 2 + M * E * 4 + R * 8) if nkern == 3 else \
        (M * H * 2 + R * 4) if fused else (R * H + (H // 128) * R * 4 + R * 4)
    gbytes = nonempty * (N1 * H + (N1 // 128) * (H // 128) * 4) + acts + R * N1 * 4
    achieved = gbytes / (gemm_us * 1e-6) / 1e9
    lbytes = nonempty * (N1 * H + (N1 // 128) * (H // 128) * 4 + H * I + (H // 128) * (I // 128) * 4) \
        + M * E * 4 + M * H * 2 + M * H * 2
    flops = 2.0 * R * (N1 * H + H * I)
    gemm_kernel = (f"gemm_fp8_fused_kernel<{H // 128}, true, true, false> (the route inside the "
                   "gate+up grouped FP8 GEMM from routed ids, rows at route ids)" if nkern == 3 else
                   f"gemm_fp8_fused_kernel<{H // 128}, true, false, false> (gate+up grouped FP8 GEMM "
                   "from routed ids, rows at route ids)" if fused else
                   "gemm_fp8_range_kernel (gate+up grouped FP8 GEMM, STORE_F32)"
                   if H == 2048 and chunk <= 16 else
                   "gemm_fp8_tile_kernel (gate+up grouped FP8 GEMM, STORE_F32)"
                   if 64 < chunk <= 256 and H <= 8192 else
                   "gemm_fp8_kernel (gate+up grouped FP8 GEMM, STORE_F32)")
    result = {
        "metric": "µs/layer + effective TFLOPS & %HBM roofline, FP8 expert MLP",
        "value": round(us, 3), "unit": "us/layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)", "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "E": E, "top_k": k, "H": H, "I": I,
                   "softcap": cap, "weight_copies_rotated": copies, "chunk_rows": chunk,
                   "path": ("3 kernels: gate+up GEMM routing its tokens itself, down GEMM "
                            "from the same ids forming silu*up and requantising it in its tile "
                            "build, combine" if nkern == 3 else
                            "4 kernels: route, gate+up GEMM from the routed ids, down GEMM from "
                            "the same ids forming silu*up and requantising it in its tile build, "
                            "combine" if fused else
                            "7 kernels: route, layout (both task lists), QSG, gate+up GEMM, "
                            "silu*up requantise, down GEMM, combine")},
        "effective_tflops": round(flops / (us * 1e-6) / 1e12, 3),
        "us_p10_p50_p90": [round(float(np.percentile(per, q)), 2) for q in (10, 50, 90)],
        "layer_hbm_frac": round(lbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_algorithmic_bytes": lbytes,
        "nonempty_experts": nonempty,
        "roofline": {"bound": "hbm", "kernel": gemm_kernel,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, gemm_kernel.split(" (")[0]),
                     "algorithmic_bytes_per_launch": gbytes,
                     "avg_launch_us": round(gemm_us, 3)},
    }
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=not os.path.exists(oracle.LIB_PATH))
        times = []
        t_end = time.perf_counter() + 12.0
        while time.perf_counter() < t_end or len(times) < 2:
            t0 = time.perf_counter()
            oracle.mlp_tokens(d["logits"], d["x"], d["w1_q"], d["w1_s"], d["w2_q"], d["w2_s"],
                              k, cap)
            times.append(time.perf_counter() - t0)
        result["cpu_baseline"] = {
            "value": statistics.median(times) * 1e6, "unit": "us/layer", "cores": 1,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"whole layer ({M} tokens, fp64 single-threaded C oracle), median of "
                      f"{len(times)} runs; host has {os.cpu_count()} cores"}
    print(json.dumps(result))


def staged_gemm(args, moe, torch, wsp, M, E, k, K, N, chunk, wqs, wss, copies, rows_out):
    """The staged step's grouped GEMM alone (ROUTE_F32 epilogue) on the task list, FP8 rows and
    scales the last staged forward left in the workspace."""
    R = M * k
    a_q = wsp(9, torch.uint8, R * K).view(R, K)
    a_s = wsp(10, torch.float32, (K // 128) * R)
    max_tasks = moe.max_tasks(M, k, E, N // 128, chunk)
    tasks = wsp(5, torch.int32, 4 * max_tasks).view(max_tasks, 4)
    ntasks = wsp(6, torch.int32, 1)
    queue = None if args.static_grid else wsp(7, torch.int32, moe.MOE_QUEUE_WORDS)
    sorted_ids = wsp(8, torch.int32, R)

    def gemm(i):
        moe.grouped_gemm(moe.MOE_GEMM_FP8_B128, a_q, a_s, wqs[i % copies], wss[i % copies],
                         tasks, ntasks, chunk, rows_out, moe.MOE_EPI_ROUTE_F32, queue=queue,
                         sorted_route_ids=sorted_ids)
    return gemm


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the expert-parallel path across GPUs is not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_layer_softcap_amd import moe, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 10}))
        return
    rc = moe.device_check()
    assert rc == moe.MOE_OK, f"not a gfx950 device ({rc})"

    if args.workload.startswith("bf16_grouped_gemm_"):
        bench_bf16_gemm(args, moe, synth, torch, np)
        return
    if args.workload.startswith("bf16_dense_library_"):
        bench_dense_library(args, synth, torch, np)
        return
    if args.workload.startswith("ffn_mixtral_"):
        bench_ffn(args, moe, synth, torch, np)
        return
    if args.workload.startswith("mlp_fp8_"):
        bench_mlp(args, moe, synth, torch, np)
        return
    if args.workload.startswith("router_"):
        bench_router(args, moe, synth, torch, np)
        return
    d = synth.workload_inputs(args.workload)
    M, E, k, K, N, cap = d["M"], d["E"], d["k"], d["K"], d["N"], d["cap"]

    # inputs resident in HBM; weights quantised on the GPU by the library
    logits = torch.from_numpy(d["logits"]).to(dev)
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
    w32 = torch.from_numpy(d["w"]).to(dev)
    wq0 = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    ws0 = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
    moe.quantize_weights(w32, wq0, ws0)
    del w32
    copies = max(1, -(-WEIGHT_BYTES_ROTATION // wq0.numel()))
    wqs = [wq0] + [wq0.clone() for _ in range(copies - 1)]
    wss = [ws0] + [ws0.clone() for _ in range(copies - 1)]
    out = torch.empty((M, N), dtype=torch.int16, device=dev)
    ws = torch.empty(moe.forward_workspace_bytes(M, E, k, K, N), dtype=torch.uint8, device=dev)
    sched = SCHEDS[args.sched]
    flags = (moe.MOE_FWD_STATIC_GRID if args.static_grid else 0) | \
        (moe.MOE_FWD_GRAPH if args.graph else 0) | (moe.MOE_FWD_STAGED if args.staged else 0) | \
        (moe.MOE_FWD_SCHED(sched) if sched >= 0 else 0) | \
        (moe.MOE_FWD_ATOMIC_COMBINE if args.atomic_combine else 0) | \
        (moe.MOE_FWD_ROUTE_KERNEL if args.route_kernel else 0)

    def step(i):
        moe.forward(logits, x, wqs[i % copies], wss[i % copies], k, cap, out, ws,
                    chunk_rows=args.chunk_rows, flags=flags)

    for i in range(max(args.warmup, copies)):
        step(i)
    torch.cuda.synchronize()

    # ---- whole-step timing: K back-to-back steps between two events (the value), then K
    # more with an event after every step for the spread (an event between steps adds its
    # own marker to the stream, so the second pass is not the value) ----------------------
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    us_layer = total_ms * 1e3 / args.steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(args.steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)]   # us
    us_evented = evs[0].elapsed_time(evs[-1]) * 1e3 / args.steps

    # routing statistics of this input (its routed ids read back, outside timing)
    off = moe.forward_workspace_offset(M, E, k, K, N, 0)
    ids_np = ws[off:off + 4 * M * k].view(torch.int32).cpu().numpy()
    counts = np.bincount(ids_np[(ids_np >= 0) & (ids_np < E)], minlength=E)

    # ---- dominant kernel alone: the grouped GEMM, same launch configuration ------------
    def wsp(i, dtype, n):
        o = moe.forward_workspace_offset(M, E, k, K, N, i)
        return ws[o:o + n * torch.tensor([], dtype=dtype).element_size()].view(dtype)

    R = M * k
    chunk = args.chunk_rows or (16 if -(-R // E) <= 16 else (128 if K <= 8192 else 64))
    nkern = moe.forward_kernels(M, E, k, K, N, args.chunk_rows, flags)
    fused = nkern in (2, 3)
    gather = not args.staged and 64 < chunk <= 256 and K <= 8192
    rows_out = torch.empty((R, N), dtype=torch.float32, device=dev)
    if gather:
        # the step's tiled GEMM on what the last step left in the workspace: token-major codes
        # and scales, the task list and the sorted route ids
        x_q = wsp(13, torch.uint8, M * K).view(M, K)
        x_s = wsp(14, torch.float32, (K // 128) * M)
        max_tasks = moe.max_tasks(M, k, E, N // 128, chunk)
        tasks = wsp(5, torch.int32, 4 * max_tasks).view(max_tasks, 4)
        ntasks = wsp(6, torch.int32, 1)
        sorted_ids = wsp(8, torch.int32, R)
        queue = wsp(7, torch.int32, moe.MOE_QUEUE_WORDS)

        def gemm(i):
            moe.grouped_gemm_gather(x_q, x_s, k, wqs[i % copies], wss[i % copies], tasks, ntasks,
                                    chunk, sorted_ids, rows_out, queue=queue, sched=sched)
    elif nkern == 2:
        # the step's first kernel alone: the route inside the grouped GEMM (its route words
        # need no clearing between launches: each launch tags them anew)
        ids_b = torch.empty((M, k), dtype=torch.int32, device=dev)
        wts_b = torch.empty((M, k), dtype=torch.float32, device=dev)
        words = torch.zeros(R, dtype=torch.int32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)

        def gemm(i):
            moe.route_grouped_gemm(logits, x, k, cap, wqs[i % copies], wss[i % copies], ids_b,
                                   wts_b, words, status, rows_out)
    elif fused:
        # the step's GEMM reads the routed ids (workspace part 0, written by its route stage)
        ids_ws = wsp(0, torch.int32, R).view(M, k)

        def gemm(i):
            moe.grouped_gemm_routed(x, ids_ws, E, wqs[i % copies], wss[i % copies], rows_out)
    else:
        # one staged step writes the task list, FP8 rows, scales and sorted ids it times
        moe.forward(logits, x, wqs[0], wss[0], k, cap, out, ws, chunk_rows=args.chunk_rows,
                    flags=flags | moe.MOE_FWD_STAGED)
        torch.cuda.synchronize()
        gemm = staged_gemm(args, moe, torch, wsp, M, E, k, K, N, chunk, wqs, wss, copies,
                           rows_out)
    for i in range(copies * 2):
        gemm(i)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for i in range(args.steps):
        gemm(i)
    g1.record(stream)
    torch.cuda.synchronize()
    gemm_us = g0.elapsed_time(g1) * 1e3 / args.steps
    gbytes = gemm_algorithmic_bytes(counts, M, k, K, N, fused, gather, E if nkern == 2 else 0)
    achieved = gbytes / (gemm_us * 1e-6) / 1e9

    if gather:
        gemm_kernel = ("gemm_fp8_tile_kernel (grouped FP8 GEMM, LDS-staged tiles gathered from "
                       "token-major rows, ROUTE_F32)")
    elif nkern == 2:
        gemm_kernel = (f"gemm_fp8_fused_kernel<{K // 128}, true, true, false> (the route inside the "
                       "grouped FP8 GEMM from routed ids, rows at route ids)")
    elif fused:
        gemm_kernel = (f"gemm_fp8_fused_kernel<{K // 128}, true, false, false> (grouped FP8 GEMM from "
                       "routed ids, rows at route ids)")
    elif K in (512, 1024, 2048) and chunk <= 16:
        gemm_kernel = "gemm_fp8_range_kernel (grouped FP8 GEMM, ROUTE_F32)"
    elif 64 < chunk <= 256 and K <= 8192:
        gemm_kernel = "gemm_fp8_tile_kernel (grouped FP8 GEMM, LDS-staged tiles, ROUTE_F32)"
    else:
        gemm_kernel = "gemm_fp8_kernel (grouped FP8 GEMM, ROUTE_F32)"
    lbytes = layer_algorithmic_bytes(counts, M, E, k, K, N)
    flops = 2.0 * M * k * N * K
    result = {
        "metric": "µs/layer + effective TFLOPS & %HBM roofline, fused MoE M=128 E=256 top-8",
        "value": round(us_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "E": E, "top_k": k, "K": K, "N": N,
                   "softcap": cap, "weight_copies_rotated": copies,
                   "path": ("2 kernels: grouped GEMM routing its tokens itself, combine"
                            if nkern == 2
                            else "3 kernels: route, grouped GEMM from the routed ids, combine"
                            if fused
                            else "4 kernels: route+quantise, layout, gathering grouped GEMM, "
                                 "combine" if gather
                            else "5 kernels: route, layout, QSG, grouped GEMM, combine"),
                   "gemm_task_walk": ("weight slices split evenly over the CUs" if fused
                                      else "contiguous ranges, per-wave pull"
                                      if K in (512, 1024, 2048) and chunk <= 16
                                      else "one task per workgroup, chunks spread over XCDs"
                                      if 64 < chunk <= 256 and K <= 8192
                                      else "static stride" if args.static_grid else "atomic queue"),
                   "launch": "graph" if args.graph else "plain",
                   "chunk_rows": chunk, "sched": args.sched if gather else None},
        "effective_tflops": round(flops / (us_layer * 1e-6) / 1e12, 3),
        "us_p10_p50_p90": [round(float(np.percentile(per, q)), 2) for q in (10, 50, 90)],
        "us_with_event_per_step": round(us_evented, 3),
        "layer_hbm_frac": round(lbytes / (us_layer * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_algorithmic_bytes": lbytes,
        "nonempty_experts": int((counts > 0).sum()),
        "roofline": {"bound": "hbm",
                     "kernel": gemm_kernel,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, gemm_kernel.split(" (")[0]),
                     "algorithmic_bytes_per_launch": gbytes,
                     "avg_launch_us": round(gemm_us, 3)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, k, cap)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
