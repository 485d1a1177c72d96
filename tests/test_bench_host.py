"""bench.py on the host, with no GPU: it refuses more than one GPU before touching a device,
and the algorithmic byte counts behind its roofline figure equal counts made by hand from the
operand shapes (the numerator of `roofline.achieved`)."""
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench_module():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert not r.stdout.strip()                 # no JSON line


# the M=128, E=256, top-8, K=2048, N=512 layer with 254 experts chosen (the seeded routing of
# its bench input leaves two experts unused)
M, E, k, K, N = 128, 256, 8, 2048, 512
USED = 254
PER_EXPERT = N * K + (N // 128) * (K // 128) * 4      # E4M3 codes + one fp32 per 128x128 block


def counts_with(used):
    c = np.zeros(E, np.int64)
    c[:used] = 1
    c[0] += M * k - used
    return c


def test_route_fused_gemm_bytes_by_hand():
    b = bench_module()
    hand = (USED * PER_EXPERT          # 254 x (1 MiB codes + 256 B scales)
            + M * K * 2                 # bf16 token rows
            + M * E * 4                 # fp32 logits
            + M * k * N * 4             # fp32 routed output rows
            + M * k * 8)                # ids and weights written
    assert hand == 269_164_032
    assert b.gemm_algorithmic_bytes(counts_with(USED), M, k, K, N, fused=True, E=E) == hand


def test_committed_bench_line_uses_the_same_count():
    # the committed bench line of this workload reports the same bytes per launch
    with open(os.path.join(ROOT, "profiles", "bench_fused_fp8_M128_E256_k8_K2048_N512.json")) as f:
        line = json.load(f)["line"]
    assert line["roofline"]["algorithmic_bytes_per_launch"] == 269_164_032
    assert line["roofline"]["unit"] == "GB/s" and line["roofline"]["peak"] == 8000.0
    frac = line["roofline"]["achieved"] / line["roofline"]["peak"]
    assert abs(frac - line["roofline"]["frac"]) < 1e-3


def test_staged_and_gather_gemm_bytes_by_hand():
    b = bench_module()
    m, kk, kd, n = 5, 2, 256, 128               # 10 routes, two k-blocks, one 128-row block
    c = np.array([4, 0, 6])                     # two experts used
    w = 2 * (n * kd + 1 * 2 * 4)
    out = m * kk * n * 4
    staged = m * kk * kd + 2 * m * kk * 4 + m * kk * 4      # routed codes, scales, sorted ids
    gather = m * kd + 2 * m * 4 + m * kk * 4                # token codes, scales, sorted ids
    fused = m * kd * 2 + m * kk * 4                         # bf16 rows, routed ids
    assert b.gemm_algorithmic_bytes(c, m, kk, kd, n) == w + staged + out
    assert b.gemm_algorithmic_bytes(c, m, kk, kd, n, gather=True) == w + gather + out
    assert b.gemm_algorithmic_bytes(c, m, kk, kd, n, fused=True) == w + fused + out


def test_layer_bytes_by_hand():
    b = bench_module()
    hand = USED * PER_EXPERT + M * E * 4 + M * K * 2 + M * N * 2   # + logits, x, bf16 out
    assert b.layer_algorithmic_bytes(counts_with(USED), M, E, k, K, N) == hand
