"""GPU parity of the router projection (moe_router_logits) against the oracle.

fp32 logits: bf16 products are exact in fp32 and the matrix core accumulates in fp32, so each
logit carries at most a few fp32 roundings of its running sum: the bound per element is
H * 2^-24 * sum_h |x_h w_h| (the textbook bound for H additions), and in aggregate the
relative Frobenius error stays near 2^-24 * sqrt(H).  The route then decides integers (the
top-k) from fp32 logits, so the ids are compared with the oracle's route applied to the
device's own logits: both sides take that decision on the same numbers."""
import numpy as np
import pytest
import torch

import oracle as orc
from mixture_experts_layer_softcap_amd import moe, synth

from gpu_util import (WEIGHT_RTOL, assert_bf16_close, oracle_rows_parallel, to_dev, to_np,
                      zeros)

pytestmark = pytest.mark.gpu

CAP = synth.SOFTCAP


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    orc.build(force=False)
    assert moe.device_check() == moe.MOE_OK


def oracle_logits(x, wg):
    return oracle_rows_parallel(lambda xs, wg_, rows: orc.router_logits(xs[rows], wg_),
                                np.arange(x.shape[0], dtype=np.int32), x, wg)


def gpu_logits(x, wg, reps=1):
    M, E = x.shape[0], wg.shape[0]
    outs = []
    xd, wd = to_dev(x), to_dev(wg)
    for _ in range(reps):
        out = torch.full((M, E), float("nan"), dtype=torch.float32, device="cuda")
        moe.router_logits(xd, wd, out)
        torch.cuda.synchronize()
        outs.append(to_np(out))
    return outs


def check_logits(y, ref64, x, wg, what):
    xa = np.abs(synth.bf16_to_f32(x).astype(np.float64))
    wa = np.abs(synth.bf16_to_f32(wg).astype(np.float64))
    H = x.shape[1]
    bound = H * 2.0 ** -24 * (xa @ wa.T) + 1e-30
    d = np.abs(y.astype(np.float64) - ref64)
    assert np.isfinite(y).all(), what
    assert (d <= bound).all(), f"{what}: max |d|/bound {float((d / bound).max()):.3f}"
    fro = float(np.linalg.norm(d) / np.linalg.norm(ref64))
    assert fro <= 2.0 ** -24 * np.sqrt(H) * 4, f"{what}: relative Frobenius {fro:.3e}"


@pytest.mark.parametrize("M,H,E", [
    (128, 2048, 256),     # the M=128, E=256, K=2048 layer's gate
    (4096, 2048, 256),    # the same layer at M=4096
    (8192, 4096, 8),      # Mixtral-like gate: 8 experts, hidden 4096
    (37, 192, 10),        # ragged tokens and experts, 3 k steps
    (1, 64, 1),           # one token, one expert, one k step
    (300, 320, 1000),     # many experts, E not a multiple of 16 or 64
    # tile shapes the launcher picks on a 256-CU chip (16*TB tokens x 16*EB experts):
    (2048, 256, 256),     # 32 x 64 tiles, expert blocks spread over the 8 XCDs
    (4100, 128, 200),     # 64 x 64 tiles, ragged tokens and experts, 4 expert blocks
    (4096, 128, 512),     # 64 x 64 tiles, 8 expert blocks (one per XCD)
    (16384, 128, 8),      # 64 x 16 tiles, 8 experts padded to 16 gate rows
])
def test_router_logits_match_oracle(M, H, E):
    d = synth.router_inputs(M, H, E, seed=M + E)
    y, y2 = gpu_logits(d["x"], d["w_gate"], reps=2)
    np.testing.assert_array_equal(y, y2)                  # fixed summation order
    _, ref64 = oracle_logits(d["x"], d["w_gate"])
    check_logits(y, ref64, d["x"], d["w_gate"], f"M={M} H={H} E={E}")


def test_router_then_route_then_forward():
    # the M=128, E=256, top-8 layer from hidden states: router projection -> moe_forward; ids
    # against the oracle's route of the device's logits, the output against the oracle's
    # forward from those logits
    M, H, E, k, N = 128, 2048, 256, 8, 512
    d = synth.router_inputs(M, H, E, seed=9)
    w = synth.fused_inputs(M, E, k, H, N, seed=9)["w"]
    w_q, w_s = orc.quant_weights(w)
    logits = gpu_logits(d["x"], d["w_gate"])[0]
    ws = zeros(moe.forward_workspace_bytes(M, E, k, H, N), torch.uint8)
    out = zeros((M, N), torch.int16)
    moe.forward(to_dev(logits), to_dev(d["x"]), to_dev(w_q), to_dev(w_s), k, CAP, out, ws)
    torch.cuda.synchronize()
    ids = to_np(ws[moe.forward_workspace_offset(M, E, k, H, N, 0):][:4 * M * k]).view(np.int32)
    r_ids, _ = orc.route(logits, k, CAP)
    np.testing.assert_array_equal(ids.reshape(M, k), r_ids)
    ref = orc.forward(logits, d["x"], w_q, w_s, k, CAP)["y64"]
    assert_bf16_close(to_np(out, np.uint16), ref, "router -> forward")
