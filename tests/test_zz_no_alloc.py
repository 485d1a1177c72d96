"""moe_forward_noalloc (the forward on the library's own scratch, for callers that cannot
allocate) against moe_forward on the same inputs: outputs bit for bit, and the oracle's BF16
bar.  Two calls in a row, the second on a smaller layer, so the second runs on what the first
left in the scratch; a layer whose workspace exceeds the scratch is refused with
MOE_E_NOSPC before anything is launched."""
import numpy as np
import pytest
import torch

import oracle as orc
from mixture_experts_layer_softcap_amd import moe, synth

from gpu_util import assert_bf16_close, to_dev, to_np, workload, zeros

pytestmark = pytest.mark.gpu

CAP = synth.SOFTCAP


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    orc.build(force=False)
    assert moe.device_check() == moe.MOE_OK


def run_both(d):
    M, E, k, K, N = d["M"], d["E"], d["k"], d["K"], d["N"]
    args = [to_dev(d["logits"]), to_dev(d["x"]), to_dev(d["w_q"]), to_dev(d["w_s"])]
    ws = zeros(moe.forward_workspace_bytes(M, E, k, K, N), torch.uint8)
    ref_out = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    moe.forward(*args, k, CAP, ref_out, ws)
    out = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    moe.forward_noalloc(*args, k, CAP, out)
    torch.cuda.synchronize()
    return to_np(out, np.uint16), to_np(ref_out, np.uint16)


def test_forward_noalloc_matches_forward_twice():
    # the benchmark layer (M=128, E=256, top-8, K=2048, N=512), then the small one (M=8,
    # E=16, top-2, K=N=256) on the same scratch
    for name in ("fused_fp8_M128_E256_k8_K2048_N512", "fused_fp8_M8_E16_k2_K256_N256"):
        d = workload(name)
        y, y_ref = run_both(d)
        np.testing.assert_array_equal(y, y_ref)
        ref = orc.forward(d["logits"], d["x"], d["w_q"], d["w_s"], d["k"], CAP)["y64"]
        assert_bf16_close(y, ref, f"noalloc {name}")


def test_forward_noalloc_staged_size_then_small():
    # a batch on the tiled gathering path (M=256 at E=256, top-8: 128-row chunks, 8.8 MiB of
    # scratch), then a smaller one on the small-batch path
    for M in (256, 40):
        d = synth.fused_inputs(M, 256, 8, 2048, 512, seed=M)
        d.update(M=M, E=256, k=8, K=2048, N=512)
        d["w_q"], d["w_s"] = orc.quant_weights(d["w"])
        y, y_ref = run_both(d)
        np.testing.assert_array_equal(y, y_ref)


def test_forward_noalloc_refuses_layers_beyond_its_scratch():
    M, E, k, K, N = 1024, 256, 8, 2048, 512          # a 35 MiB workspace
    assert moe.forward_workspace_bytes(M, E, k, K, N) > 16 << 20
    logits = zeros((M, E), torch.float32)
    x = zeros((M, K), torch.int16)
    w_q = zeros((E, N, K), torch.uint8)
    w_s = zeros((E, N // 128, K // 128), torch.float32)
    out = torch.full((M, N), 7, dtype=torch.int16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.forward_noalloc(logits, x, w_q, w_s, k, CAP, out)
    assert ei.value.status == moe.MOE_E_NOSPC
    torch.cuda.synchronize()
    assert (out == 7).all()                          # nothing was launched
