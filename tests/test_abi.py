"""The C ABI on the host: libmoe.so loads, exports every entry point include/moe.h
declares, and rejects bad arguments with status codes before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_softcap_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from mixture_experts_layer_softcap_amd import build

        build.build()
    return moe.lib()


def test_every_declared_entry_point_is_exported(L):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(moe.SIGNATURES), "binding and header disagree"


def test_status_strings(L):
    assert L.moe_status_string(0) == b"MOE_OK"
    for s in (-1, -2, -3, -4):
        assert L.moe_status_string(s).startswith(b"MOE_E_")


def test_max_tasks_bound(L):
    # (floor(M*k/chunk) + min(E, M*k)) * n_blocks
    assert L.moe_max_tasks(128, 8, 256, 4, 16) == (1024 // 16 + 256) * 4
    assert L.moe_max_tasks(8, 2, 16, 2, 64) == (0 + 16) * 2
    assert L.moe_max_tasks(1, 1, 256, 4, 16) == (0 + 1) * 4
    assert L.moe_max_tasks(0, 8, 256, 4, 16) == 0
    assert L.moe_max_tasks(128, 8, 256, 4, 0) == -1
    assert L.moe_max_tasks(128, 9, 8, 4, 16) == -1      # k > E
    assert L.moe_max_tasks(128, 65, 256, 4, 16) == -1   # k > 64
    assert L.moe_max_tasks(128, 8, 2048, 4, 16) == -1   # E > 1024


def test_workspace_queries(L):
    b = L.moe_forward_workspace_bytes(128, 256, 8, 2048, 512)
    R = 128 * 8
    assert b >= R * 2048 + R * 512 * 4 + 16 * 4 * R
    offs = [L.moe_forward_workspace_offset(128, 256, 8, 2048, 512, i) for i in range(15)]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs) and offs[-1] < b
    assert L.moe_forward_workspace_bytes(128, 256, 8, 2000, 512) == 0   # K % 128
    assert L.moe_forward_workspace_offset(128, 256, 8, 2048, 512, 15) == -1
    fo = [L.moe_ffn_workspace_offset(64, 8, 2, 512, 256, i) for i in range(13)]
    assert fo == sorted(fo) and all(o % 256 == 0 for o in fo)
    assert fo[-1] < L.moe_ffn_workspace_bytes(64, 8, 2, 512, 256)
    assert L.moe_ffn_workspace_offset(64, 8, 2, 512, 256, 13) == -1
    mo = [L.moe_mlp_workspace_offset(128, 256, 8, 2048, 512, i) for i in range(16)]
    mb = L.moe_mlp_workspace_bytes(128, 256, 8, 2048, 512)
    assert mo == sorted(mo) and all(o % 256 == 0 for o in mo) and mo[-1] < mb
    # x codes + gate/up rows + act codes + down rows at least
    assert mb >= R * 2048 + R * 1024 * 4 + R * 512 + R * 2048 * 4
    assert mo[15] - mo[12] >= R * 1024 * 4 + R * 512 + (512 // 128) * R * 4
    assert L.moe_mlp_workspace_offset(128, 256, 8, 2048, 512, 16) == -1
    assert L.moe_mlp_workspace_bytes(128, 256, 8, 2048, 500) == 0                 # I % 128
    assert L.moe_mlp_workspace_bytes(128, 256, 8, 2000, 512) == 0                 # H % 128
    assert L.moe_gemm_n_tile(0) == 128 and L.moe_gemm_n_tile(1) == 256
    assert L.moe_gemm_n_tile(5) == -1


NULL = None
S = ctypes.c_void_p(0)
P = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def test_invalid_arguments_are_rejected_on_the_host(L):
    INVAL, NOSPC = moe.MOE_E_INVAL, moe.MOE_E_NOSPC
    assert L.moe_route(P, 4, 0, 1, 30.0, P, P, S) == INVAL            # E = 0
    assert L.moe_route(P, 4, 8, 9, 30.0, P, P, S) == INVAL            # k > E
    assert L.moe_route(NULL, 4, 8, 2, 30.0, P, P, S) == INVAL         # null logits
    assert L.moe_route(P, 4, 8, 2, float("nan"), P, P, S) == INVAL    # NaN cap
    assert L.moe_route(P, -1, 8, 2, 30.0, P, P, S) == INVAL
    need = L.moe_max_tasks(16, 2, 8, 2, 4)
    bl = L.moe_build_layout
    assert bl(P, 16, 2, 8, 2, 4, P, P, P, P, need - 1, P, P, NULL, NULL, S) == NOSPC
    assert bl(P, 16, 2, 8, 2, 2000, P, P, P, P, 10 ** 6, P, P, NULL, NULL, S) == INVAL
    assert bl(P, 16, 2, 8, 2, 4, NULL, P, P, P, need, P, P, NULL, NULL, S) == INVAL
    assert bl(P, 16, 2, 8, 2, 4, P, P, P, P, need, P, P, NULL, P, S) == INVAL  # slots alone
    rq = L.moe_route_quantize
    assert rq(P, P, 4, 8, 2, 200, 30.0, P, P, P, P, S) == INVAL      # K % 128
    assert rq(P, NULL, 4, 8, 2, 256, 30.0, P, P, P, P, S) == INVAL   # null x
    assert rq(P, P, 4, 8, 2, 256, 30.0, P, P, NULL, P, S) == INVAL   # null x_q
    assert rq(P, P, 4, 8, 9, 256, 30.0, P, P, P, P, S) == INVAL      # k > E
    gga = L.moe_grouped_gemm_gather
    assert gga(P, P, 4, 2, 256, P, P, 8, 256, P, P, 8, 64, P, P, P, -1, S) == INVAL     # chunk <= 64
    assert gga(P, P, 4, 2, 256, P, P, 8, 256, P, P, 8, 257, P, P, P, -1, S) == INVAL    # chunk > 256
    assert gga(P, P, 4, 2, 8320, P, P, 8, 256, P, P, 8, 128, P, P, P, -1, S) == INVAL   # K > 8192
    assert gga(P, P, 4, 2, 256, P, P, 8, 200, P, P, 8, 128, P, P, P, -1, S) == INVAL    # N % 128
    assert gga(P, P, 4, 2, 256, P, P, 8, 256, P, P, 8, 128, NULL, P, P, -1, S) == INVAL # sorted ids
    assert gga(P, P, 4, 2, 256, P, P, 8, 256, P, P, 8, 128, P, P, NULL, 2, S) == INVAL  # queue
    assert gga(P, P, 4, 2, 256, P, P, 8, 256, P, P, 8, 256, P, P, P, 3, S) == INVAL  # 256 rows
    assert gga(P, P, 4, 2, 256, P, P, 8, 256, P, P, 8, 128, P, P, P, 4, S) == INVAL  # sched
    assert L.moe_quant_sort_gather(P, 4, 200, P, 2, 8, P, P, P, P, P, S) == INVAL  # K % 128
    assert L.moe_quant_sort_gather(P, 4, 256, NULL, 2, 8, P, P, P, P, P, S) == INVAL
    assert L.moe_quantize_weights(P, 2, 100, 256, P, P, S) == INVAL
    assert L.moe_quantize_weights(NULL, 2, 128, 256, P, P, S) == INVAL
    gg = L.moe_grouped_gemm
    assert gg(7, P, P, 4, 256, P, P, 2, 256, P, P, 8, 16, P, 0, P, P, -1, S) == INVAL  # mode
    assert gg(0, P, P, 4, 256, P, P, 2, 256, P, P, 8, 257, P, 0, P, P, -1, S) == INVAL  # chunk
    assert gg(0, P, P, 4, 8320, P, P, 2, 256, P, P, 8, 65, P, 0, P, P, -1, S) == INVAL  # tiled K
    assert gg(0, P, P, 4, 256, P, P, 2, 256, P, P, 8, 16, P, 9, P, P, -1, S) == INVAL  # epilogue
    assert gg(0, P, P, 4, 256, P, P, 2, 256, P, P, 8, 16, P, 2, NULL, P, -1, S) == INVAL  # route ids
    assert gg(0, P, P, 4, 250, P, P, 2, 256, P, P, 8, 16, P, 0, P, P, -1, S) == INVAL  # K % 128
    assert L.moe_scatter(P, P, P, P, 4, 2, 8, 6, P, S) == INVAL       # N % 4
    ws = L.moe_forward_workspace_bytes(8, 16, 2, 256, 256)
    f = L.moe_forward_ex
    assert f(P, P, P, P, 8, 16, 2, 256, 256, 30.0, P, P, ws - 1, 0, 0, S) == NOSPC
    assert f(P, P, P, P, 8, 16, 2, 256, 256, 30.0, P, P, ws, 0, 64, S) == INVAL    # flags
    assert f(P, P, P, P, 8, 16, 2, 256, 256, 30.0, P, P, ws, 0, 5 << 3, S) == INVAL  # sched
    assert f(P, P, P, P, 8, 16, 2, 256, 256, 30.0, P, P, ws, 0, 512, S) == INVAL    # bit 9
    rg = L.moe_route_grouped_gemm
    assert rg(P, P, 128, 256, 8, 2048, 30.0, P, P, 512, P, P, NULL, P, P, S) == INVAL  # words
    assert rg(P, P, 128, 256, 8, 2048, 30.0, P, P, 512, P, P, P, NULL, P, S) == INVAL  # status
    assert rg(P, P, 128, 256, 8, 2048, float("nan"), P, P, 512, P, P, P, P, P, S) == INVAL
    assert rg(P, P, 128, 256, 8, 2048, 30.0, P, P, 500, P, P, P, P, P, S) == INVAL  # N % 128
    assert rg(P, P, 128, 8, 9, 2048, 30.0, P, P, 512, P, P, P, P, P, S) == INVAL    # k > E
    assert f(P, P, P, P, 8, 16, 2, 256, 256, 30.0, P, P, ws, 256, moe.MOE_FWD_SCHED(2),
             S) == INVAL                                                       # 256 rows
    assert f(P, P, P, P, 8, 16, 2, 256, 256, 30.0, P, P, ws, 257, 0, S) == INVAL   # chunk
    assert f(P, P, NULL, P, 8, 16, 2, 256, 256, 30.0, P, P, ws, 0, 0, S) == INVAL
    assert L.moe_forward(P, P, P, P, 0, 16, 2, 256, 256, 30.0, P, P, ws, S) == INVAL
    assert L.moe_sort_gather_bf16(P, 4, 100, P, 2, 8, P, P, P, P, S) == INVAL   # K % 8
    assert gg(1, P, P, 4, 96, P, P, 2, 256, P, P, 8, 256, P, 1, P, P, -1, S) == INVAL  # K % 64
    assert gg(1, P, P, 4, 128, P, P, 2, 384, P, P, 8, 256, P, 1, P, P, -1, S) == INVAL  # N % 256
    assert gg(1, P, P, 4, 128, P, P, 2, 256, P, P, 8, 257, P, 1, P, P, -1, S) == INVAL  # chunk
    assert gg(1, P, P, 4, 128, P, P, 2, 256, P, P, 8, 256, P, 2, P, P, -1, S) == INVAL  # ROUTE_F32
    fw = L.moe_ffn_workspace_bytes(16, 8, 2, 512, 256)
    assert fw > 0 and L.moe_ffn_workspace_bytes(16, 8, 2, 500, 256) == 0         # H % 256
    assert L.moe_ffn_workspace_bytes(16, 8, 2, 512, 200) == 0                    # F % 128
    ff = L.moe_ffn_forward
    assert ff(P, P, P, P, 16, 8, 2, 512, 256, 30.0, P, P, fw - 1, 0, 0, S) == NOSPC
    assert ff(P, P, P, P, 16, 8, 2, 512, 256, 30.0, P, P, fw, 300, 0, S) == INVAL   # chunk
    assert ff(P, NULL, P, P, 16, 8, 2, 512, 256, 30.0, P, P, fw, 0, 0, S) == INVAL
    assert ff(P, P, P, P, 16, 8, 2, 512, 256, 30.0, P, P, fw, 0, 1, S) == INVAL    # flags
    assert gg(1, P, P, 4, 128, P, P, 2, 256, P, P, 8, 256, NULL, 1, P, P, 2, S) == INVAL  # queue
    assert gg(0, P, P, 4, 256, P, P, 2, 256, P, P, 8, 16, P, 0, P, P, 0, S) == INVAL  # FP8 sched
    sq = L.moe_swiglu_quant
    assert sq(P, 4, 200, P, P, S) == INVAL                                       # I % 128
    assert sq(P, -1, 256, P, P, S) == INVAL
    assert sq(NULL, 4, 256, P, P, S) == INVAL
    assert L.moe_mlp_forward_kernels(16, 8, 2, 256, 100, 0) == INVAL            # I % 128
    assert L.moe_mlp_forward_kernels(16, 8, 2, 256, 128, 300) == INVAL           # chunk
    mw = L.moe_mlp_workspace_bytes(16, 8, 2, 256, 128)
    mf = L.moe_mlp_forward
    assert mf(P, P, P, P, P, P, 16, 8, 2, 256, 128, 30.0, P, P, mw - 1, 0, S) == NOSPC
    assert mf(P, P, P, P, P, P, 16, 8, 2, 256, 128, 30.0, P, P, mw, 300, S) == INVAL  # chunk
    assert mf(P, P, P, P, P, P, 16, 8, 2, 256, 100, 30.0, P, P, mw, 0, S) == INVAL    # I % 128
    assert mf(P, P, P, NULL, P, P, 16, 8, 2, 256, 128, 30.0, P, P, mw, 0, S) == INVAL
    assert mf(P, P, P, P, P, P, 16, 8, 9, 256, 128, 30.0, P, P, mw, 0, S) == INVAL    # k > E
    assert mf(P, P, P, P, P, P, 16, 8, 2, 256, 128, float("nan"), P, P, mw, 0, S) == INVAL


def test_no_gpu_gives_a_device_status():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert moe.lib().moe_device_check() == moe.MOE_E_DEVICE


def test_forward_noalloc_rejects_on_the_host(L):
    # the no-allocation forward: bad arguments, and layers whose workspace exceeds its 16 MiB
    # scratch, are refused before any HIP call (so also without a GPU)
    INVAL, NOSPC = moe.MOE_E_INVAL, moe.MOE_E_NOSPC
    na = L.moe_forward_noalloc
    assert L.moe_forward_workspace_bytes(1024, 256, 8, 2048, 512) > 16 << 20
    assert na(P, P, P, P, 1024, 256, 8, 2048, 512, 30.0, P, S) == NOSPC
    assert na(P, P, P, P, 8, 16, 2, 250, 256, 30.0, P, S) == INVAL       # K % 128
    assert na(P, P, NULL, P, 8, 16, 2, 256, 256, 30.0, P, S) == INVAL    # null weights
    assert na(P, P, P, P, 8, 16, 2, 256, 256, 30.0, NULL, S) == INVAL    # null out
    assert na(P, P, P, P, 8, 16, 2, 256, 256, float("nan"), P, S) == INVAL


def test_router_logits_rejects_on_the_host(L):
    INVAL = moe.MOE_E_INVAL
    rl = L.moe_router_logits
    assert rl(P, 8, 100, P, 4, P, S) == INVAL          # H % 64
    assert rl(P, 8, 128, P, 0, P, S) == INVAL          # E = 0
    assert rl(P, 8, 128, P, 1025, P, S) == INVAL       # E > 1024
    assert rl(NULL, 8, 128, P, 4, P, S) == INVAL       # null x
    assert rl(P, 8, 128, P, 4, NULL, S) == INVAL       # null logits
    assert rl(P, -1, 128, P, 4, P, S) == INVAL
    assert rl(P, 2 ** 30, 64, P, 1024, P, S) == INVAL  # 2^26 x 64 workgroups
