"""MI355X-native fused MoE forward: softcapped top-k routing, blockwise FP8 quantisation
with sort/gather, block-scaled FP8 grouped GEMM and routing-weighted combine, as hand-written
HIP kernels for gfx950 behind the C ABI declared in include/moe.h.

``mixture_experts_layer_softcap_amd.moe`` is the thin ctypes binding of that library.
"""
