"""MI355X-native Q4_0 fused-dequantization matmul and routed-expert MoE decode.

Entry points (HIP kernels behind the C ABI in ``include/q4moe.h``):
``q4_0_gemv`` (and ``q4_0_gemv_noalloc``, the same without any allocation), ``q8_0_gemv`` (Q8_0 weights), ``q4_0_gemm``, ``moe_q4_0_decode``, ``moe_q4_0_prefill`` (experts on the
matrix cores), the on-device router
``moe_router_topk``, the whole layer ``moe_q4_0_layer`` (router, routed and
shared experts) and their workspace-size helpers. They are loaded from ``libq4moe.so`` on first use; there is no CPU
fallback. ``moe_experts_amd.datagen`` (seeded synthetic inputs) does not need
the library.
"""
_EXPORTS = ("q4_0_gemv", "q8_0_gemv", "q8_0_gemv_workspace_bytes", "q4_0_gemm", "moe_q4_0_decode", "moe_q4_0_prefill",
            "moe_q4_0_prefill_workspace_bytes", "moe_router_topk", "moe_q4_0_layer",
            "q4_0_gemv_workspace_bytes", "moe_q4_0_workspace_bytes",
            "moe_router_workspace_bytes", "moe_q4_0_layer_workspace_bytes", "q4_strerror",
            "moe_q4_0_route_layout", "moe_q4_0_prefill_route_layout", "q4_0_gemv_noalloc", "GEMV_NOALLOC_MAX_WS",
            "Q4Error")


def __getattr__(name):
    if name in _EXPORTS:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)


__all__ = list(_EXPORTS)
