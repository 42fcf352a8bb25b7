"""MI355X (gfx950) MoE token routing: top-k routing, dispatch into per-rank receive buffers, and
weighted combine, as hand-written HIP kernels behind the C ABI of include/moe_route.h.

The binding functions carry the C names; importing them loads libmoe_route.so and fails loudly if
it has not been built.
"""

_EXPORTS = ("moe_route_topk", "moe_dispatch_workspace_bytes", "moe_dispatch_layout",
            "moe_dispatch_pack", "moe_dispatch", "moe_route_dispatch", "moe_combine",
            "moe_status_str", "alloc_dispatch_out", "alloc_workspace", "DispatchBuffers",
            "MoeError", "moe_ep_capacity", "moe_ep_send", "moe_ep_recv", "moe_ep_return",
            "moe_ep_combine", "moe_ep_partial_rows", "moe_ep_reduce", "moe_ep_reduce_workspace",
            "moe_ep_combine_reduced", "moe_check_topk")


def __getattr__(name):
    if name in _EXPORTS:
        from . import _lib
        _lib.load()
        return getattr(_lib, name)
    raise AttributeError(name)
