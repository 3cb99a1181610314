"""MI355X (gfx950) MoE routing front-end: split-K router GEMV with in-launch
fixup, softmax top-k gate, token -> expert sort and MXFP8 (or MXFP4) quantisation, behind
the C ABI of include/rgt.h.

The binding (``router_gemv_top_amd._binding``) is imported lazily so that the
seeded input generators (``router_gemv_top_amd.inputs``) can be used without
loading the HIP library.
"""

_API = (
    "rmsnorm", "router_logits", "router_partial_slices", "router_shared_swiglu", "topk_gate", "topk_gate_partials", "moe_sort_quant", "route_sort_quant", "moe_sort_quant_mxfp4",
    "route_sort_quant_mxfp4", "route_sort_quant_noalloc", "rmsnorm_route_sort_quant", "moe_stage1_swiglu", "Workspace",
    "workspace_bytes", "sort_capacity", "router_supported", "reset_workspace", "check_workspace",
    "status_string", "last_launch_count", "alloc_sort_outputs", "RgtError", "RgtUnsupported", "lib",
    "exported_symbols", "version", "diag_read", "diag_copy", "reload_env",
)


def __getattr__(name):
    if name in _API:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
