"""Grouped Query Experts (GQE) attention layer on MI355X (gfx950).

The layer's steps (projections, router, attention, output projection) run as
hand-written HIP kernels behind a C ABI
(include/gqe.h, built into libgqe.so); this package is the ctypes binding.
"""
from .gqe import (  # noqa: F401
    EXPORTED, GQE_BF16, GQE_ERR_ALIGNMENT, GQE_ERR_HIP, GQE_ERR_INVALID_ARG,
    GQE_ERR_SCRATCH, GQE_ERR_UNSUPPORTED, GQE_ERR_WORKSPACE, GQE_F32, GQE_OK, GQE_SLOTS_FULL, GQE_SLOTS_HARD,
    GQE_SLOTS_WEIGHTED, GQE_WEIGHTS_PROB, GQE_WEIGHTS_RENORM, GQEError, LIB_PATH, decode,
    decode_paged, decode_workspace, gqe_attn_decode, gqe_attn_decode_noalloc, gqe_attn_decode_paged, gqe_attn_prefill, gqe_attn_prefill_bwd,
    gqe_attn_prefill_bwd_workspace_bytes, gqe_attn_prefill_train, gqe_decode_scratch_bytes, gqe_decode_workspace_bytes, gqe_dims,
    gqe_out_proj, gqe_out_proj_bwd, gqe_out_proj_bwd_workspace_bytes, gqe_out_proj_variant, gqe_qkv_proj, gqe_qkv_proj_decode, gqe_route, gqe_route_bwd, gqe_route_bwd_workspace_bytes, gqe_route_workspace_bytes,
    load_library, out_proj, out_proj_bwd, prefill, prefill_bwd, prefill_train, qkv_proj, route, route_bwd, status_string,
)
