"""Beam MoE sublayer on MI355X: Python binding of libbeam_moe.so.

The binding only marshals arguments (torch tensors -> device pointers, the
current HIP stream) into the C ABI declared in include/beam_moe.h; every step of
the computation runs in the library's HIP kernels. There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from .binding import (  # noqa: F401
    BeamError,
    BeamMoE,
    LIB_PATH,
    beam_dense_forward,
    beam_dense_init,
    beam_grouped_topk,
    beam_moe_destroy,
    beam_moe_forward,
    beam_moe_forward_noalloc,
    beam_moe_set_activation_format,
    beam_moe_inspect,
    ACT_BF16,
    ACT_MXFP4,
    beam_moe_forward_boundary,
    beam_moe_forward_boundary_route,
    beam_moe_init,
    beam_moe_init_mxfp4,
    beam_mxfp4_quantize,
    beam_router_topk,
    beam_sublayer_forward,
    beam_sublayer_norm_residual,
    kernel_names,
    lib,
    profile_enable,
    profile_read,
    profile_reset,
)
