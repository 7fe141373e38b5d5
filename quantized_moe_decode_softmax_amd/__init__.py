"""MI355X (gfx950) quantized MoE decode: C-ABI library libmoe.so + Python binding.

The hot path (router GEMV, renormalised softmax top-k, group-affine dequant
gate/up/down GEMVs with SwiGLU, sigmoid-gated shared expert, weighted combine,
residual, layer stacking) runs entirely in the HIP kernels of libmoe.so. This
package only marshals arguments to it; PyTorch, where used by callers, only
provides device memory and streams.
"""

from ._lib import (  # noqa: F401
    MOE_ERR_ALIGNMENT,
    MOE_ERR_HIP,
    MOE_ERR_INVALID_ARG,
    MOE_ERR_TIMEOUT,
    MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE,
    MOE_OK,
    MOE_PATH_DEFAULT,
    MOE_PATH_NO_MFMA,
    MOE_PATH_PER_LAYER,
    MoeError,
    header_functions,
    lib,
    make_shape,
    moe_decode_layer,
    moe_decode_stack,
    moe_decode_stack_static,
    moe_expert_bytes,
    moe_attn_shape_t,
    moe_gdn_shape_t,
    moe_gdn_step,
    moe_gemv,
    moe_gemv_mat_t,
    moe_generate_layer,
    moe_generate_matrix,
    moe_gqa_decode,
    moe_gqa_workspace_bytes,
    moe_generate_rows,
    moe_last_error,
    moe_layer_bytes,
    moe_layer_layout,
    moe_matrix_bytes,
    moe_pack_matrix,
    moe_shape_t,
    moe_stack_decode,
    moe_stack_init,
    moe_stack_status,
    moe_stack_t,
    moe_unpack_matrix,
    moe_validate,
    moe_validate_shape,
    moe_version,
    moe_workspace_bytes,
)
from .workloads import WORKLOADS, Workload  # noqa: F401
