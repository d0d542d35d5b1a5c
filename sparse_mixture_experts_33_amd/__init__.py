"""MI355X (gfx950) sparse mixture-of-experts layer: HIP kernels behind a C ABI (include/moe.h).

The layer is Mixtral 8x7B's: y = sum over the top-2 of softmax(TopK(x . W_g)) times
SwiGLU experts (arXiv 2401.04088), and the decoder block around it (grouped-query attention,
norms, residuals). ``moe`` is the ctypes binding of ``libmoe.so`` (argument marshalling only;
every step runs in the library's kernels).
"""
from .moe import (  # noqa: F401
    MOE_BF16, MOE_BLOCK_NUM_STAGES, MOE_F32, MOE_LAYOUT_PACKED, MOE_LAYOUT_ROWMAJOR, MOE_NOALLOC_SCRATCH_BYTES,
    MOE_NUM_STAGES, MOE_STAGE_ATTENTION, MOE_STAGE_COMBINE,
    MOE_STAGE_EXPERT_DOWN, MOE_STAGE_EXPERT_UP, MOE_STAGE_PERMUTE, MOE_STAGE_ROUTE, MOE_W_DOWN, MOE_W_UP, AttnDims,
    Dims, MoeError, lib, moe_abi_version, moe_attention, moe_backward, moe_backward_workspace_bytes,
    moe_block_forward, moe_block_workspace_bytes, moe_combine, moe_expert_ffn, moe_forward, moe_forward_noalloc,
    moe_last_error, moe_pack_weights, moe_permute, moe_rmsnorm, moe_route, moe_status_string, moe_workspace_bytes,
    stage_event_array,
)
