"""combine_experts_amd: the one-GPU share of a sparse MoE layer on MI355X (gfx950).

Python side of libmoe.so: a ctypes binding with the C ABI's entry-point names (``_lib``) and the
buffer set + call order of one layer forward (``layer``). The kernels live in ``csrc/`` and are
built in-tree by ``python -m combine_experts_amd.build``.
"""
from ._lib import (  # noqa: F401
    MoEError, moe_dims, make_dims, dims_from_config, load_library, LIB_PATH,
    moe_abi_version, moe_status_str, moe_capacity, moe_workspace_size, moe_route, moe_route_ex,
    moe_load_balance, moe_dispatch_layout, moe_dispatch_layout_noalloc, MOE_LAYOUT_NOALLOC_SCRATCH_BYTES,
    moe_dispatch_matrix, moe_recv_layout, moe_gather_rows, moe_scatter_rows,
    moe_padded_layout, moe_permute_padded, moe_expert_ffn_padded_up, moe_expert_ffn_padded_down,
    moe_unpermute_combine_add, moe_layer_forward, moe_layer_args, moe_event_create, moe_event_destroy,
    moe_expert_ffn_up_train, moe_expert_ffn_up_train_gather, moe_group_transpose_gather, moe_transpose_weights, moe_backward_combine, moe_expert_ffn_down_backward,
    moe_expert_ffn_up_backward, moe_expert_ffn_down_backward_w, moe_expert_ffn_up_backward_w, moe_router_backward, moe_backward_dx, moe_wgrad_ld, moe_group_transpose,
    moe_expert_wgrad, MOE_STAGE_ROUTER_BWD, moe_layer_backward, moe_backward_args,
    moe_permute, moe_expert_ffn, moe_expert_ffn_up, moe_expert_ffn_up_gather, moe_expert_ffn_down,
    moe_expert_ffn_down_splitk, MOE_STAGE_FFN_DOWN,
    moe_unpermute_combine,
    MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
    MOE_GATE_SOFTMAX_TOPK, MOE_GATE_SIGMOID_TOPK, MOE_GATE_SOFTMAX_FULL, MOE_ACT_SWIGLU, MOE_ACT_GELU,
    MOE_F32, MOE_BF16, MOE_STAGE_LAYOUT, MOE_STAGE_FFN, MOE_STAGE_ROUTE_STATS,
)
from .layer import (MoELayerBuffers, forward, LayerExecutor, GraphLayer, BackwardBuffers, forward_train,  # noqa: F401
                    backward)
