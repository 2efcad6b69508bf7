"""MI355X-native dropless mixture-of-experts layer hot path.

The compute lives in libmoe_mi355x.so (hand-written HIP kernels for gfx950,
C ABI in include/moe.h); `_lib` binds it with ctypes and `layer.MoELayer`
strings the four calls together on torch-allocated device memory.
"""
from . import _lib  # noqa: F401  (fails loudly when the library is not built)
from ._lib import (  # noqa: F401
    BF16, F32, MXFP4, MXFP8, SIGMOID, SOFTMAX, DEVERR_BAD_ID, DEVERR_NONFINITE, DEVERR_OVERFLOW, DEVERR_WORKSPACE,
    MoEError,
    moe_grouped_mlp, moe_grouped_mlp_workspace_bytes, moe_mx_quantize, moe_permute, moe_permute_workspace_bytes,
    moe_prepare_router, moe_prepare_weights, moe_prepared_weight_bytes, moe_route_topk, moe_route_topk_grouped,
    moe_route_workspace_bytes, moe_router_prepared_bytes, moe_unpermute_combine,
    moe_unpermute_combine_backward, moe_permute_backward, moe_route_backward, moe_prepare_weights_backward,
    moe_grouped_mlp_backward_workspace_bytes, moe_grouped_mlp_backward_data,
    moe_grouped_mlp_backward_weights_workspace_bytes, moe_grouped_mlp_backward_weights,
    moe_mx_columns_grouped_max_blocks, moe_mx_quantize_columns_grouped, moe_query_sizes,
    moe_grouped_mlp_with_act, moe_calib_copy, moe_calib_read, moe_calib_read_out_words, moe_calib_write,
    moe_calib_mfma,
)
from .layer import MoELayer  # noqa: F401
