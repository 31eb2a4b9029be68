"""Single-GPU MoE layer forward on MI355X: Python binding of libmoe.

The binding only marshals arguments: every step of the layer runs in the HIP
kernels of ``libmoe.so`` (C ABI declared in ``include/moe.h``).  PyTorch
supplies device memory and the stream.  There is no fallback: if the
library is missing, importing this package raises.

Function names match the C ABI: ``moe_route_topk``, ``moe_permute``,
``moe_grouped_ffn``, ``moe_unpermute_combine``, ``moe_layer_forward``,
``moe_workspace_size``, ``moe_num_segments``, ``moe_status_string``.
"""
from __future__ import annotations

import ctypes
import os

from ._lib import (  # noqa: F401
    LIB_PATH, MOE_DT_BF16, MOE_DT_F32, MOE_SCORE_SIGMOID, MOE_SCORE_SOFTMAX, MOE_SPLIT_BOUNDED,
    MOE_SPLIT_PARITY, MoEConfig,
    MoEError, lib, make_config, moe_grouped_ffn, moe_layer_forward, moe_num_segments,
    moe_permute, moe_route_topk, moe_status_string, moe_unpermute_combine,
    moe_workspace_size, moe_quantize_fp8, moe_grouped_ffn_fp8w, moe_layer_forward_fp8w,
    moe_layer_plan_offsets, moe_num_rows, moe_quantize_act_fp8, moe_grouped_ffn_w8a8,
    moe_layer_forward_w8a8, moe_layer_forward_static, MOE_STATIC_WORKSPACE_BYTES,
    EXPORTED_SYMBOLS,
)
