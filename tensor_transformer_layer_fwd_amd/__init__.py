"""MI355X-native tensor-parallel Transformer MLP / attention-projection shard.

The arithmetic lives in libtpmlp.so (hand-written HIP for gfx950, C ABI in
include/tp_mlp.h); this package is its Python binding and a step driver.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    TP_ACT_GELU_TANH,
    TP_ACT_NONE,
    TP_BF16,
    TP_F32,
    TPError,
    lib,
    tp_attention_bwd,
    tp_attention_fwd,
    tp_bias_act,
    TP_FP8_E4M3,
    TP_FP8_E5M2,
    tp_fp8_column_linear_fwd,
    tp_fp8_linear_bwd_dgrad,
    tp_fp8_linear_bwd_wgrad,
    tp_fp8_linear_bwd_wgrad_workspace_size,
    tp_fp8_quantize,
    tp_fp8_quantize_both,
    tp_fp8_quantize_workspace_size,
    tp_fp8_row_linear_fwd_partial,
    tp_column_linear_fwd,
    tp_gemm_plan,
    tp_last_hip_error,
    tp_linear_bwd_dgrad,
    tp_linear_bwd_dgrad_recompute,
    tp_linear_bwd_wgrad,
    tp_linear_bwd_wgrad_workspace_size,
    tp_reduce_partials,
    tp_row_linear_fwd_partial,
    tp_set_gemm_override,
    tp_status_string,
)
