"""MI355X-native W8A8 quantized-verification hot path.

The kernels live in libw8a8.so (HIP for gfx950, C ABI in include/w8a8.h);
this package is its thin torch-tensor binding.  Build the library with
``python -m w8a8_quantized_verification_amd.build``.
"""
from .api import (W8A8Error, Workspace, accept_from_keys, bf16_linear, bf16_tiled_shape,
                  tile_weight_bf16, linear,
                  linear_workspace_bytes, lm_head_argmax, lm_head_argmax_tiled_act, lm_head_verify,
                  quantize_act,
                  quantize_weight, sample_weights, tile_weight, tiled_shape, verify_accept,
                  verify_accept_workspace_bytes, verify_sample, verify_sample_workspace_bytes,
                  w4_shape, quantize_weight_w4, linear_w4, lm_head_argmax_w4,
                  residual_rmsnorm_quant, silu_mul_quant, quantize_act_tiled,
                  linear_tiled_act, linear_tiled_act_workspace_bytes, verify_attention,
                  qk_norm_rope_append, pack_v_cache,
                  hbm_read_probe, HBM_PROBE_SINK_WORDS, lm_head_verify_noalloc,
                  NOALLOC_MAX_ROWS)

__all__ = [
    "W8A8Error", "Workspace", "accept_from_keys", "bf16_linear", "bf16_tiled_shape",
    "tile_weight_bf16", "linear", "linear_workspace_bytes",
    "lm_head_argmax", "lm_head_argmax_tiled_act", "lm_head_verify",
    "quantize_act", "quantize_weight", "tile_weight", "tiled_shape", "verify_accept",
    "verify_accept_workspace_bytes", "verify_sample", "verify_sample_workspace_bytes",
    "sample_weights", "w4_shape", "quantize_weight_w4", "linear_w4", "lm_head_argmax_w4",
    "residual_rmsnorm_quant", "silu_mul_quant", "quantize_act_tiled", "linear_tiled_act",
    "linear_tiled_act_workspace_bytes", "verify_attention", "qk_norm_rope_append", "pack_v_cache", "hbm_read_probe",
    "HBM_PROBE_SINK_WORDS", "lm_head_verify_noalloc", "NOALLOC_MAX_ROWS",
]
