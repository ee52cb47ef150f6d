"""qlq: an MI355X (gfx950) quantized linear layer -- W8A16, W8A8-static and W8A8-dynamic GEMMs.

The compute lives in libqlq.so (hand-written HIP kernels behind a C ABI,
include/qlq.h); this package is its Python binding.
"""
from .binding import (QTYPES, GRANULARITIES, QlqError, QuantizedKV, QuantizedWeight, calibrate_input_scale,
                      code_dtype, gemm_plan, kv_dequantize, kv_quantize, lib, library_path, linear, linear_workspace_bytes, packed_weight_bytes, qlinear_w8a16, qlinear_w8a16_noalloc,
                      qlinear_w8a8_dynamic, qlinear_w8a8_static, qlinear_w8a8_static_fused,
                      qlinear_w8a8_static_requant,
                      quantize_act_dynamic, quantize_act_static, quantize_weight, scale_is_calibrated, unpack_weight,
                      workspace_bytes)
from .graphs import DEFAULT_BUCKETS, GraphBuckets

__all__ = [
    "DEFAULT_BUCKETS", "GraphBuckets", "QTYPES", "GRANULARITIES", "QlqError", "QuantizedKV", "QuantizedWeight", "calibrate_input_scale", "code_dtype",
    "gemm_plan", "kv_dequantize", "kv_quantize", "linear", "linear_workspace_bytes",
    "lib", "library_path", "packed_weight_bytes", "qlinear_w8a16", "qlinear_w8a16_noalloc", "qlinear_w8a8_dynamic",
    "qlinear_w8a8_static", "qlinear_w8a8_static_fused", "qlinear_w8a8_static_requant", "quantize_act_dynamic",
    "quantize_act_static",
    "quantize_weight", "scale_is_calibrated", "unpack_weight", "workspace_bytes",
]
