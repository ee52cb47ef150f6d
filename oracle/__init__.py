"""Oracle: a plain, slow, CPU-only statement of what the quantized linear layer computes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, tables or helpers); the only thing both
sides take from a common place are the seeded inputs in ``synth``.

Form: NumPy on the host.  Number formats (bf16, OCP e4m3fn) are decoded and
encoded from their bit-level definitions with integer operations; every
contraction is a float64 (or exact integer) matmul, so the oracle's only
roundings are the ones the method itself prescribes.

Sources ("the pages"):
* "Nano-vLLM-MoE" README (GitHub), sections "FP8 W8A16 weight-only
  quantization" (Setup: Triton FP8->BF16 dequant GEMM with a bf16 x bf16 dot
  accumulating in fp32) and "FP8 W8A8 static quantization" (offline-calibrated
  activation scales; scaled-mm and CUTLASS backends with a custom epilogue;
  Analysis: the W8A8 kernel agrees in value with the BF16-dequant reference).
* "Nano-vLLM-MOE" README mirror, section "INT8 量化支持" (INT8 quantization
  support): scheme table (int8_w8a16 / int8_w8a8_static) and key-design list
  (W8A16 dequantizes int8 weights to BF16 for a standard matmul; W8A8 static
  quantizes activations at run time with one fixed, offline-calibrated scalar
  per layer and runs an INT8 GEMM with int32 accumulation; the per-token
  absmax alternative it contrasts with is the dynamic scheme here).
* "tiny-vLLM" README, section "Quantization Results" / "Quality Check":
  reconstruction error of the quantized weights (relative L2, cosine).
* "Nano-vLLM-MoE" README, section "KV cache compression": the mixed K-int8
  (group 32, fp16 scales) / V-FP8 per-token codec (``kvcache``).

Parity status: every public function here is pinned by ``tests/test_oracle_*.py``
(closed forms, exhaustive codec checks against torch's casts, exact rational
brute force, integer exact cases).  The FP8 W8A8 accumulation order of a GPU
is not fixed by the pages; the oracle gives the exact sum and the GPU is held
to a tolerance there.
"""
from .codecs import (bf16_bits_to_f32, f32_to_bf16_bits, bf16_round,
                     e4m3fn_decode, e4m3fn_encode_sat, E4M3FN_MAX, INT8_QMAX)
from .qlinear import (qmax_of, weight_scale, quantize_weight, dequantize_weight_bf16,
                      calibrate_input_scale, quantize_act_static, quantize_act_dynamic,
                      qlinear_w8a16, w8a8_accumulate, w8a8_epilogue, qlinear_w8a8_static,
                      w8a8_epilogue_per_token, qlinear_w8a8_dynamic, linear, reconstruction_error)
from .kvcache import (K_GROUP, fp16_encode, fp16_decode, kv_quantize, kv_dequantize,
                      kv_bytes_per_token_head)

__all__ = [
    "bf16_bits_to_f32", "f32_to_bf16_bits", "bf16_round", "e4m3fn_decode",
    "e4m3fn_encode_sat", "E4M3FN_MAX", "INT8_QMAX", "qmax_of", "weight_scale",
    "quantize_weight", "dequantize_weight_bf16", "calibrate_input_scale",
    "quantize_act_static", "quantize_act_dynamic", "qlinear_w8a16", "w8a8_accumulate",
    "w8a8_epilogue", "qlinear_w8a8_static", "w8a8_epilogue_per_token", "qlinear_w8a8_dynamic",
    "linear", "reconstruction_error", "K_GROUP", "fp16_encode", "fp16_decode", "kv_quantize", "kv_dequantize",
    "kv_bytes_per_token_head",
]
