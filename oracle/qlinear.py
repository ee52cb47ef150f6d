"""Oracle quantized linear layer: weight quantizer, static and dynamic (per-token)
activation quantizers, W8A16, W8A8-static and W8A8-dynamic GEMMs with their
epilogues.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Conventions (the pages never print them; this is the plainest reading of an
``nn.Linear`` whose projections the pages call q_proj / up_proj / down_proj):
x is [M, K] (tokens x in-features), W is [N, K] (out x in), y = x W^T is [M, N].
Activations and outputs are bf16, carried here as uint16 bit patterns.

Readings where the pages are silent:
* symmetric quantization, no zero point; scale = absmax / qmax computed in
  fp32 (one correctly rounded division), qmax = 127 for INT8 and 448 for
  e4m3fn; an all-zero row (or tensor) gets scale 1.0;
* codes are round-to-nearest-even of the fp32 quotient value / scale (an IEEE
  fp32 division, not a multiply by a reciprocal); INT8 codes are clamped to
  +-127 (-128 is never produced); FP8 codes saturate at +-448;
* W8A16 dequantizes each weight to bf16 *before* the product:
  wd = bf16(fp32(q) * s[n]) (one fp32 multiply, one rounding), the products
  x * wd accumulate without further rounding and the sum is rounded to fp32
  and then to bf16;
* W8A8 INT8 accumulates exactly (int32 on the device); W8A8 FP8 accumulates
  exactly here and is rounded once to fp32; the epilogue is
  y = bf16(fp32(acc) * fp32(s_x * s_w[n])), the combined scale formed in fp32;
* dynamic per-token activation quantization ("Nano-vLLM-MOE" README mirror,
  section "INT8 量化支持", key-design list: the W8A8 static bullet names the
  per-token absmax variant whose extra run-time reduce static scaling avoids)
  uses, for every row m, the weight
  quantizer's rule on that row alone: s_x[m] = absmax(x[m, :]) / qmax (1.0
  for an all-zero row) and xq = sat(RNE(x / s_x[m])); its epilogue is the
  static one with s_x replaced by s_x[m]:
  y = bf16(fp32(acc) * fp32(s_x[m] * s_w[n]));
* an optional bias b[n] (bf16, as the q/k/v projections of Qwen2-family models
  carry) is added in fp32 after the scale epilogue, before the bf16 rounding:
  y = bf16(fp32(v + b[n])) with v the fp32 value the epilogue would round.
"""
from __future__ import annotations

import numpy as np

from .codecs import (E4M3FN_MAX, INT8_QMAX, bf16_bits_to_f32, bf16_round,
                     e4m3fn_decode, e4m3fn_encode_sat, f32_to_bf16_bits)

INT8 = "int8"
FP8 = "fp8_e4m3fn"


def qmax_of(qtype: str) -> np.float32:
    """Largest code magnitude: 127 for INT8, 448 for e4m3fn."""
    if qtype == INT8:
        return np.float32(INT8_QMAX)
    if qtype == FP8:
        return np.float32(E4M3FN_MAX)
    raise ValueError(qtype)


def _to_f32(a: np.ndarray, is_bf16: bool) -> np.ndarray:
    return bf16_bits_to_f32(a) if is_bf16 else np.asarray(a, dtype=np.float32)


def weight_scale(absmax: np.ndarray, qtype: str) -> np.ndarray:
    """scale = fp32(absmax) / qmax in fp32; 1.0 where absmax is 0."""
    am = np.asarray(absmax, dtype=np.float32)
    s = (am / qmax_of(qtype)).astype(np.float32)
    return np.where(am == 0, np.float32(1.0), s).astype(np.float32)


def _encode(v_f32: np.ndarray, qtype: str) -> np.ndarray:
    """Quantize already-divided fp32 values to codes (int8 or e4m3fn uint8)."""
    if qtype == INT8:
        return np.clip(np.rint(v_f32), -INT8_QMAX, INT8_QMAX).astype(np.int8)
    return e4m3fn_encode_sat(v_f32)


def _decode(codes: np.ndarray, qtype: str) -> np.ndarray:
    """Codes -> exact values (float64)."""
    if qtype == INT8:
        return np.asarray(codes, dtype=np.int8).astype(np.float64)
    return e4m3fn_decode(codes)


def quantize_weight(w: np.ndarray, qtype: str, granularity: str = "per_channel",
                    w_is_bf16: bool = False):
    """Symmetric weight quantization of W[N, K].

    Per output channel n (or once for the whole tensor): absmax over the row,
    scale s = absmax / qmax, codes q = sat(RNE(w / s)).
    Returns (codes [N, K] int8 or uint8 e4m3fn, scales fp32 [N] or [1]).
    """
    wf = _to_f32(w, w_is_bf16)
    a = np.abs(wf)
    if granularity == "per_channel":
        s = weight_scale(a.max(axis=1), qtype)               # [N]
        q = _encode((wf / s[:, None]).astype(np.float32), qtype)
    elif granularity == "per_tensor":
        s = weight_scale(np.array([a.max()], dtype=np.float32), qtype)   # [1]
        q = _encode((wf / s[0]).astype(np.float32), qtype)
    else:
        raise ValueError(granularity)
    return q, s


def dequantize_weight_bf16(codes: np.ndarray, scales: np.ndarray, qtype: str) -> np.ndarray:
    """wd[n, k] = bf16(fp32(q[n, k]) * s[n]) as fp32 values (per-tensor: s broadcast)."""
    qf = _decode(codes, qtype).astype(np.float32)            # exact
    s = np.asarray(scales, dtype=np.float32).reshape(-1, 1)
    return bf16_round((qf * s).astype(np.float32))


def calibrate_input_scale(x_calib_bf16: np.ndarray, qtype: str) -> np.float32:
    """Static per-tensor input scale: absmax of the calibration batch / qmax (fp32)."""
    xf = bf16_bits_to_f32(x_calib_bf16)
    return weight_scale(np.array([np.abs(xf).max()], dtype=np.float32), qtype)[0]


def quantize_act_static(x_bf16: np.ndarray, input_scale, qtype: str) -> np.ndarray:
    """xq = sat(RNE(x / s_x)) with one fixed fp32 scalar s_x for the whole tensor."""
    xf = bf16_bits_to_f32(x_bf16)
    return _encode((xf / np.float32(input_scale)).astype(np.float32), qtype)


def quantize_act_dynamic(x_bf16: np.ndarray, qtype: str):
    """Per-token (per-row) dynamic quantization of x[M, K].

    Row m gets s_x[m] = fp32(absmax(x[m, :])) / qmax (1.0 if the row is all
    zero) and codes xq[m, k] = sat(RNE(x[m, k] / s_x[m])).
    Returns (codes [M, K] int8 or uint8 e4m3fn, scales fp32 [M]).
    """
    xf = bf16_bits_to_f32(x_bf16)
    s = weight_scale(np.abs(xf).max(axis=1), qtype)           # [M]
    q = _encode((xf / s[:, None]).astype(np.float32), qtype)
    return q, s


def _add_bias(v_f32: np.ndarray, bias_bf16) -> np.ndarray:
    """fp32(v + b[n]) for a bf16 bias [N] (no bias: v unchanged)."""
    if bias_bf16 is None:
        return v_f32
    b = bf16_bits_to_f32(np.asarray(bias_bf16, dtype=np.uint16)).reshape(1, -1)
    return (v_f32 + b).astype(np.float32)


def qlinear_w8a16(x_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                  qtype: str, bias_bf16=None) -> np.ndarray:
    """Weight-only quantized linear: y = bf16(fp32(sum_k x[m,k] * wd[n,k]) [+ b[n]]), bf16 bits [M, N]."""
    x = bf16_bits_to_f32(x_bf16).astype(np.float64)
    wd = dequantize_weight_bf16(codes, scales, qtype).astype(np.float64)
    acc = x @ wd.T
    return f32_to_bf16_bits(_add_bias(acc.astype(np.float32), bias_bf16))


def w8a8_accumulate(xq: np.ndarray, codes: np.ndarray, qtype: str) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * q[n, k].

    INT8: exact integers (every partial sum is an integer below 2^53 in
    magnitude for K <= 2^17, so the float64 matmul is exact), returned as int64.
    FP8: e4m3fn values are multiples of 2^-9 below 2^9 in magnitude, so the
    float64 matmul is exact for K <= 2^17; returned rounded once to fp32.
    """
    a = _decode(xq, qtype)
    b = _decode(codes, qtype)
    acc = a @ b.T
    if qtype == INT8:
        return np.rint(acc).astype(np.int64)
    return acc.astype(np.float32)


def w8a8_epilogue(acc: np.ndarray, input_scale, scales: np.ndarray, bias_bf16=None) -> np.ndarray:
    """y = bf16(fp32(acc) * fp32(s_x * s_w[n]) [+ b[n]]), bf16 bits [M, N]."""
    comb = (np.float32(input_scale) * np.asarray(scales, dtype=np.float32)).astype(np.float32)
    accf = np.asarray(acc).astype(np.float32)
    return f32_to_bf16_bits(_add_bias((accf * comb.reshape(1, -1)).astype(np.float32), bias_bf16))


def qlinear_w8a8_static(xq: np.ndarray, input_scale, codes: np.ndarray, scales: np.ndarray,
                        qtype: str, out: str = "bf16") -> np.ndarray:
    """W8A8 static GEMM on already-quantized activations.

    out="acc": int32 accumulators (INT8) or fp32 accumulators (FP8), no epilogue.
    out="bf16": the scaled and rounded bf16 bits.
    """
    acc = w8a8_accumulate(xq, codes, qtype)
    if out == "acc":
        if qtype == INT8:
            if np.abs(acc).max(initial=0) >= 2 ** 31:
                raise OverflowError("int32 accumulator overflow")
            return acc.astype(np.int32)
        return acc
    return w8a8_epilogue(acc, input_scale, scales)


def w8a8_epilogue_per_token(acc: np.ndarray, x_scale: np.ndarray, scales: np.ndarray,
                            bias_bf16=None) -> np.ndarray:
    """y[m, n] = bf16(fp32(acc[m, n]) * fp32(s_x[m] * s_w[n]) [+ b[n]]), bf16 bits [M, N]."""
    sx = np.asarray(x_scale, dtype=np.float32).reshape(-1, 1)
    comb = (sx * np.asarray(scales, dtype=np.float32).reshape(1, -1)).astype(np.float32)
    accf = np.asarray(acc).astype(np.float32)
    return f32_to_bf16_bits(_add_bias((accf * comb).astype(np.float32), bias_bf16))


def qlinear_w8a8_dynamic(xq: np.ndarray, x_scale: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                         qtype: str, out: str = "bf16") -> np.ndarray:
    """W8A8 GEMM on per-token quantized activations (row scales x_scale [M]).

    out="acc" is the same accumulator as the static scheme's; out="bf16" applies
    the per-token epilogue.
    """
    if out == "acc":
        return qlinear_w8a8_static(xq, 1.0, codes, scales, qtype, out="acc")
    return w8a8_epilogue_per_token(w8a8_accumulate(xq, codes, qtype), x_scale, scales)


def linear(scheme: str, x_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray, qtype: str,
           input_scale=None, bias_bf16=None, bf16_fallback_max_m: int = 0) -> np.ndarray:
    """The routed quantized Linear from bf16 x: bf16 bits [M, N].

    scheme "w8a16": qlinear_w8a16.  "w8a8_static": quantize_act_static with
    input_scale, then the static GEMM.  "w8a8_dynamic": per-token quantization,
    then the dynamic GEMM.  With bf16_fallback_max_m > 0, a W8A8 call with
    M <= bf16_fallback_max_m skips activation quantization and computes the
    W8A16 result on the same weight codes and scales (the small-batch BF16
    fallback of the INT8 key-design list; it changes the numerics, so it is opt-in).
    A bias is added in fp32 after the scale epilogue, before the bf16 rounding.
    """
    M = np.asarray(x_bf16).shape[0]
    if scheme == "w8a16" or (bf16_fallback_max_m > 0 and M <= bf16_fallback_max_m):
        return qlinear_w8a16(x_bf16, codes, scales, qtype, bias_bf16)
    if scheme == "w8a8_static":
        xq = quantize_act_static(x_bf16, input_scale, qtype)
        return w8a8_epilogue(w8a8_accumulate(xq, codes, qtype), input_scale, scales, bias_bf16)
    if scheme == "w8a8_dynamic":
        xq, sx = quantize_act_dynamic(x_bf16, qtype)
        return w8a8_epilogue_per_token(w8a8_accumulate(xq, codes, qtype), sx, scales, bias_bf16)
    raise ValueError(scheme)


def reconstruction_error(w: np.ndarray, codes: np.ndarray, scales: np.ndarray, qtype: str):
    """(relative L2 error, minimum row cosine) of dequant(q) = q * s against W.

    The quality measure the "tiny-vLLM" README reports for its quantized weights
    ("Quantization Results", "Quality Check": artifact check).
    """
    wf = np.asarray(w, dtype=np.float64)
    dq = _decode(codes, qtype) * np.asarray(scales, dtype=np.float64).reshape(-1, 1)
    rel = np.linalg.norm(dq - wf) / np.linalg.norm(wf)
    num = (dq * wf).sum(axis=1)
    den = np.linalg.norm(dq, axis=1) * np.linalg.norm(wf, axis=1)
    cos = np.where(den > 0, num / np.where(den > 0, den, 1.0), 1.0)
    return float(rel), float(cos.min())
