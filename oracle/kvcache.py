"""Oracle KV-cache codec: mixed K-int8 (groups of 32, fp16 scales) / V-FP8 per-token.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Nano-vLLM-MoE" README, section "KV cache compression": its Setup list
(K as int8 in groups of 32 channels with float16 scales, V as FP8; quantized per
token at run time, as the README's overview also says), the "Historical
mixed-KV PPL" table (bytes per block 0.5195x BF16 at K group 32) and the Memory
table (7B, 512 fixed blocks:
KV arena 7.00 GiB BF16 -> 3.64 GiB mixed).

Layout (the pages' KV tensors are per token, per KV head, head_dim D): k and v
are bf16 [T, H, D] with D a multiple of 32.

Readings where the pages are silent:
* K: for every (token t, head h, group g of 32 consecutive channels),
  s = fp16(fp32(absmax) / 127) -- an fp32 division, then round to nearest even
  into IEEE binary16 -- and codes q = clamp(RNE(k / fp32(s)), -127, 127), the
  division by the stored fp16 value, so that decoding with the stored scale
  inverts exactly the step that was taken;
* V: one scale per (token, head): s = fp16(fp32(absmax over D) / 448), codes
  e4m3fn_sat(RNE(v / fp32(s))); "FP8" read as OCP e4m3fn, as for the weights;
* an all-zero group (row) gets s = 1; a positive absmax whose scale would round
  to 0 in fp16 gets the smallest positive fp16 value 2^-24; a scale above the
  largest finite fp16 value saturates to 65504;
* decoding gives bf16(fp32(q) * fp32(s)), one fp32 product and one bf16
  rounding, the rule the W8A16 weights follow.
These choices reproduce the pages' storage figures exactly: per (token, head)
with D = 128, K takes 128 + 4 * 2 bytes and V 128 + 2, i.e. 266 / 512 = 0.5195
of bf16, and the 7.00 GiB arena becomes 3.64 GiB.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_bits_to_f32, e4m3fn_decode, e4m3fn_encode_sat, f32_to_bf16_bits

K_GROUP = 32
FP16_MAX = 65504.0
FP16_MIN_SUB = 2.0 ** -24


def fp16_encode(x: np.ndarray) -> np.ndarray:
    """fp32 values -> IEEE binary16 bits (uint16): round to nearest even, saturating at +-65504.

    binary16: 1 sign bit, 5 exponent bits with bias 15, 10 fraction bits;
    exponent field 0 holds subnormals f * 2^-24.  For |x| in binade e (values
    below 2^-14 use the subnormal binade e = -14) the grid spacing is 2^(e-10);
    |x| / 2^(e-10) is rounded to the nearest integer n (ties to even) and the
    bits are (e + 15) * 1024 + (n - 1024), which also covers the carry n = 2048
    and the subnormals (e = -14 gives bits n).
    """
    a64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    neg = np.signbit(a64)
    a = np.minimum(np.abs(a64), FP16_MAX)
    _, ex = np.frexp(a)                      # a = f 2^ex, f in [0.5, 1)
    e = np.where(a == 0.0, -14, np.maximum(ex - 1, -14))
    step = np.exp2((e - 10).astype(np.float64))
    n = np.rint(a / step).astype(np.int64)   # a / step is exact in float64; rint is ties-to-even
    bits = np.where(e == -14, n, (e + 15) * 1024 + (n - 1024))
    return (bits | np.where(neg, 0x8000, 0)).astype(np.uint16)


def fp16_decode(bits: np.ndarray) -> np.ndarray:
    """binary16 bits -> exact values (float64); only finite patterns are meaningful here."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    mag = np.where(e == 0, f * 2.0 ** -24, (1.0 + f / 1024.0) * np.exp2((e - 15).astype(np.float64)))
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def _scale_bits(absmax: np.ndarray, qmax: float) -> np.ndarray:
    """Stored fp16 scale for fp32 absmax values (the readings above)."""
    am = np.asarray(absmax, dtype=np.float32)
    s = fp16_encode((am / np.float32(qmax)).astype(np.float32))
    s = np.where(am == 0, fp16_encode(np.float32(1.0)), s)
    s = np.where((am > 0) & (s == 0), np.uint16(1), s)          # 2^-24
    return s.astype(np.uint16)


def kv_quantize(k_bf16: np.ndarray, v_bf16: np.ndarray):
    """Quantize bf16 K and V [T, H, D] for the cache.

    Returns (k_codes int8 [T,H,D], k_scales fp16 bits [T,H,D/32],
             v_codes e4m3fn uint8 [T,H,D], v_scales fp16 bits [T,H]).
    """
    kf = bf16_bits_to_f32(k_bf16)
    vf = bf16_bits_to_f32(v_bf16)
    T, H, D = kf.shape
    if D % K_GROUP:
        raise ValueError("head_dim must be a multiple of 32")
    kg = kf.reshape(T, H, D // K_GROUP, K_GROUP)
    ks = _scale_bits(np.abs(kg).max(axis=3), 127.0)                       # [T,H,G]
    ksf = fp16_decode(ks).astype(np.float32)
    kq = np.clip(np.rint((kg / ksf[..., None]).astype(np.float32)), -127, 127).astype(np.int8)
    vs = _scale_bits(np.abs(vf).max(axis=2), 448.0)                       # [T,H]
    vsf = fp16_decode(vs).astype(np.float32)
    vq = e4m3fn_encode_sat((vf / vsf[..., None]).astype(np.float32))
    return kq.reshape(T, H, D), ks, vq, vs


def kv_dequantize(k_codes, k_scales, v_codes, v_scales):
    """Cache entries -> bf16 bits of K and V [T, H, D]: bf16(fp32(q) * fp32(s))."""
    kq = np.asarray(k_codes, dtype=np.int8)
    T, H, D = kq.shape
    ksf = fp16_decode(k_scales).astype(np.float32)                        # exact in fp32
    kd = (kq.reshape(T, H, D // K_GROUP, K_GROUP).astype(np.float32) * ksf[..., None]).astype(np.float32)
    vsf = fp16_decode(v_scales).astype(np.float32)
    vd = (e4m3fn_decode(v_codes).astype(np.float32) * vsf[..., None]).astype(np.float32)
    return f32_to_bf16_bits(kd.reshape(T, H, D)), f32_to_bf16_bits(vd)


def kv_bytes_per_token_head(D: int) -> int:
    """Storage of one (token, head) entry: K codes + K fp16 scales + V codes + one V fp16 scale."""
    return D + 2 * (D // K_GROUP) + D + 2
