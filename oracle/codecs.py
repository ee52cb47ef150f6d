"""Oracle number formats: bf16 and OCP FP8 e4m3fn, from their bit-level definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats but not their definitions: "FP8" / "e4m3" weights
and activations ("Nano-vLLM-MoE" README, sections "FP8 W8A16 weight-only
quantization" and "FP8 W8A8 static quantization") and BF16 activations and
outputs.  The definitions used here are the public ones:

* bf16: the upper 16 bits of an IEEE binary32; fp32 -> bf16 rounds to
  nearest, ties to even; a NaN stays a (quiet) NaN.
* e4m3fn (OCP 8-bit floating point, the "fn" variant -- not the fnuz variant):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
  holds subnormals m * 2^-9; no infinities; S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448 (code 0x7E).

Reading (the pages are silent): encoding into e4m3fn rounds to nearest, ties
to even, and SATURATES at +-448 -- a value of magnitude above 448 (including
one that would round past 448) becomes +-448 rather than NaN, the FP8
counterpart of clamping int8 codes to +-127.
"""
from __future__ import annotations

import numpy as np

E4M3FN_MAX = 448.0
INT8_QMAX = 127.0


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the fp32 values they denote (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN of the same sign."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16          # carries into the exponent when needed
    quiet = (u >> 16) | 0x0040
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value, returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> exact values as float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    sub = m * 2.0 ** -9
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def e4m3fn_encode_sat(v: np.ndarray) -> np.ndarray:
    """fp32 values -> e4m3fn codes (uint8): round to nearest even, saturate at +-448.

    Steps: take |v| exactly in float64; clamp it to 448; find its binade
    e = floor(log2|v|), with every value below the smallest normal 2^-6 placed
    in the subnormal binade e = -6; the code grid in that binade has spacing
    2^(e-3); round |v| / 2^(e-3) to the nearest integer n (ties to even);
    the code is (e + 7) * 8 + (n - 8), which also covers n = 16 (carry into the
    next binade) and the subnormals (e = -6 gives code n).
    NaN maps to 0x7F with the input's sign bit.
    """
    x = np.asarray(v, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    nan = np.isnan(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3FN_MAX)
    _, ex = np.frexp(a)                      # a = f * 2^ex with f in [0.5, 1)
    e = np.where(a == 0.0, -6, ex - 1)
    e = np.maximum(e, -6)
    n = np.rint(a / np.exp2((e - 3).astype(np.float64)))   # exact scaling, half-even
    code = (e + 7) * 8 + (n.astype(np.int64) - 8)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)
