"""Pins of the oracle's KV-cache codec (CPU only): the fp16 codec against numpy's
float16, the pages' storage figures (tests/golden/kv_cache_figures.txt), exact
rational brute force, round-trip bounds and structural invariants."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_figures.txt")
F16 = (11, -14)          # binary16: 11 significand bits, minimum normal exponent -14


def _golden():
    kv = {}
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            kv[k] = float(v)
    return kv


def test_fp16_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.fp16_decode(bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_fp16_encode_matches_numpy_cast_incl_midpoints():
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(200000).astype(np.float32) * np.float32(s) for s in (1e-6, 1e-3, 1.0, 100.0, 3e4)]
    # every finite fp16 value, the midpoints to its neighbour, and one fp32 ulp either side
    f = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((f[:-1] + f[1:]) / 2).astype(np.float32)
    vals += [mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0)), f.astype(np.float32)]
    x = np.concatenate(vals)
    x = np.concatenate([x, -x])
    ref = np.clip(x, -65504, 65504).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.fp16_encode(x), ref)


def test_fp16_encode_saturates():
    assert list(oracle.fp16_encode(np.array([7e4, -1e30, 65519.0, 65520.0], np.float32))) == [0x7BFF, 0xFBFF,
                                                                                              0x7BFF, 0x7BFF]


def test_storage_figures_of_the_pages():
    g = _golden()
    D = int(g["head_dim"])
    per = oracle.kv_bytes_per_token_head(D)
    assert round(per / (4 * D), 4) == g["bytes_per_block_ratio"]
    entries = g["blocks"] * g["block_tokens"] * g["layers"] * g["kv_heads"]
    assert round(entries * 4 * D / 2 ** 30, 2) == g["arena_bf16_gib"]
    assert round(entries * per / 2 ** 30, 2) == g["arena_mixed_gib"]


def _exact_scale(vals, qmax):
    am = max(abs(Fraction(float(v))) for v in vals)
    if am == 0:
        return Fraction(1)
    s = exact.round_to_format(exact.f32(am / qmax), *F16)
    return s if s != 0 else Fraction(1, 2 ** 24)


def test_kv_quantize_bruteforce():
    rng = np.random.default_rng(2)
    T, H, D = 3, 2, 64
    k = rng.standard_normal((T, H, D)).astype(np.float32) * np.float32(3.0)
    v = rng.standard_normal((T, H, D)).astype(np.float32) * np.float32(0.5)
    k[1, 0, 32:] = 0.0                                   # a zero group
    k[2, 1, :32] *= np.float32(1e-9)                     # a group whose scale underflows fp16
    kb, vb = oracle.f32_to_bf16_bits(k), oracle.f32_to_bf16_bits(v)
    kq, ks, vq, vs = oracle.kv_quantize(kb, vb)
    kf, vf = oracle.bf16_bits_to_f32(kb), oracle.bf16_bits_to_f32(vb)
    for t in range(T):
        for h in range(H):
            for g in range(D // 32):
                grp = kf[t, h, 32 * g: 32 * g + 32]
                s = _exact_scale(grp, 127)
                assert Fraction(float(oracle.fp16_decode(ks[t, h, g]))) == s
                for i, x in enumerate(grp):
                    c = max(-127, min(127, exact.rne_int(exact.f32(Fraction(float(x)) / s))))
                    assert int(kq[t, h, 32 * g + i]) == c
            s = _exact_scale(vf[t, h], 448)
            assert Fraction(float(oracle.fp16_decode(vs[t, h]))) == s
            for i, x in enumerate(vf[t, h]):
                assert int(vq[t, h, i]) & 0x7F == exact.e4m3fn_nearest(exact.f32(Fraction(float(x)) / s)) & 0x7F
    assert ks[1, 0, 1] == 0x3C00 and np.all(kq[1, 0, 32:] == 0)       # zero group: scale 1, codes 0
    assert ks[2, 1, 0] == 0x0001                                      # underflow: smallest fp16


def test_kv_roundtrip_bounds():
    rng = np.random.default_rng(3)
    k = oracle.f32_to_bf16_bits(rng.standard_normal((64, 4, 128)).astype(np.float32))
    v = oracle.f32_to_bf16_bits(rng.standard_normal((64, 4, 128)).astype(np.float32))
    kq, ks, vq, vs = oracle.kv_quantize(k, v)
    kd, vd = oracle.kv_dequantize(kq, ks, vq, vs)
    kf, kdf = oracle.bf16_bits_to_f32(k).astype(np.float64), oracle.bf16_bits_to_f32(kd).astype(np.float64)
    s = np.repeat(oracle.fp16_decode(ks), 32, axis=2)
    # int8: |k - q s| <= s/2 (the fp16 scale never makes 127 s smaller than the absmax by more
    # than one code), then one bf16 rounding
    assert np.all(np.abs(kf - kdf) <= s * 0.5 * (1 + 2 ** -10) + np.abs(kdf) * 2.0 ** -8)
    vf, vdf = oracle.bf16_bits_to_f32(v).astype(np.float64), oracle.bf16_bits_to_f32(vd).astype(np.float64)
    sv = oracle.fp16_decode(vs)[..., None]
    # e4m3: relative half-ulp 2^-4 of the code value (or half the subnormal step 2^-10 s), then bf16
    bound = np.maximum(np.abs(vf) * 2.0 ** -4, sv * 2.0 ** -10) * (1 + 2 ** -9) + np.abs(vdf) * 2.0 ** -8
    assert np.all(np.abs(vf - vdf) <= bound)
    # the measured quality sits where 8-bit codes put it
    assert np.linalg.norm(kf - kdf) / np.linalg.norm(kf) < 0.01
    assert np.linalg.norm(vf - vdf) / np.linalg.norm(vf) < 0.04


def test_kv_groups_and_tokens_are_independent():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((2, 2, 96)).astype(np.float32)
    v = rng.standard_normal((2, 2, 96)).astype(np.float32)
    a = oracle.kv_quantize(oracle.f32_to_bf16_bits(k), oracle.f32_to_bf16_bits(v))
    k2, v2 = k.copy(), v.copy()
    k2[0, 1, 40] = 100.0                                 # one K group of one (token, head)
    v2[1, 0, 3] = -50.0                                  # one V row
    b = oracle.kv_quantize(oracle.f32_to_bf16_bits(k2), oracle.f32_to_bf16_bits(v2))
    kq, ks, vq, vs = a
    kq2, ks2, vq2, vs2 = b
    mask = np.ones(ks.shape, bool)
    mask[0, 1, 1] = False
    assert np.array_equal(ks[mask], ks2[mask]) and not np.array_equal(ks[0, 1, 1], ks2[0, 1, 1])
    kmask = np.ones(kq.shape, bool)
    kmask[0, 1, 32:64] = False
    assert np.array_equal(kq[kmask], kq2[kmask])
    vmask = np.ones(vs.shape, bool)
    vmask[1, 0] = False
    assert np.array_equal(vs[vmask], vs2[vmask]) and np.array_equal(vq[vmask], vq2[vmask])


def test_kv_power_of_two_scaling():
    # scaling a (token, head) by 2^j leaves the codes and multiplies the fp16 scales by 2^j
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 3, 64)).astype(np.float32)
    v = rng.standard_normal((1, 3, 64)).astype(np.float32)
    f = np.array([2.0 ** -3, 1.0, 2.0 ** 4], np.float32)[None, :, None]
    a = oracle.kv_quantize(oracle.f32_to_bf16_bits(k), oracle.f32_to_bf16_bits(v))
    b = oracle.kv_quantize(oracle.f32_to_bf16_bits(k * f), oracle.f32_to_bf16_bits(v * f))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    assert np.array_equal(oracle.fp16_decode(b[1]), oracle.fp16_decode(a[1]) * f[..., 0][..., None])
    assert np.array_equal(oracle.fp16_decode(b[3]), oracle.fp16_decode(a[3]) * f[..., 0])


def test_kv_dequantize_bruteforce():
    rng = np.random.default_rng(6)
    kq = rng.integers(-127, 128, size=(2, 1, 32)).astype(np.int8)
    vq = rng.integers(0, 256, size=(2, 1, 32)).astype(np.uint8)
    vq[(vq & 0x7F) == 0x7F] = 0x10                       # no NaN codes
    ks = oracle.fp16_encode(np.array([[[0.0123]], [[3.5]]], np.float32))
    vs = oracle.fp16_encode(np.array([[0.07], [1e-3]], np.float32))
    kd, vd = oracle.kv_dequantize(kq, ks, vq, vs)
    for t in range(2):
        sk = Fraction(float(oracle.fp16_decode(ks[t, 0, 0])))
        sv = Fraction(float(oracle.fp16_decode(vs[t, 0])))
        for i in range(32):
            assert kd[t, 0, i] == exact.bf16_bits_of(exact.bf16(exact.f32(int(kq[t, 0, i]) * sk)))
            assert vd[t, 0, i] == exact.bf16_bits_of(exact.bf16(exact.f32(exact.e4m3fn_value(int(vq[t, 0, i])) * sv)))
