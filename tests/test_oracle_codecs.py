"""Pins of the oracle's number formats (CPU only).

bf16 and OCP e4m3fn are checked exhaustively against torch's CPU casts (an
independent implementation of the same public format definitions) and against
exact rational rounding written in tests/exact.py.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _torch_bf16_bits(a_f32):
    return torch.from_numpy(np.ascontiguousarray(a_f32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_bf16_decode_all_patterns():
    ours = oracle.bf16_bits_to_f32(ALL16)
    ref = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_encode_matches_torch_random_and_ties():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    # force a block of exact ties (low 16 bits == 0x8000) and near-ties
    u[:50_000] = (u[:50_000] & 0xFFFF0000) | 0x8000
    u[50_000:60_000] = (u[50_000:60_000] & 0xFFFF0000) | 0x7FFF
    u[60_000:70_000] = (u[60_000:70_000] & 0xFFFF0000) | 0x8001
    x = u.view(np.float32)
    fin = np.isfinite(x)
    ours = oracle.f32_to_bf16_bits(x[fin])
    ref = _torch_bf16_bits(x[fin])
    assert np.array_equal(ours, ref)
    # NaN stays NaN
    nans = x[~fin & np.isnan(x)]
    if nans.size:
        assert np.all(np.isnan(oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(nans))))


def test_bf16_encode_matches_exact_rounding():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(2000) * np.exp2(rng.integers(-30, 30, 2000))).astype(np.float32)
    bits = oracle.f32_to_bf16_bits(x)
    for xi, b in zip(x, bits):
        want = exact.bf16(Fraction(float(xi)))
        assert exact.bf16_bits_of(want) == int(b)


def test_bf16_overflow_rounds_to_inf():
    big = np.array([np.finfo(np.float32).max, -np.finfo(np.float32).max], np.float32)
    assert list(oracle.f32_to_bf16_bits(big)) == [0x7F80, 0xFF80]


def test_e4m3fn_decode_closed_form_points():
    codes = np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x39, 0x7E, 0xFE, 0x77], np.uint8)
    want = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 448.0, -448.0, 240.0]
    got = oracle.e4m3fn_decode(codes)
    assert list(got) == want
    assert np.signbit(got[1])
    assert np.isnan(oracle.e4m3fn_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3fn_decode_all_codes_vs_torch_and_exact():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert Fraction(float(ours[c])) == exact.e4m3fn_value(c)


def test_e4m3fn_encode_exhaustive_bf16_vs_torch_saturating():
    x = oracle.bf16_bits_to_f32(ALL16)
    fin = np.isfinite(x)
    ours = oracle.e4m3fn_encode_sat(x[fin])
    ref = torch.from_numpy(x[fin].copy()).clamp(-448, 448).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3fn_encode_midpoints_vs_bruteforce():
    # every midpoint between neighbouring finite codes, and one fp32 ulp either side
    vals = []
    for (c0, v0), (c1, v1) in zip(exact.E4M3_POS[:-1], exact.E4M3_POS[1:]):
        mid = np.float32(float((v0 + v1) / 2))
        vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    vals += [np.float32(448), np.float32(460), np.float32(464), np.float32(1e6), np.float32(np.inf)]
    x = np.array(vals + [-v for v in vals], np.float32)
    ours = oracle.e4m3fn_encode_sat(x)
    for xi, c in zip(x, ours):
        if np.isinf(xi):
            assert int(c) & 0x7F == 0x7E
            continue
        assert int(c) == exact.e4m3fn_nearest(Fraction(float(xi))), float(xi)


def test_e4m3fn_encode_random_fp32_vs_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(300_000) * np.exp2(rng.integers(-14, 10, 300_000))).astype(np.float32)
    ours = oracle.e4m3fn_encode_sat(x)
    ref = torch.from_numpy(x).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3fn_signed_zero_and_nan():
    z = oracle.e4m3fn_encode_sat(np.array([0.0, -0.0, np.nan], np.float32))
    assert z[0] == 0x00 and z[1] == 0x80 and (z[2] & 0x7F) == 0x7F
