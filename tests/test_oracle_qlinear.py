"""Pins of the oracle's quantizers and GEMMs (CPU only).

Each test checks the oracle against something other than itself: exact
rational arithmetic (tests/exact.py), closed forms, integer special cases, an
independent library routine (numpy int64 matmul, torch bf16 matmul) or a
statistical law of uniform quantization noise.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import exact

QTYPES = ["int8", "fp8_e4m3fn"]
QMAX = {"int8": 127, "fp8_e4m3fn": 448}


# ---------------------------------------------------------------- brute force helpers
def _exact_scale(row_vals, qtype):
    am = max(abs(Fraction(float(v))) for v in row_vals)
    if am == 0:
        return Fraction(1)
    return exact.f32(am / QMAX[qtype])


def _exact_code(v, s, qtype):
    """Code of one fp32 value v for scale s, from exact rationals."""
    t = exact.f32(Fraction(float(v)) / s)          # IEEE fp32 division
    if qtype == "int8":
        return max(-127, min(127, exact.rne_int(t)))
    return exact.e4m3fn_nearest(t)


def _code_value(c, qtype):
    return Fraction(int(np.int8(c))) if qtype == "int8" else exact.e4m3fn_value(int(c))


# ---------------------------------------------------------------- weight quantizer
@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("gran", ["per_channel", "per_tensor"])
def test_quantize_weight_bruteforce(qtype, gran):
    rng = np.random.default_rng(11)
    for N, K in [(1, 1), (3, 5), (8, 8), (5, 7)]:
        w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
        q, s = oracle.quantize_weight(w, qtype, gran)
        if gran == "per_channel":
            ss = [_exact_scale(w[n], qtype) for n in range(N)]
        else:
            ss = [_exact_scale(w.ravel(), qtype)] * N
        assert s.shape == ((N,) if gran == "per_channel" else (1,))
        for n in range(N):
            assert Fraction(float(s[n if gran == "per_channel" else 0])) == ss[n]
            for k in range(K):
                assert int(q[n, k]) & 0xFF == _exact_code(w[n, k], ss[n], qtype) & 0xFF


@pytest.mark.parametrize("qtype", QTYPES)
def test_absmax_element_maps_to_qmax(qtype):
    w, _, _ = synth.small_inputs(5, 1, 300, 64)
    q, s = oracle.quantize_weight(w, qtype)
    dec = oracle.e4m3fn_decode(q) if qtype != "int8" else q.astype(np.float64)
    idx = np.abs(w).argmax(axis=1)
    got = dec[np.arange(64), idx]
    assert np.array_equal(np.abs(got), np.full(64, QMAX[qtype], np.float64))
    assert np.array_equal(np.sign(got), np.sign(w[np.arange(64), idx]))


@pytest.mark.parametrize("qtype", QTYPES)
def test_zero_rows_get_unit_scale(qtype):
    w = np.zeros((4, 70), np.float32)
    w[2, 3] = 0.5
    q, s = oracle.quantize_weight(w, qtype)
    assert s[0] == 1.0 and s[1] == 1.0 and s[3] == 1.0
    assert not q[[0, 1, 3]].any()
    q2, s2 = oracle.quantize_weight(np.zeros((3, 9), np.float32), qtype, "per_tensor")
    assert s2[0] == 1.0 and not q2.any()


def test_int8_roundtrip_bound():
    # |w - q s| <= s (1/2 + 127 * 2^-24): RNE of the fp32 quotient, which itself
    # carries at most half an fp32 ulp of relative error.
    w, _, _ = synth.small_inputs(6, 1, 2048, 512)
    q, s = oracle.quantize_weight(w, "int8")
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 127 * 2.0 ** -24))


def test_fp8_roundtrip_bound():
    # |w/s - dec(q)| <= half the e4m3fn spacing at |w/s| (+ fp32 quotient rounding)
    w, _, _ = synth.small_inputs(7, 1, 2048, 256)
    q, s = oracle.quantize_weight(w, "fp8_e4m3fn")
    t = w.astype(np.float64) / s.astype(np.float64)[:, None]
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(t), 2.0 ** -30))), -6)
    half_spacing = 0.5 * np.exp2(e - 3)
    err = np.abs(t - oracle.e4m3fn_decode(q))
    assert np.all(err <= half_spacing * (1 + 2.0 ** -20) + np.abs(t) * 2.0 ** -23)


def test_int8_relative_error_matches_uniform_noise_law():
    # Uniform rounding noise of width s has variance s^2/12 per element, so
    # relL2^2 ~= sum_n K s_n^2 / 12 / sum w^2.  A wrong qmax (255, 128) or a
    # missing clamp would be off by a large factor.
    w = synth.weight(np.random.default_rng(0), 512, 2048)
    q, s = oracle.quantize_weight(w, "int8")
    rel, cos = oracle.reconstruction_error(w, q, s, "int8")
    pred = np.sqrt((2048 * (s.astype(np.float64) ** 2)).sum() / 12 / (w.astype(np.float64) ** 2).sum())
    assert abs(rel / pred - 1) < 0.03
    # Same order as the trained-weight artifact check the tiny-vLLM README
    # reports for INT8 weights (relative L2 about 0.0095, min cosine about 0.9999).
    assert 0.005 < rel < 0.0095 * 1.5 and cos > 0.9998


@pytest.mark.parametrize("qtype", QTYPES)
def test_reconstruction_error_closed_form(qtype):
    """Rows built from Pythagorean pairs have known cosines: dequant (3, 4) against
    W (4, 3) has cosine 24/25, (5, 12) against (12, 5) has 120/169; a zero row and
    an exact row have cosine 1.  The minimum over rows is 120/169 and the relative
    L2 error is sqrt(100 / 243).  A column-wise cosine (0.976), a mean over rows
    (0.917) or scales applied along the wrong axis give other values."""
    W = np.array([[4, 3, 0, 0], [12, 5, 0, 0], [0, 0, 0, 0], [0, 0, 7, 0]], np.float32)
    q = np.array([[6, 8, 0, 0], [5, 12, 0, 0], [0, 0, 0, 0], [0, 0, 7, 0]], np.float32)
    s = np.array([0.5, 1.0, 1.0, 1.0], np.float32)          # row 0 dequantizes to (3, 4)
    codes = q.astype(np.int8) if qtype == "int8" else oracle.e4m3fn_encode_sat(q)
    assert np.array_equal(oracle.e4m3fn_decode(codes), q) if qtype != "int8" else True
    rel, cos = oracle.reconstruction_error(W, codes, s, qtype)
    assert cos == pytest.approx(120 / 169, abs=1e-15)
    assert rel == pytest.approx(np.sqrt(100 / 243), abs=1e-15)
    # a per-tensor scale broadcasts over every row
    rel1, cos1 = oracle.reconstruction_error(W[1:], codes[1:], np.array([1.0], np.float32), qtype)
    assert cos1 == pytest.approx(120 / 169, abs=1e-15) and rel1 == pytest.approx(np.sqrt(98 / 218), abs=1e-15)


def test_integer_weights_scale_one_int8():
    rng = np.random.default_rng(9)
    W = rng.integers(-127, 128, size=(16, 40)).astype(np.float32)
    W[:, 0] = np.where(rng.random(16) < 0.5, 127, -127)
    q, s = oracle.quantize_weight(W, "int8")
    assert np.all(s == 1.0) and np.array_equal(q.astype(np.float32), W)


def test_representable_weights_scale_one_fp8_per_tensor():
    vals = np.array([float(v) for _, v in exact.E4M3_POS], np.float32)
    W = np.concatenate([vals, -vals]).reshape(2, -1)
    q, s = oracle.quantize_weight(W, "fp8_e4m3fn", "per_tensor")
    assert s[0] == 1.0
    assert np.array_equal(oracle.e4m3fn_decode(q), W.astype(np.float64))


def test_weight_quantizer_uses_division_not_reciprocal():
    # Find fp32 (w, s) where RNE(w / s) != RNE(w * (1/s)) by aiming w at the
    # midpoints (j + 1/2) s; the oracle must follow the division (the plain
    # reading of "w divided by its scale").
    rng = np.random.default_rng(12)
    am = (np.abs(rng.standard_normal(4000)) * 0.06 + 0.01).astype(np.float32)
    s = (am / np.float32(127)).astype(np.float32)
    j = rng.integers(0, 126, 4000).astype(np.float32)
    base = ((j + np.float32(0.5)) * s).astype(np.float32)
    hits = 0
    for d in range(-3, 4):
        w = base.copy()
        for _ in range(abs(d)):
            w = np.nextafter(w, np.float32(np.sign(d) * 1e9)).astype(np.float32)
        a = np.rint((w / s).astype(np.float32))
        b = np.rint((w * (np.float32(1) / s).astype(np.float32)).astype(np.float32))
        for i in np.nonzero(a != b)[0][:3]:
            row = np.array([[w[i], am[i]]], np.float32)
            q, ss = oracle.quantize_weight(row, "int8")
            assert ss[0] == s[i]
            assert q[0, 0] == _exact_code(w[i], Fraction(float(s[i])), "int8") == a[i]
            hits += 1
    assert hits >= 3


# ---------------------------------------------------------------- activation quantizer
@pytest.mark.parametrize("qtype", QTYPES)
def test_act_quant_integer_values_scale_one(qtype):
    x = np.arange(-127, 128, dtype=np.float32).reshape(5, 51)
    xb = oracle.f32_to_bf16_bits(x)            # integers up to 127 are exact in bf16
    q = oracle.quantize_act_static(xb, 1.0, qtype)
    if qtype == "int8":
        assert np.array_equal(q.astype(np.float32), x)
    else:   # e4m3fn rounds integers above 16 to its 3-bit mantissa grid
        want = np.array([exact.e4m3fn_nearest(Fraction(int(v))) for v in x.ravel()]).reshape(x.shape)
        assert np.array_equal(q.astype(np.int64), want)


@pytest.mark.parametrize("qtype", QTYPES)
def test_act_quant_saturates(qtype):
    x = oracle.f32_to_bf16_bits(np.array([[1e4, -1e4, 5.0, -5.0]], np.float32))
    q = oracle.quantize_act_static(x, 0.01, qtype)
    if qtype == "int8":
        assert list(q[0]) == [127, -127, 127, -127]
    else:
        assert list(q[0]) == [0x7E, 0xFE, 0x7E, 0xFE]


@pytest.mark.parametrize("qtype", QTYPES)
def test_act_quant_bruteforce(qtype):
    _, calib, x = synth.small_inputs(13, 6, 7, 3)
    s = oracle.calibrate_input_scale(calib, qtype)
    cal = oracle.bf16_bits_to_f32(calib)
    assert Fraction(float(s)) == exact.f32(max(abs(Fraction(float(v))) for v in cal.ravel()) / QMAX[qtype])
    q = oracle.quantize_act_static(x, s, qtype)
    xf = oracle.bf16_bits_to_f32(x)
    for m in range(6):
        for k in range(7):
            assert int(q[m, k]) & 0xFF == _exact_code(xf[m, k], Fraction(float(s)), qtype) & 0xFF


def test_calibration_absmax_element_is_qmax():
    _, calib, _ = synth.small_inputs(14, 1, 512, 1)
    for qtype in QTYPES:
        s = oracle.calibrate_input_scale(calib, qtype)
        q = oracle.quantize_act_static(calib, s, qtype)
        i = np.abs(oracle.bf16_bits_to_f32(calib)).argmax()
        v = q.ravel()[i]
        mag = abs(int(np.int8(v))) if qtype == "int8" else abs(float(oracle.e4m3fn_decode(np.array([v], np.uint8))[0]))
        assert mag == QMAX[qtype]


# ---------------------------------------------------------------- W8A16
def _bruteforce_w8a16(xb, q, s, qtype):
    M, K = xb.shape
    N = q.shape[0]
    xf = oracle.bf16_bits_to_f32(xb)
    out = np.zeros((M, N), np.uint16)
    for n in range(N):
        sn = Fraction(float(s[n if s.size > 1 else 0]))
        wd = [exact.bf16(exact.f32(_code_value(q[n, k], qtype) * sn)) for k in range(K)]
        for m in range(M):
            acc = sum(Fraction(float(xf[m, k])) * wd[k] for k in range(K))
            out[m, n] = exact.bf16_bits_of(exact.bf16(exact.f32(acc)))
    return out


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("MKN", [(1, 1, 1), (2, 8, 3), (8, 8, 8), (3, 5, 7), (8, 1, 4)])
def test_w8a16_bruteforce_exact(qtype, MKN):
    M, K, N = MKN
    w, _, x = synth.small_inputs(21 + M * 100 + K * 10 + N, M, K, N)
    q, s = oracle.quantize_weight(w, qtype)
    got = oracle.qlinear_w8a16(x, q, s, qtype)
    assert np.array_equal(got, _bruteforce_w8a16(x, q, s, qtype))


@pytest.mark.parametrize("qtype", QTYPES)
def test_w8a16_one_hot_returns_dequantized_weight(qtype):
    w, _, _ = synth.small_inputs(31, 1, 96, 40)
    q, s = oracle.quantize_weight(w, qtype)
    wd = oracle.dequantize_weight_bf16(q, s, qtype)
    for k in [0, 17, 95]:
        x = np.zeros((1, 96), np.float32)
        x[0, k] = 1.0
        y = oracle.qlinear_w8a16(oracle.f32_to_bf16_bits(x), q, s, qtype)
        assert np.array_equal(oracle.bf16_bits_to_f32(y[0]), wd[:, k])


def test_w8a16_integer_weights_exact():
    rng = np.random.default_rng(32)
    M, K, N = 4, 64, 12
    W = rng.integers(-127, 128, size=(N, K)).astype(np.float32)
    W[:, 5] = 127
    X = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    q, s = oracle.quantize_weight(W, "int8")
    assert np.all(s == 1.0)
    y = oracle.qlinear_w8a16(oracle.f32_to_bf16_bits(X), q, s, "int8")
    ref = X.astype(np.int64) @ W.astype(np.int64).T            # exact integers
    want = [exact.bf16_bits_of(exact.bf16(exact.f32(Fraction(int(v))))) for v in ref.ravel()]
    assert np.array_equal(y.ravel(), np.array(want, np.uint16))


@pytest.mark.parametrize("qtype", QTYPES)
def test_w8a16_matches_bf16_dequant_gemm(qtype):
    # The pages' identity: the weight-only kernel equals a plain bf16 GEMM on the
    # dequantized weights (torch CPU bf16 matmul as the independent routine).
    w, _, x = synth.small_inputs(33, 16, 512, 200)
    q, s = oracle.quantize_weight(w, qtype)
    y = oracle.bf16_bits_to_f32(oracle.qlinear_w8a16(x, q, s, qtype)).astype(np.float64)
    wd = torch.from_numpy(oracle.dequantize_weight_bf16(q, s, qtype)).to(torch.bfloat16)
    xt = torch.from_numpy(oracle.bf16_bits_to_f32(x)).to(torch.bfloat16)
    ref = (xt @ wd.T.contiguous()).float().numpy().astype(np.float64)
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 4e-3
    assert np.max(np.abs(y - ref) / (np.abs(ref) + np.sqrt(np.mean(ref ** 2)))) < 8e-3


def test_w8a16_scale_after_product_is_a_different_reading():
    # Applying the per-channel scale after the accumulation instead of before it
    # gives a measurably different result; the oracle must not do that.
    w, _, x = synth.small_inputs(34, 16, 1024, 256)
    q, s = oracle.quantize_weight(w, "fp8_e4m3fn")
    y = oracle.qlinear_w8a16(x, q, s, "fp8_e4m3fn")
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    late = (xf @ oracle.e4m3fn_decode(q).T) * s.astype(np.float64)[None, :]
    late_bits = oracle.f32_to_bf16_bits(late.astype(np.float32))
    assert (late_bits != y).mean() > 0.05


# ---------------------------------------------------------------- W8A8 static
@pytest.mark.parametrize("qtype", QTYPES)
def test_w8a8_accumulator_bruteforce(qtype):
    rng = np.random.default_rng(41)
    for M, K, N in [(1, 1, 1), (3, 8, 5), (8, 8, 8), (2, 7, 3)]:
        if qtype == "int8":
            xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
            q = rng.integers(-127, 128, (N, K)).astype(np.int8)
        else:
            pool = np.array([c for c, _ in exact.E4M3_POS] + [c | 0x80 for c, _ in exact.E4M3_POS], np.uint8)
            xq = rng.choice(pool, (M, K))
            q = rng.choice(pool, (N, K))
        acc = oracle.qlinear_w8a8_static(xq, 1.0, q, np.ones(N, np.float32), qtype, out="acc")
        for m in range(M):
            for n in range(N):
                ex = sum(_code_value(xq[m, k], qtype) * _code_value(q[n, k], qtype) for k in range(K))
                if qtype == "int8":
                    assert int(acc[m, n]) == ex
                else:
                    assert Fraction(float(acc[m, n])) == exact.f32(ex)


def test_w8a8_int8_accumulator_vs_integer_matmul():
    rng = np.random.default_rng(42)
    xq = rng.integers(-127, 128, (37, 11008)).astype(np.int8)
    q = rng.integers(-127, 128, (29, 11008)).astype(np.int8)
    acc = oracle.qlinear_w8a8_static(xq, 1.0, q, np.ones(29, np.float32), "int8", out="acc")
    ref = np.matmul(xq.astype(np.int64), q.astype(np.int64).T)    # integer loop, not BLAS
    assert acc.dtype == np.int32 and np.array_equal(acc.astype(np.int64), ref)


def test_w8a8_int8_worst_case_accumulator_fits_int32():
    K = 11008
    xq = np.full((1, K), 127, np.int8)
    q = np.full((2, K), -127, np.int8)
    acc = oracle.qlinear_w8a8_static(xq, 1.0, q, np.ones(2, np.float32), "int8", out="acc")
    assert int(acc[0, 0]) == -127 * 127 * K


@pytest.mark.parametrize("qtype", QTYPES)
def test_w8a8_epilogue_bruteforce(qtype):
    w, calib, x = synth.small_inputs(43, 5, 8, 6)
    gran = "per_channel" if qtype == "int8" else "per_tensor"
    q, s = oracle.quantize_weight(w, qtype, gran)
    sx = oracle.calibrate_input_scale(calib, qtype)
    xq = oracle.quantize_act_static(x, sx, qtype)
    y = oracle.qlinear_w8a8_static(xq, sx, q, s, qtype)
    for m in range(5):
        for n in range(6):
            acc = sum(_code_value(xq[m, k], qtype) * _code_value(q[n, k], qtype) for k in range(8))
            comb = exact.f32(Fraction(float(sx)) * Fraction(float(s[n if s.size > 1 else 0])))
            v = exact.bf16(exact.f32(exact.f32(acc) * comb))
            assert y[m, n] == exact.bf16_bits_of(v)


@pytest.mark.parametrize("qtype,gran", [("int8", "per_channel"), ("fp8_e4m3fn", "per_tensor")])
def test_w8a8_matches_bf16_dequant_reference(qtype, gran):
    # The pages check the W8A8 kernel against a BF16-dequant reference and find the values agree.
    w, calib, x = synth.small_inputs(44, 64, 1024, 256)
    q, s = oracle.quantize_weight(w, qtype, gran)
    sx = oracle.calibrate_input_scale(calib, qtype)
    xq = oracle.quantize_act_static(x, sx, qtype)
    y = oracle.bf16_bits_to_f32(oracle.qlinear_w8a8_static(xq, sx, q, s, qtype)).astype(np.float64)
    dec = (lambda c: c.astype(np.float64)) if qtype == "int8" else oracle.e4m3fn_decode
    xd = torch.from_numpy(dec(xq) * float(sx)).to(torch.bfloat16)
    wd = torch.from_numpy(dec(q) * s.astype(np.float64).reshape(-1, 1)).to(torch.bfloat16)
    ref = (xd @ wd.T.contiguous()).float().numpy().astype(np.float64)
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 4e-3
    assert np.max(np.abs(y - ref) / (np.abs(ref) + np.sqrt(np.mean(ref ** 2)))) < 8e-3


def test_w8a8_fp8_integer_weights_scale_one():
    rng = np.random.default_rng(45)
    W = rng.integers(-16, 17, size=(8, 32)).astype(np.float32)
    W[0, 0] = 448.0
    q, s = oracle.quantize_weight(W, "fp8_e4m3fn", "per_tensor")
    assert s[0] == 1.0 and np.array_equal(oracle.e4m3fn_decode(q), W.astype(np.float64))
    xq = oracle.quantize_act_static(oracle.f32_to_bf16_bits(rng.integers(-4, 5, (3, 32)).astype(np.float32)),
                                    1.0, "fp8_e4m3fn")
    acc = oracle.qlinear_w8a8_static(xq, 1.0, q, s, "fp8_e4m3fn", out="acc")
    ref = oracle.e4m3fn_decode(xq) @ W.astype(np.float64).T
    assert np.array_equal(acc.astype(np.float64), ref)


# ---------------------------------------------------------------- dynamic per-token activations
@pytest.mark.parametrize("qtype", QTYPES)
def test_act_dynamic_bruteforce(qtype):
    # every row's scale and every code from exact rationals, row by row
    _, _, x = synth.small_inputs(51, 5, 9, 1)
    xf = oracle.bf16_bits_to_f32(x)
    xf[2] = 0.0                                  # an all-zero row gets scale 1.0, codes 0
    xb = oracle.f32_to_bf16_bits(xf)
    q, s = oracle.quantize_act_dynamic(xb, qtype)
    assert s.dtype == np.float32 and s.shape == (5,)
    for m in range(5):
        sm = _exact_scale(xf[m], qtype)
        assert Fraction(float(s[m])) == sm
        for k in range(9):
            assert int(q[m, k]) & 0xFF == _exact_code(xf[m, k], sm, qtype) & 0xFF


@pytest.mark.parametrize("qtype", QTYPES)
def test_act_dynamic_row_absmax_maps_to_qmax_and_rows_are_independent(qtype):
    # rows of very different magnitude: a tensor-wide scale would crush the small rows
    rng = np.random.default_rng(52)
    xf = rng.standard_normal((4, 300)).astype(np.float32) * np.array([[1e-3], [1.0], [30.0], [1e3]], np.float32)
    xb = oracle.f32_to_bf16_bits(xf)
    q, s = oracle.quantize_act_dynamic(xb, qtype)
    xr = oracle.bf16_bits_to_f32(xb)
    for m in range(4):
        i = np.abs(xr[m]).argmax()
        top = 127 if qtype == "int8" else 448.0
        val = float(q[m, i]) if qtype == "int8" else float(oracle.e4m3fn_decode(q[m, i:i + 1])[0])
        assert abs(val) == top
        q1, s1 = oracle.quantize_act_dynamic(xb[m:m + 1], qtype)     # the row alone
        assert np.array_equal(q1[0], q[m]) and s1[0] == s[m]


@pytest.mark.parametrize("qtype", QTYPES)
def test_act_dynamic_power_of_two_scaling(qtype):
    # x -> 2^j x (exact in bf16) leaves the codes unchanged and scales s_x by 2^j
    _, _, x = synth.small_inputs(53, 3, 64, 1)
    xf = oracle.bf16_bits_to_f32(x)
    q0, s0 = oracle.quantize_act_dynamic(x, qtype)
    f = np.array([[2.0 ** -7], [1.0], [2.0 ** 9]], np.float32)
    q1, s1 = oracle.quantize_act_dynamic(oracle.f32_to_bf16_bits(xf * f), qtype)
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, (s0 * f[:, 0]).astype(np.float32))


def test_act_dynamic_integer_rows_scale_one():
    # integer rows whose absmax is 127 quantize to themselves at scale 1 (INT8)
    rng = np.random.default_rng(54)
    xf = rng.integers(-126, 127, size=(3, 40)).astype(np.float32)
    xf[:, 5] = [127, -127, 127]
    q, s = oracle.quantize_act_dynamic(oracle.f32_to_bf16_bits(xf), "int8")
    assert np.all(s == 1.0) and np.array_equal(q.astype(np.float32), xf)


@pytest.mark.parametrize("qtype", QTYPES)
def test_w8a8_dynamic_epilogue_bruteforce(qtype):
    w, _, x = synth.small_inputs(55, 4, 8, 6)
    gran = "per_channel" if qtype == "int8" else "per_tensor"
    q, s = oracle.quantize_weight(w, qtype, gran)
    xq, sx = oracle.quantize_act_dynamic(x, qtype)
    y = oracle.qlinear_w8a8_dynamic(xq, sx, q, s, qtype)
    for m in range(4):
        for n in range(6):
            acc = sum(_code_value(xq[m, k], qtype) * _code_value(q[n, k], qtype) for k in range(8))
            comb = exact.f32(Fraction(float(sx[m])) * Fraction(float(s[n if s.size > 1 else 0])))
            v = exact.bf16(exact.f32(exact.f32(acc) * comb))
            assert y[m, n] == exact.bf16_bits_of(v)


@pytest.mark.parametrize("qtype,gran", [("int8", "per_channel"), ("fp8_e4m3fn", "per_tensor")])
def test_w8a8_dynamic_matches_bf16_dequant_reference(qtype, gran):
    # same identity as the static scheme, with one scale per row of x
    w, _, x = synth.small_inputs(56, 64, 1024, 256)
    xf = oracle.bf16_bits_to_f32(x) * np.linspace(0.01, 50.0, 64, dtype=np.float32)[:, None]
    x = oracle.f32_to_bf16_bits(xf)
    q, s = oracle.quantize_weight(w, qtype, gran)
    xq, sx = oracle.quantize_act_dynamic(x, qtype)
    y = oracle.bf16_bits_to_f32(oracle.qlinear_w8a8_dynamic(xq, sx, q, s, qtype)).astype(np.float64)
    dec = (lambda c: c.astype(np.float64)) if qtype == "int8" else oracle.e4m3fn_decode
    xd = torch.from_numpy(dec(xq) * sx.astype(np.float64)[:, None]).to(torch.bfloat16)
    wd = torch.from_numpy(dec(q) * s.astype(np.float64).reshape(-1, 1)).to(torch.bfloat16)
    ref = (xd.float() @ wd.float().T).numpy().astype(np.float64)
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 4e-3
    rms = np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))      # per-row scale of y
    assert np.max(np.abs(y - ref) / (np.abs(ref) + rms)) < 8e-3


def test_w8a8_dynamic_accumulator_is_the_static_one():
    w, _, x = synth.small_inputs(57, 7, 128, 9)
    q, s = oracle.quantize_weight(w, "int8")
    xq, sx = oracle.quantize_act_dynamic(x, "int8")
    acc = oracle.qlinear_w8a8_dynamic(xq, sx, q, s, "int8", out="acc")
    ref = xq.astype(np.int64) @ q.astype(np.int64).T            # numpy integer matmul
    assert acc.dtype == np.int32 and np.array_equal(acc.astype(np.int64), ref)


# ---------------------------------------------------------------- routed Linear: bias and fallback
def _bias_bits(seed, N):
    rng = np.random.default_rng(seed)
    return oracle.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.5))


@pytest.mark.parametrize("scheme", ["w8a16", "w8a8_static", "w8a8_dynamic"])
@pytest.mark.parametrize("qtype", QTYPES)
def test_linear_bias_bruteforce(scheme, qtype):
    w, calib, x = synth.small_inputs(61, 3, 8, 5)
    gran = "per_tensor" if (qtype != "int8" and scheme != "w8a16") else "per_channel"
    q, s = oracle.quantize_weight(w, qtype, gran)
    sx = oracle.calibrate_input_scale(calib, qtype)
    b = _bias_bits(62, 5)
    y = oracle.linear(scheme, x, q, s, qtype, input_scale=sx, bias_bf16=b)
    xf = oracle.bf16_bits_to_f32(x)
    if scheme == "w8a8_static":
        xq, rows = oracle.quantize_act_static(x, sx, qtype), [Fraction(float(sx))] * 3
    elif scheme == "w8a8_dynamic":
        xq, sxr = oracle.quantize_act_dynamic(x, qtype)
        rows = [Fraction(float(v)) for v in sxr]
    wd = oracle.dequantize_weight_bf16(q, s, qtype)
    for m in range(3):
        for n in range(5):
            bn = Fraction(float(oracle.bf16_bits_to_f32(b[n:n + 1])[0]))
            if scheme == "w8a16":
                v = exact.f32(sum(Fraction(float(xf[m, k])) * Fraction(float(wd[n, k])) for k in range(8)))
            else:
                acc = sum(_code_value(xq[m, k], qtype) * _code_value(q[n, k], qtype) for k in range(8))
                comb = exact.f32(rows[m] * Fraction(float(s[n if s.size > 1 else 0])))
                v = exact.f32(exact.f32(acc) * comb)
            assert y[m, n] == exact.bf16_bits_of(exact.bf16(exact.f32(v + bn)))


def test_linear_zero_bias_changes_nothing_and_zero_x_gives_the_bias():
    w, calib, x = synth.small_inputs(63, 4, 64, 16)
    q, s = oracle.quantize_weight(w, "int8")
    sx = oracle.calibrate_input_scale(calib, "int8")
    zero = np.zeros(16, np.uint16)
    for scheme in ["w8a16", "w8a8_static", "w8a8_dynamic"]:
        y0 = oracle.linear(scheme, x, q, s, "int8", input_scale=sx)
        assert np.array_equal(oracle.linear(scheme, x, q, s, "int8", input_scale=sx, bias_bf16=zero), y0)
        b = _bias_bits(64, 16)
        yb = oracle.linear(scheme, np.zeros_like(x), q, s, "int8", input_scale=sx, bias_bf16=b)
        assert np.array_equal(yb, np.broadcast_to(b, yb.shape))      # bf16 bias survives exactly


def test_linear_bf16_fallback_is_the_weight_only_result_and_differs_from_w8a8():
    w, calib, x = synth.small_inputs(65, 32, 512, 64)
    q, s = oracle.quantize_weight(w, "int8")
    sx = oracle.calibrate_input_scale(calib, "int8")
    y_fb = oracle.linear("w8a8_static", x, q, s, "int8", input_scale=sx, bf16_fallback_max_m=32)
    assert np.array_equal(y_fb, oracle.qlinear_w8a16(x, q, s, "int8"))
    y_q = oracle.linear("w8a8_static", x, q, s, "int8", input_scale=sx, bf16_fallback_max_m=16)
    assert np.array_equal(y_q, oracle.qlinear_w8a8_static(oracle.quantize_act_static(x, sx, "int8"), sx, q, s, "int8"))
    assert not np.array_equal(y_fb, y_q)                               # the fallback changes the numerics
