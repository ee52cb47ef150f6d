"""GPU parity of the widened rows: dynamic per-token activation quantization with
its W8A8 GEMM, and the static W8A8 GEMM fed bf16 x (quantization fused in).

Codes and per-token scales are compared bit for bit with the oracle; INT8
accumulators and INT8 outputs bit for bit; FP8 outputs within relL2 <= 4e-3 and
|err| <= 8e-3 (|ref| + rms(ref)), with rms taken per row for the per-token
scheme (rows are scaled independently).
"""
import numpy as np
import pytest

import oracle
import synth
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_bits, bf16_to_gpu, bits_to_f64, check_close, codes, f32_to_gpu

pytestmark = pytest.mark.gpu

QTYPES = ["int8", "fp8_e4m3fn"]
# small-M kernel (with one and with several 16-column tiles per workgroup, and several 16-row
# groups with and without K slices), direct-to-LDS kernel (K % 64 == 0), register-staged kernel
# (ragged K), split-K plans, tails in every dimension
SHAPES = [(1, 1, 1), (1, 64, 16), (2, 5, 3), (1, 2048, 2048), (3, 100, 37), (16, 640, 200), (13, 1000, 300),
          (16, 11008, 128), (17, 640, 200), (31, 512, 129), (64, 128, 4096), (255, 1024, 136), (257, 320, 250),
          (130, 4096, 96), (37, 1000, 300), (300, 100, 1100), (13, 704, 10338), (20, 8192, 1024)]


def _rows_spread(x_bits, seed):
    """Give the rows of x very different magnitudes (powers of two keep bf16 exact) and zero one row."""
    xf = oracle.bf16_bits_to_f32(x_bits)
    rng = np.random.default_rng(seed)
    xf = xf * (2.0 ** rng.integers(-12, 12, size=(xf.shape[0], 1))).astype(np.float32)
    if xf.shape[0] > 2:
        xf[1] = 0.0
    return oracle.f32_to_bf16_bits(xf)


def _check_rows(got_bits, ref_bits, what):
    g, r = bits_to_f64(got_bits), bits_to_f64(ref_bits)
    assert np.all(np.isfinite(g)), what
    nz = np.linalg.norm(r, axis=1) > 0
    assert np.array_equal(g[~nz], r[~nz]), what          # an all-zero row gives zeros
    for m in np.nonzero(nz)[0]:
        check_close(g[m], r[m], f"{what} row {m}")


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("MK", [(1, 1), (1, 2048), (4, 7), (16, 2048), (5, 1000), (256, 11008), (1024, 2048),
                                (3, 8), (64, 4104),
                                # many rows: a wave per row up to K = 4096, a workgroup per row above
                                (1030, 4096), (1024, 11008), (1100, 5000)])
def test_quantize_act_dynamic_bit_exact(qtype, MK):
    M, K = MK
    print(f"act dynamic {qtype} M={M} K={K}", flush=True)
    _, _, x = synth.small_inputs(600 + M + K, M, K, 1)
    x = _rows_spread(x, M * 31 + K)
    xq, sx = qlq.quantize_act_dynamic(bf16_to_gpu(x), qtype)
    q_ref, s_ref = oracle.quantize_act_dynamic(x, qtype)
    assert np.array_equal(sx.cpu().numpy(), s_ref)
    assert np.array_equal(codes(xq), q_ref.view(np.uint8))


def _rows_below(abits: int, K: int) -> np.ndarray:
    """bf16 rows of K whose absmax is a (the bf16 value with bits `abits`), together holding every
    bf16 x with |x| <= a, both signs."""
    mags = np.arange(0, abits + 1, dtype=np.uint16)
    xs = np.concatenate([mags, mags | np.uint16(0x8000)])
    n = -(-xs.size // (K - 1))
    rows = np.zeros((n, K), np.uint16)
    rows[:, 0] = abits
    fill = np.zeros(n * (K - 1), np.uint16)
    fill[:xs.size] = xs
    rows[:, 1:] = fill.reshape(n, K - 1)
    return rows


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("part", range(2))
def test_quantize_act_dynamic_every_bf16_below_absmax(qtype, part):
    # The per-token quantizer divides by its row scale with a refined reciprocal above 2^-100 and
    # by the IEEE division below: every bf16 x with |x| <= absmax, for absmax values across the
    # bf16 range (subnormals, whose scales take the IEEE branch, every fourth binade, the largest
    # finite value), against the oracle's IEEE division, codes and scales bit for bit.
    abits_all = [0x0001, 0x0003, 0x007F, 0x0A00, 0x0C9A] + [(e << 7) | m for e in range(1, 255, 4)
                                                            for m in (0x00, 0x2B, 0x7F)] + [0x7F7F]
    abits = abits_all[part::2]
    print(f"act dynamic every x below absmax {qtype}: part {part}, {len(abits)} absmax values", flush=True)
    x = np.concatenate([_rows_below(a, 4096) for a in abits])
    xq, sx = qlq.quantize_act_dynamic(bf16_to_gpu(x), qtype)
    q_ref, s_ref = oracle.quantize_act_dynamic(x, qtype)
    assert np.array_equal(sx.cpu().numpy(), s_ref)
    assert np.array_equal(codes(xq), q_ref.view(np.uint8))


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("MKN", SHAPES)
def test_w8a8_dynamic_parity(qtype, MKN):
    M, K, N = MKN
    print(f"w8a8 dynamic {qtype} M={M} K={K} N={N}", flush=True)
    gran = "per_channel" if qtype == "int8" else "per_tensor"
    w, _, x = synth.small_inputs(700 + M * 5 + K + N, M, K, N)
    x = _rows_spread(x, M + 3 * N)
    qw = qlq.quantize_weight(f32_to_gpu(w), qtype, gran)
    q_ref, s_ref = oracle.quantize_weight(w, qtype, gran)
    xq_ref, sx_ref = oracle.quantize_act_dynamic(x, qtype)
    xq, sx = qlq.quantize_act_dynamic(bf16_to_gpu(x), qtype)
    assert np.array_equal(codes(xq), xq_ref.view(np.uint8)) and np.array_equal(sx.cpu().numpy(), sx_ref)
    acc = qlq.qlinear_w8a8_dynamic(xq, sx, qw, "acc").cpu().numpy()
    acc_ref = oracle.qlinear_w8a8_dynamic(xq_ref, sx_ref, q_ref, s_ref, qtype, out="acc")
    y = bf16_bits(qlq.qlinear_w8a8_dynamic(xq, sx, qw))
    y_ref = oracle.qlinear_w8a8_dynamic(xq_ref, sx_ref, q_ref, s_ref, qtype)
    if qtype == "int8":
        assert np.array_equal(acc, acc_ref)
        assert np.array_equal(y, y_ref)
    else:
        check_close(acc, acc_ref, f"dynamic acc {MKN}")
        _check_rows(y, y_ref, f"dynamic {MKN}")


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("MKN", SHAPES + [(1, 11008, 2048), (16, 2048, 11008)])
def test_w8a8_static_fused_parity(qtype, MKN):
    M, K, N = MKN
    print(f"w8a8 static fused {qtype} M={M} K={K} N={N}", flush=True)
    gran = "per_channel" if qtype == "int8" else "per_tensor"
    w, calib, x = synth.small_inputs(800 + M * 3 + K + N, M, K, N)
    qw = qlq.quantize_weight(f32_to_gpu(w), qtype, gran)
    q_ref, s_ref = oracle.quantize_weight(w, qtype, gran)
    sx = oracle.calibrate_input_scale(calib, qtype)
    xq_ref = oracle.quantize_act_static(x, sx, qtype)
    xg = bf16_to_gpu(x)
    acc = qlq.qlinear_w8a8_static_fused(xg, float(sx), qw, "acc").cpu().numpy()
    acc_ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, qtype, out="acc")
    y = bf16_bits(qlq.qlinear_w8a8_static_fused(xg, float(sx), qw))
    y_ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, qtype)
    if qtype == "int8":
        assert np.array_equal(acc, acc_ref)
        assert np.array_equal(y, y_ref)
    else:
        check_close(acc, acc_ref, f"fused acc {MKN}")
        check_close(bits_to_f64(y), bits_to_f64(y_ref), f"fused {MKN}")
    # same codes as the two-call path, so the GPU results agree bit for bit too
    y2 = bf16_bits(qlq.qlinear_w8a8_static(qlq.quantize_act_static(xg, float(sx), qtype), float(sx), qw))
    assert np.array_equal(y, y2)


def test_w8a8_static_fused_saturating_codes():
    # activations far beyond the calibrated range saturate inside the fused kernel as in the quantizer
    M, K, N = 4, 256, 32
    w, _, x = synth.small_inputs(901, M, K, N)
    xf = oracle.bf16_bits_to_f32(x) * np.float32(64.0)
    x = oracle.f32_to_bf16_bits(xf)
    for qtype in QTYPES:
        qw = qlq.quantize_weight(f32_to_gpu(w), qtype)
        q_ref, s_ref = oracle.quantize_weight(w, qtype)
        sx = np.float32(0.01)
        xq_ref = oracle.quantize_act_static(x, sx, qtype)
        acc = qlq.qlinear_w8a8_static_fused(bf16_to_gpu(x), float(sx), qw, "acc").cpu().numpy()
        acc_ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, qtype, out="acc")
        if qtype == "int8":
            assert np.array_equal(acc, acc_ref)
        else:
            check_close(acc, acc_ref, "fused saturation")


@pytest.mark.parametrize("cfg", [("int8", 256, 11008, 2048), ("fp8_e4m3fn", 1024, 2048, 11008),
                                 ("fp8_e4m3fn", 16, 2048, 11008), ("int8", 1, 2048, 2048)])
def test_dynamic_full_size(cfg):
    qtype, M, K, N = cfg
    print(f"dynamic full size {cfg}", flush=True)
    c = synth.CASES[{"int8": "int8_w8a8_256x11008x2048", "fp8_e4m3fn": "fp8_w8a8_1024x2048x11008"}[qtype]]
    rng = np.random.default_rng(M + K + N)
    w = (rng.standard_normal((N, K), dtype=np.float32) * 0.02).astype(np.float32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    gran = c.granularity
    qw = qlq.quantize_weight(f32_to_gpu(w), qtype, gran)
    q_ref, s_ref = oracle.quantize_weight(w, qtype, gran)
    xq, sx = qlq.quantize_act_dynamic(bf16_to_gpu(x), qtype)
    xq_ref, sx_ref = oracle.quantize_act_dynamic(x, qtype)
    assert np.array_equal(codes(xq), xq_ref.view(np.uint8)) and np.array_equal(sx.cpu().numpy(), sx_ref)
    y = bf16_bits(qlq.qlinear_w8a8_dynamic(xq, sx, qw))
    y_ref = oracle.qlinear_w8a8_dynamic(xq_ref, sx_ref, q_ref, s_ref, qtype)
    if qtype == "int8":
        assert np.array_equal(y, y_ref)
    else:
        check_close(bits_to_f64(y), bits_to_f64(y_ref), f"dynamic full {cfg}")
