"""GPU quantizers against the oracle: bit-exact codes and scales."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_to_gpu, codes, dev, f32_to_gpu

pytestmark = pytest.mark.gpu

QTYPES = ["int8", "fp8_e4m3fn"]


def _oracle_codes_u8(q):
    return np.asarray(q).view(np.uint8)


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("gran", ["per_channel", "per_tensor"])
@pytest.mark.parametrize("NK", [(1, 1), (7, 5), (16, 64), (33, 130), (100, 1000), (257, 2048)])
def test_quantize_weight_bit_exact(qtype, gran, NK):
    N, K = NK
    print(f"quantize_weight {qtype} {gran} N={N} K={K}", flush=True)
    w, _, _ = synth.small_inputs(100 + N + K, 1, K, N)
    qw = qlq.quantize_weight(f32_to_gpu(w), qtype, gran)
    q_ref, s_ref = oracle.quantize_weight(w, qtype, gran)
    torch.cuda.synchronize()
    assert np.array_equal(qw.scale.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(codes(qlq.unpack_weight(qw)), _oracle_codes_u8(q_ref))


@pytest.mark.parametrize("qtype", QTYPES)
def test_quantize_weight_bf16_input_and_zero_rows(qtype):
    w, _, _ = synth.small_inputs(5, 1, 200, 48)
    w[3] = 0.0
    wb = synth.f32_to_bf16_bits(w)
    qw = qlq.quantize_weight(bf16_to_gpu(wb), qtype)
    q_ref, s_ref = oracle.quantize_weight(wb, qtype, w_is_bf16=True)
    assert np.array_equal(qw.scale.cpu().numpy(), s_ref) and s_ref[3] == 1.0
    assert np.array_equal(codes(qlq.unpack_weight(qw)), _oracle_codes_u8(q_ref))


@pytest.mark.parametrize("name", list(synth.CASES))
def test_quantize_weight_full_size_bit_exact(name):
    c = synth.CASES[name]
    print(f"quantize_weight full {name}", flush=True)
    inp = synth.case_inputs(c)
    qw = qlq.quantize_weight(f32_to_gpu(inp.w), c.qtype, c.granularity)
    q_ref, s_ref = oracle.quantize_weight(inp.w, c.qtype, c.granularity)
    assert np.array_equal(qw.scale.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(codes(qlq.unpack_weight(qw)), _oracle_codes_u8(q_ref))


@pytest.mark.parametrize("qtype", QTYPES)
def test_calibrate_input_scale_bit_exact(qtype):
    for numel_shape in [(1, 1), (64, 2048), (64, 11008), (3, 77)]:
        _, calib, _ = synth.small_inputs(7, 1, numel_shape[1], 1)
        calib = calib[: numel_shape[0]] if numel_shape[0] <= 64 else calib
        s = qlq.calibrate_input_scale(bf16_to_gpu(calib), qtype)
        ref = oracle.calibrate_input_scale(calib, qtype)
        assert s.cpu().numpy()[0].view(np.uint32) == np.float32(ref).view(np.uint32)
    zero = torch.zeros(5, 9, dtype=torch.bfloat16, device=dev())
    assert qlq.calibrate_input_scale(zero, qtype).item() == 1.0


@pytest.mark.parametrize("qtype", QTYPES)
def test_quantize_act_exhaustive_bf16_patterns(qtype):
    # every finite bf16 value, at an awkward scale (the IEEE division) and at calibrated scales
    # fp32(a / qmax) for bf16 a (1 = 127 / 127 among them), which take the refined-reciprocal
    # division: tiny, huge and ordinary a, both qmax, so most x lie far beyond the absmax
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f32(allb)
    fin = allb[np.isfinite(vals)]
    x = np.concatenate([fin, np.zeros((-fin.size) % 256, np.uint16)]).reshape(-1, 256)
    calibrated = [oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(np.array([a], np.float32)))[0] / np.float32(q)
                  for a, q in [(3.0, 127), (0.07, 448), (1e-28, 127), (3e38, 448), (0.5, 448), (448.0, 127)]]
    for s in [1.0, float(np.float32(0.0123456))] + [float(np.float32(c)) for c in calibrated]:
        got = codes(qlq.quantize_act_static(bf16_to_gpu(x), s, qtype))
        ref = oracle.quantize_act_static(x, np.float32(s), qtype).view(np.uint8)
        assert np.array_equal(got, ref), f"scale {s}: {np.count_nonzero(got != ref)} codes differ"


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("MK", [(1, 1), (3, 7), (256, 11008), (1024, 2048), (5, 1001)])
def test_quantize_act_bit_exact(qtype, MK):
    M, K = MK
    _, calib, x = synth.small_inputs(11 + M, M, K, 1)
    s = oracle.calibrate_input_scale(calib, qtype)
    got = codes(qlq.quantize_act_static(bf16_to_gpu(x), float(s), qtype))
    ref = oracle.quantize_act_static(x, s, qtype).view(np.uint8)
    assert np.array_equal(got, ref)


def test_quantize_act_unaligned_view():
    # an offset view (not 16-byte aligned) takes the element-by-element path
    _, _, x = synth.small_inputs(12, 9, 33, 1)
    xg = bf16_to_gpu(x).reshape(-1)[1:].contiguous()
    base = torch.empty(xg.numel() + 1, dtype=torch.bfloat16, device=dev())
    base[1:] = xg
    view = base[1:].view(1, -1)
    got = codes(qlq.quantize_act_static(view, 0.05, "int8"))
    ref = oracle.quantize_act_static(x.reshape(-1)[1:].reshape(1, -1), np.float32(0.05), "int8").view(np.uint8)
    assert np.array_equal(got, ref)
