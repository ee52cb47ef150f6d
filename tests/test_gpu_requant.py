"""GPU parity of the static W8A8 GEMM that also quantizes its bf16 output for the
next static layer (qlq_qlinear_w8a8_static_requant).

The expected values are the oracle's composition: its W8A8 static output y, then
its quantize_act_static(y, next_scale).
* INT8: y and the next layer's codes bit for bit.
* FP8: y within relL2 <= 4e-3 and |err| <= 8e-3 (|ref| + rms(ref)).  FP8
  accumulation order leaves several correct bf16 outputs, so the codes must equal
  the oracle's wherever the two outputs agree bit for bit; elsewhere each code must
  decode to within that output tolerance (over next_scale) plus one e4m3 step of
  the oracle's y / next_scale (clamped to +-448), i.e. be a valid code of a valid y.
Both qtypes: the codes are identical to the separate quantize_act_static pass over
the same call's y (two GPU paths, one result), also along a three-layer chain.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_bits, bf16_to_gpu, bits_to_f64, check_close, codes, f32_to_gpu

pytestmark = pytest.mark.gpu

QTYPES = ["int8", "fp8_e4m3fn"]
# small-M kernel (4/8/16 waves, split-K, unaligned N, several 16-row groups with and without
# split-K), direct-to-LDS kernel (staged and direct epilogues, split-K), register-staged kernel
# (K not a multiple of 64, with and without split-K)
SHAPES = [(1, 1, 1), (1, 2048, 1024), (1, 2048, 2048), (3, 100, 37), (16, 640, 200), (16, 11008, 128),
          (64, 128, 4096), (20, 8192, 1024), (130, 4096, 96), (255, 1024, 136), (257, 320, 250), (256, 11008, 256),
          (1024, 2048, 1024), (130, 1000, 96), (40, 200, 64), (300, 2000, 300),
          # plans of the 3B-scale stack's chain: small-M without split (4 waves) and with split
          # (8 / 16 waves), two 16-column tiles per workgroup (up projection at M = 16), and
          # the 256x192 tile the up projection takes at M = 1024
          (1, 2048, 11008), (16, 11008, 2048), (16, 2048, 11008), (768, 512, 11008)]


def _e4m3_step(v: np.ndarray) -> np.ndarray:
    """Spacing of e4m3fn values around |v| (3 mantissa bits; 2^-9 below the normal range)."""
    a = np.maximum(np.abs(v), 2.0 ** -6)
    return 2.0 ** (np.floor(np.log2(a)) - 3)


def _case(seed, M, K, N, qtype):
    w, calib, x = synth.small_inputs(seed, M, K, N)
    gran = "per_tensor" if qtype == "fp8_e4m3fn" else "per_channel"
    qw = qlq.quantize_weight(f32_to_gpu(w), qtype, gran)
    q_ref, s_ref = oracle.quantize_weight(w, qtype, gran)
    sx = oracle.calibrate_input_scale(calib, qtype)
    xq_ref = oracle.quantize_act_static(x, sx, qtype)
    xq = qlq.quantize_act_static(bf16_to_gpu(x), float(sx), qtype)
    return qw, q_ref, s_ref, sx, xq, xq_ref


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("MKN", SHAPES)
@pytest.mark.parametrize("scale_kind", ["calibrated", "saturating"])
def test_requant_parity(qtype, MKN, scale_kind):
    M, K, N = MKN
    print(f"requant {qtype} {scale_kind} M={M} K={K} N={N}", flush=True)
    qw, q_ref, s_ref, sx, xq, xq_ref = _case(3100 + 7 * M + K + N, M, K, N, qtype)
    y_ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, qtype)
    # the next layer's scale: calibrated on the oracle's output, or a quarter of it so
    # that a good share of the codes saturate
    s_next = oracle.calibrate_input_scale(y_ref, qtype)
    if scale_kind == "saturating":
        s_next = np.float32(s_next * np.float32(0.25))
    c_ref = oracle.quantize_act_static(y_ref, s_next, qtype).view(np.uint8)
    y, c = qlq.qlinear_w8a8_static_requant(xq, float(sx), qw, float(s_next))
    yb, cb = bf16_bits(y), codes(c)
    if qtype == "int8":
        assert np.array_equal(yb, y_ref)
        assert np.array_equal(cb, c_ref)
    else:
        check_close(bits_to_f64(yb), bits_to_f64(y_ref), "fp8 requant y")
        same = yb == y_ref
        assert np.array_equal(cb[same], c_ref[same])
        yr = bits_to_f64(y_ref)
        tol = 8e-3 * (np.abs(yr) + np.sqrt(np.mean(yr ** 2))) / np.float64(s_next)
        target = np.clip(yr / np.float64(s_next), -448.0, 448.0)
        got = oracle.e4m3fn_decode(cb).astype(np.float64)
        assert np.all(np.abs(got - target) <= tol + _e4m3_step(target))
    # the separate pass over the same y writes the same codes, and y is the plain call's
    again = qlq.quantize_act_static(y, float(s_next), qtype)
    assert np.array_equal(codes(again), cb)
    plain = qlq.qlinear_w8a8_static(xq, float(sx), qw)
    assert np.array_equal(bf16_bits(plain), yb)


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M", [1, 16, 256])
def test_requant_chain_matches_separate_passes(qtype, M):
    # q -> up -> down of the 3B-scale stack's shapes, each layer's codes from the previous epilogue
    print(f"requant chain {qtype} M={M}", flush=True)
    dims = [(2048, 2048), (2048, 11008), (11008, 2048)]
    rng = np.random.default_rng(71 + M)
    gran = "per_tensor" if qtype == "fp8_e4m3fn" else "per_channel"
    ws = [qlq.quantize_weight(f32_to_gpu((rng.standard_normal((n, k), dtype=np.float32) * 0.02)), qtype, gran)
          for k, n in dims]
    x = bf16_to_gpu(synth.f32_to_bf16_bits(rng.standard_normal((M, 2048), dtype=np.float32)))
    scales = [0.03, 0.011, 0.017, 0.02]                        # input scales of layers 0..2, then the next one
    xq = qlq.quantize_act_static(x, scales[0], qtype)
    xq_sep = xq.clone()
    for layer, qw in enumerate(ws):
        y, c = qlq.qlinear_w8a8_static_requant(xq, scales[layer], qw, scales[layer + 1])
        y_sep = qlq.qlinear_w8a8_static(xq_sep, scales[layer], qw)
        assert torch.equal(y, y_sep), f"layer {layer}"
        xq_sep = qlq.quantize_act_static(y_sep, scales[layer + 1], qtype)
        assert torch.equal(c, xq_sep), f"layer {layer}"
        xq = c
    torch.cuda.synchronize()
