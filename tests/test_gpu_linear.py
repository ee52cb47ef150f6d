"""GPU routed Linear (bias epilogue, W8A8 small-batch BF16 fallback) against the oracle.

INT8 W8A8 outputs are compared bit for bit (the bias is a separately rounded
fp32 add on both sides); W8A16 and FP8 outputs within relL2 <= 4e-3 and
|err| <= 8e-3 (|ref| + rms(ref)).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_bits, bf16_to_gpu, bits_to_f64, check_close, f32_to_gpu

pytestmark = pytest.mark.gpu

# the last shape takes several 16-column tiles per small-M workgroup (the bias epilogue per tile)
SHAPES = [(1, 64, 16), (3, 100, 37), (16, 2048, 2048), (13, 1000, 300), (17, 640, 200), (64, 128, 4096),
          (255, 1024, 136), (257, 320, 250), (256, 2048, 1024), (130, 4096, 96), (37, 1000, 300),
          (300, 100, 1100), (13, 704, 10338)]


def _case(seed, M, K, N, qtype, scheme):
    gran = "per_tensor" if (qtype != "int8" and scheme != "w8a16") else "per_channel"
    w, calib, x = synth.small_inputs(seed, M, K, N)
    qw = qlq.quantize_weight(f32_to_gpu(w), qtype, gran)
    q_ref, s_ref = oracle.quantize_weight(w, qtype, gran)
    sx = oracle.calibrate_input_scale(calib, qtype)
    rng = np.random.default_rng(seed + 1)
    b = oracle.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    return x, qw, q_ref, s_ref, sx, b


def _compare(y, ref, exact_int8, what):
    if exact_int8:
        assert np.array_equal(y, ref), what
    else:
        check_close(bits_to_f64(y), bits_to_f64(ref), what)


@pytest.mark.parametrize("scheme", ["w8a16", "w8a8_static", "w8a8_dynamic"])
@pytest.mark.parametrize("qtype", ["int8", "fp8_e4m3fn"])
@pytest.mark.parametrize("MKN", SHAPES)
def test_linear_with_bias(scheme, qtype, MKN):
    M, K, N = MKN
    print(f"linear {scheme} {qtype} M={M} K={K} N={N}", flush=True)
    x, qw, q_ref, s_ref, sx, b = _case(900 + M + K + N, M, K, N, qtype, scheme)
    y = bf16_bits(qlq.linear(scheme, bf16_to_gpu(x), qw, float(sx), bias=bf16_to_gpu(b)))
    ref = oracle.linear(scheme, x, q_ref, s_ref, qtype, input_scale=sx, bias_bf16=b)
    _compare(y, ref, scheme != "w8a16" and qtype == "int8", f"{scheme} {qtype} {MKN}")
    # without a bias the routed call equals the oracle's plain scheme
    y0 = bf16_bits(qlq.linear(scheme, bf16_to_gpu(x), qw, float(sx)))
    _compare(y0, oracle.linear(scheme, x, q_ref, s_ref, qtype, input_scale=sx), scheme != "w8a16" and qtype == "int8",
             f"{scheme} {qtype} {MKN} no bias")


@pytest.mark.parametrize("scheme", ["w8a8_static", "w8a8_dynamic"])
def test_linear_bf16_fallback(scheme):
    for M in [1, 16, 32, 33, 64]:
        print(f"fallback {scheme} M={M}", flush=True)
        x, qw, q_ref, s_ref, sx, b = _case(950 + M, M, 512, 96, "int8", scheme)
        y = bf16_bits(qlq.linear(scheme, bf16_to_gpu(x), qw, float(sx), bias=bf16_to_gpu(b), bf16_fallback_max_m=32))
        ref = oracle.linear(scheme, x, q_ref, s_ref, "int8", input_scale=sx, bias_bf16=b, bf16_fallback_max_m=32)
        _compare(y, ref, M > 32, f"fallback {scheme} M={M}")


def test_linear_full_size_stack_shapes():
    # the 3B stack's q/k/v-like shape with a bias, at decode and prefill sizes
    rng = np.random.default_rng(77)
    for M, K, N in [(1, 2048, 2048), (1024, 2048, 2048), (256, 11008, 2048)]:
        print(f"linear full M={M} K={K} N={N}", flush=True)
        w = (rng.standard_normal((N, K), dtype=np.float32) * 0.02).astype(np.float32)
        x = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
        b = oracle.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.1))
        qw = qlq.quantize_weight(f32_to_gpu(w), "int8")
        q_ref, s_ref = oracle.quantize_weight(w, "int8")
        y = bf16_bits(qlq.linear("w8a8_dynamic", bf16_to_gpu(x), qw, bias=bf16_to_gpu(b)))
        assert np.array_equal(y, oracle.linear("w8a8_dynamic", x, q_ref, s_ref, "int8", bias_bf16=b))
        y = bf16_bits(qlq.linear("w8a16", bf16_to_gpu(x), qw, bias=bf16_to_gpu(b)))
        check_close(bits_to_f64(y), bits_to_f64(oracle.linear("w8a16", x, q_ref, s_ref, "int8", bias_bf16=b)))


def test_graph_replay_of_the_widened_rows():
    # one HIP graph holding a routed per-token Linear with a bias (a large-M split-K plan and a
    # small-M split-K plan), a fused static call and a KV-cache round trip; eager calls on the
    # same workspace run between the replays, and every replay must equal the eager results
    dev = torch.device("cuda:0")
    cases = []
    for i, (M, K, N) in enumerate([(256, 11008, 256), (1, 8192, 1024)]):
        x, qw, q_ref, s_ref, sx, b = _case(1400 + i, M, K, N, "int8", "w8a8_dynamic")
        cases.append((bf16_to_gpu(x), qw, bf16_to_gpu(b), float(sx)))
    ws = torch.zeros(1 << 26, dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(5)
    kv = [bf16_to_gpu(oracle.f32_to_bf16_bits(rng.standard_normal((64, 4, 128)).astype(np.float32))) for _ in range(2)]

    def work(outs):
        for (x, qw, b, sx), o in zip(cases, outs[:2]):
            qlq.linear("w8a8_dynamic", x, qw, bias=b, out=o, workspace=ws)
        x, qw, b, sx = cases[0]
        qlq.qlinear_w8a8_static_fused(x, sx, qw, out=outs[2], workspace=ws)
        q = qlq.kv_quantize(kv[0], kv[1])
        qlq.kv_dequantize(q, outs[3], outs[4])

    outs = [torch.empty((256, 256), dtype=torch.bfloat16, device=dev), torch.empty((1, 1024), dtype=torch.bfloat16,
            device=dev), torch.empty((256, 256), dtype=torch.bfloat16, device=dev), torch.empty_like(kv[0]),
            torch.empty_like(kv[1])]
    work(outs)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work(outs)
    for rep in range(4):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep}"
        # eager split-K work on the same workspace between replays
        x, qw, b, sx = cases[1]
        qlq.linear("w8a8_dynamic", x, qw, bias=b, workspace=ws)
        torch.cuda.synchronize()
