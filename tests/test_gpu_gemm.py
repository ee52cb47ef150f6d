"""GPU GEMMs against the oracle on small and ragged sizes (several tiles plus a tail).

W8A8 INT8 accumulators and outputs are compared bit for bit; W8A16 and FP8 W8A8
outputs within relL2 <= 4e-3 and |err| <= 8e-3 (|ref| + rms(ref)).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_bits, bf16_to_gpu, bits_to_f64, check_close, codes, dev, f32_to_gpu

pytestmark = pytest.mark.gpu

QTYPES = ["int8", "fp8_e4m3fn"]
# (M, K, N): decode and prefill sizes, tails in every dimension, split-K cases.  The small-M
# plans include 4, 8 and 16 waves per workgroup (e.g. (4, 4096, 8192): 8 waves, no split;
# (1, 16384, 1024): 16 waves, two K slices; (2, 2048, 11008): 4 waves), and the aligned path's
# every count of 1 to 8 K units per wave, for one and two 64-input tiles per unit (the K = 64 * odd
# case (1, 1728, 2060) leaves the last FP8 W8A8 unit half past the end of K); M > 16 with K not a
# multiple of 64 takes the register-staged kernel, with K slices (37, 1000, 300) and without
# (300, 100, 1100).
SHAPES = [(1, 1, 1), (1, 64, 16), (2, 5, 3), (8, 8, 8), (1, 2048, 2048), (3, 100, 37), (16, 640, 200),
          (13, 1000, 300), (16, 11008, 128), (17, 640, 200), (31, 512, 129), (33, 256, 64), (64, 128, 4096),
          (255, 1024, 136), (257, 320, 250), (130, 4096, 96), (128, 64, 128), (4, 4096, 8192), (5, 4096, 1024),
          (2, 2048, 11008), (512, 512, 1024), (3, 1792, 2060), (7, 1408, 2060), (9, 1280, 2060),
          (2, 3584, 2060), (11, 2816, 2060), (6, 2560, 2060), (1, 1728, 2060), (1, 16384, 1024),
          (5, 1152, 2060), (37, 1000, 300), (300, 100, 1100)]


def _prep(seed, M, K, N, qtype, gran="per_channel"):
    w, calib, x = synth.small_inputs(seed, M, K, N)
    qw = qlq.quantize_weight(f32_to_gpu(w), qtype, gran)
    q_ref, s_ref = oracle.quantize_weight(w, qtype, gran)
    return w, calib, x, qw, q_ref, s_ref


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("MKN", SHAPES)
def test_w8a16_parity(qtype, MKN):
    M, K, N = MKN
    print(f"w8a16 {qtype} M={M} K={K} N={N}", flush=True)
    _, _, x, qw, q_ref, s_ref = _prep(1000 + M * 7 + K + N, M, K, N, qtype)
    y = qlq.qlinear_w8a16(bf16_to_gpu(x), qw)
    ref = oracle.qlinear_w8a16(x, q_ref, s_ref, qtype)
    check_close(bits_to_f64(bf16_bits(y)), bits_to_f64(ref), f"w8a16 {qtype} {MKN}")


@pytest.mark.parametrize("qtype", QTYPES)
def test_w8a16_per_tensor_scale(qtype):
    M, K, N = 20, 256, 80
    _, _, x, qw, q_ref, s_ref = _prep(3, M, K, N, qtype, "per_tensor")
    y = qlq.qlinear_w8a16(bf16_to_gpu(x), qw)
    ref = oracle.qlinear_w8a16(x, q_ref, s_ref, qtype)
    check_close(bits_to_f64(bf16_bits(y)), bits_to_f64(ref))


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M", [1, 16, 64])
def test_w8a16_one_hot_gives_dequantized_weight_exactly(qtype, M):
    K, N = 192, 48
    w, _, _ = synth.small_inputs(4, 1, K, N)
    qw = qlq.quantize_weight(f32_to_gpu(w), qtype)
    q_ref, s_ref = oracle.quantize_weight(w, qtype)
    wd = oracle.dequantize_weight_bf16(q_ref, s_ref, qtype)
    ks = np.arange(M) * 3 % K
    x = np.zeros((M, K), np.float32)
    x[np.arange(M), ks] = 1.0
    y = bf16_bits(qlq.qlinear_w8a16(bf16_to_gpu(oracle.f32_to_bf16_bits(x)), qw))
    assert np.array_equal(y, oracle.f32_to_bf16_bits(wd[:, ks].T.copy()))


def test_w8a16_fp8_all_codes_decode_exactly():
    # per-tensor scale 1 (absmax 448): every finite e4m3fn value as a weight
    vals = oracle.e4m3fn_decode(np.arange(256, dtype=np.uint8))
    vals = vals[np.isfinite(vals)].astype(np.float32)
    W = vals.reshape(-1, 1).repeat(64, axis=1)        # [254, 64]
    qw = qlq.quantize_weight(f32_to_gpu(W), "fp8_e4m3fn", "per_tensor")
    assert qw.scale.item() == 1.0
    x = np.zeros((1, 64), np.float32)
    x[0, 5] = 1.0
    y = bf16_bits(qlq.qlinear_w8a16(bf16_to_gpu(oracle.f32_to_bf16_bits(x)), qw))
    assert np.array_equal(bits_to_f64(y)[0], vals.astype(np.float64))


def test_w8a16_integer_exact():
    rng = np.random.default_rng(5)
    M, K, N = 24, 128, 40
    W = rng.integers(-127, 128, (N, K)).astype(np.float32)
    W[:, 0] = 127
    X = rng.integers(-4, 5, (M, K)).astype(np.float32)
    qw = qlq.quantize_weight(f32_to_gpu(W), "int8")
    y = bf16_bits(qlq.qlinear_w8a16(bf16_to_gpu(oracle.f32_to_bf16_bits(X)), qw))
    ref = oracle.f32_to_bf16_bits((X.astype(np.int64) @ W.astype(np.int64).T).astype(np.float32))
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("MKN", SHAPES)
def test_w8a8_int8_bit_exact(MKN):
    M, K, N = MKN
    print(f"w8a8 int8 M={M} K={K} N={N}", flush=True)
    _, calib, x, qw, q_ref, s_ref = _prep(2000 + M * 7 + K + N, M, K, N, "int8")
    sx = oracle.calibrate_input_scale(calib, "int8")
    xq_ref = oracle.quantize_act_static(x, sx, "int8")
    xq = qlq.quantize_act_static(bf16_to_gpu(x), float(sx), "int8")
    assert np.array_equal(codes(xq), xq_ref.view(np.uint8))
    acc = qlq.qlinear_w8a8_static(xq, float(sx), qw, "acc").cpu().numpy()
    acc_ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, "int8", out="acc")
    assert np.array_equal(acc, acc_ref)
    y = bf16_bits(qlq.qlinear_w8a8_static(xq, float(sx), qw, "bf16"))
    assert np.array_equal(y, oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, "int8"))


@pytest.mark.parametrize("gran", ["per_tensor", "per_channel"])
@pytest.mark.parametrize("MKN", SHAPES)
def test_w8a8_fp8_parity(MKN, gran):
    M, K, N = MKN
    print(f"w8a8 fp8 {gran} M={M} K={K} N={N}", flush=True)
    _, calib, x, qw, q_ref, s_ref = _prep(3000 + M * 7 + K + N, M, K, N, "fp8_e4m3fn", gran)
    sx = oracle.calibrate_input_scale(calib, "fp8_e4m3fn")
    xq_ref = oracle.quantize_act_static(x, sx, "fp8_e4m3fn")
    xq = qlq.quantize_act_static(bf16_to_gpu(x), float(sx), "fp8_e4m3fn")
    assert np.array_equal(codes(xq), xq_ref)
    acc = qlq.qlinear_w8a8_static(xq, float(sx), qw, "acc").cpu().numpy()
    acc_ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, "fp8_e4m3fn", out="acc")
    check_close(acc, acc_ref, "fp8 acc")
    y = bf16_bits(qlq.qlinear_w8a8_static(xq, float(sx), qw, "bf16"))
    ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, "fp8_e4m3fn")
    check_close(bits_to_f64(y), bits_to_f64(ref), "fp8 y")


def test_w8a8_fp8_integer_exact():
    rng = np.random.default_rng(6)
    M, K, N = 40, 256, 24
    W = rng.integers(-16, 17, (N, K)).astype(np.float32)
    W[0, 0] = 448.0
    X = rng.integers(-8, 9, (M, K)).astype(np.float32)
    qw = qlq.quantize_weight(f32_to_gpu(W), "fp8_e4m3fn", "per_tensor")
    xq = qlq.quantize_act_static(bf16_to_gpu(oracle.f32_to_bf16_bits(X)), 1.0, "fp8_e4m3fn")
    acc = qlq.qlinear_w8a8_static(xq, 1.0, qw, "acc").cpu().numpy()
    assert np.array_equal(acc.astype(np.float64), X.astype(np.float64) @ W.astype(np.float64).T)


@pytest.mark.parametrize("scheme", ["w8a16", "w8a8_static"])
def test_split_k_workspace_is_reusable(scheme):
    # repeated split-K calls on one workspace give identical results
    M, K, N = (1, 8192, 1024) if scheme == "w8a16" else (256, 11008, 256)
    assert qlq.workspace_bytes(scheme, M, K, N, "int8") > 0
    _, calib, x, qw, q_ref, s_ref = _prep(77, M, K, N, "int8")
    xg = bf16_to_gpu(x)
    if scheme == "w8a16":
        outs = [bf16_bits(qlq.qlinear_w8a16(xg, qw)) for _ in range(3)]
    else:
        xq = qlq.quantize_act_static(xg, 0.03, "int8")
        outs = [qlq.qlinear_w8a8_static(xq, 0.03, qw, "acc").cpu().numpy() for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_zero_input_gives_zero_output():
    _, _, _, qw, _, _ = _prep(8, 4, 256, 64, "fp8_e4m3fn")
    y = qlq.qlinear_w8a16(torch.zeros(4, 256, dtype=torch.bfloat16, device=dev()), qw)
    assert torch.count_nonzero(y).item() == 0


def test_hip_graph_replay_matches_eager():
    M, K, N = 16, 8192, 1024                    # a split-K plan: its workspace is reused by every replay
    _, _, x, qw, _, _ = _prep(9, M, K, N, "fp8_e4m3fn")
    xg = bf16_to_gpu(x)
    eager = qlq.qlinear_w8a16(xg, qw).clone()
    out = torch.empty_like(eager)
    qlq.qlinear_w8a16(xg, qw, out=out)           # warm up (workspace allocated outside capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qlq.qlinear_w8a16(xg, qw, out=out)
    for _ in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def test_split_k_plans_interleaved_on_one_workspace():
    # Split-K calls with different plans (column-block counts, slice counts, kernel
    # families) alternate on the one shared workspace; each must stay correct.
    cases = [(1, 8192, 1024, "w8a16", "int8"), (16, 11008, 128, "w8a8_static", "int8"),
             (1, 8192, 512, "w8a8_static", "fp8_e4m3fn"), (256, 11008, 256, "w8a8_static", "int8"),
             (13, 5000, 300, "w8a16", "fp8_e4m3fn"), (64, 4096, 512, "w8a16", "int8")]
    prepared = []
    for i, (M, K, N, scheme, qtype) in enumerate(cases):
        assert qlq.workspace_bytes(scheme, M, K, N, qtype) > 0
        _, calib, x, qw, q_ref, s_ref = _prep(500 + i, M, K, N, qtype)
        sx = oracle.calibrate_input_scale(calib, qtype)
        if scheme == "w8a16":
            ref = bits_to_f64(oracle.qlinear_w8a16(x, q_ref, s_ref, qtype))
        else:
            ref = oracle.qlinear_w8a8_static(oracle.quantize_act_static(x, sx, qtype), sx, q_ref, s_ref, qtype,
                                             out="acc")
        prepared.append((scheme, qtype, bf16_to_gpu(x), sx, qw, ref))
    for rep in range(3):
        for scheme, qtype, xg, sx, qw, ref in prepared:
            print(f"interleaved rep={rep} {scheme} {qtype} M={xg.shape[0]} K={qw.K} N={qw.N}", flush=True)
            if scheme == "w8a16":
                check_close(bits_to_f64(bf16_bits(qlq.qlinear_w8a16(xg, qw))), ref)
            else:
                acc = qlq.qlinear_w8a8_static(qlq.quantize_act_static(xg, float(sx), qtype), float(sx), qw,
                                              "acc").cpu().numpy()
                if qtype == "int8":
                    assert np.array_equal(acc, ref)
                else:
                    check_close(acc, ref)


@pytest.mark.parametrize("MKN", [(1, 11008, 2048), (256, 11008, 2048), (16, 8192, 1024)])
def test_split_k_int8_repeated_bit_exact(MKN):
    # Split-K slices may land on different XCDs; the integer accumulators must
    # come out identical to the oracle on every one of many repeated calls.
    M, K, N = MKN
    assert qlq.workspace_bytes("w8a8_static", M, K, N, "int8") > 0
    _, calib, x, qw, q_ref, s_ref = _prep(901 + M, M, K, N, "int8")
    sx = oracle.calibrate_input_scale(calib, "int8")
    ref = oracle.qlinear_w8a8_static(oracle.quantize_act_static(x, sx, "int8"), sx, q_ref, s_ref, "int8", out="acc")
    xq = qlq.quantize_act_static(bf16_to_gpu(x), float(sx), "int8")
    out = torch.empty((M, N), dtype=torch.int32, device=dev())
    for rep in range(20):
        out.fill_(-1)
        qlq.qlinear_w8a8_static(xq, float(sx), qw, "acc", out=out)
        assert np.array_equal(out.cpu().numpy(), ref), f"rep {rep}"


# small-M decode shapes with many column tiles: odd tile counts, ragged N, split-K over long K
PAIR_SHAPES = [(8, 2048, 8208), (16, 128, 8200), (9, 11008, 8208), (16, 640, 16 * 600)]


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("MKN", PAIR_SHAPES)
def test_small_m_many_column_tiles(qtype, MKN):
    M, K, N = MKN
    print(f"small-M many tiles {qtype} M={M} K={K} N={N}", flush=True)
    _, calib, x, qw, q_ref, s_ref = _prep(1300 + M + K + N, M, K, N, qtype)
    y = qlq.qlinear_w8a16(bf16_to_gpu(x), qw)
    check_close(bits_to_f64(bf16_bits(y)), bits_to_f64(oracle.qlinear_w8a16(x, q_ref, s_ref, qtype)),
                f"w8a16 many tiles {MKN}")
    sx = oracle.calibrate_input_scale(calib, qtype)
    xq_ref = oracle.quantize_act_static(x, sx, qtype)
    xq = qlq.quantize_act_static(bf16_to_gpu(x), float(sx), qtype)
    acc = qlq.qlinear_w8a8_static(xq, float(sx), qw, "acc").cpu().numpy()
    acc_ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, qtype, out="acc")
    if qtype == "int8":
        assert np.array_equal(acc, acc_ref)
    else:
        check_close(acc, acc_ref, f"w8a8 many tiles {MKN}")
