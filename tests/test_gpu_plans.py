"""Parity of every launch plan the planner chooses (large M: tile configuration, split or
not; small M: waves per workgroup, 16-column tiles per workgroup, split or not, aligned
K or not, one or several 16-row groups, one or two of them per workgroup), beyond the
ones the small shapes of test_gpu_gemm.py reach.

The direct-to-LDS kernel has one instantiation per tile configuration, and the
loop of each differs (waves per tile, stages, whether a wave copies exactly the
weight tiles it reads); the planner takes several of them only for large
problems.  Each shape below is a small ragged (M, N) case that the planner sends
to the plan named beside it; test_abi.py checks that these shapes together with
test_gpu_gemm.py's reach every plan the planner chooses over a grid of shapes,
so a refit of the planner cannot leave a plan without an oracle comparison.
"""
import numpy as np
import pytest

import oracle
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_bits, bf16_to_gpu, bits_to_f64, check_close, codes
from tests.test_gpu_gemm import _prep

pytestmark = pytest.mark.gpu

QTYPES = ["int8", "fp8_e4m3fn"]
# (M, K, N) -> (tile configuration, split-K) of the W8A16 planner
W8A16_PLAN_SHAPES = [(257, 64, 11072),    # 128x256, four-stage ring, no split
                     (33, 6720, 11072),   # 128x256, four-stage ring, K slices
                     (257, 640, 11072),   # 128x256, two-stage ring, no split
                     (33, 6272, 11072),   # 128x256, two-stage ring, K slices
                     (769, 256, 14026),   # 256x256, no split
                     (129, 5824, 11072)]  # 256x256, K slices
# (M, K, N) of the W8A8 planner
W8A8_PLAN_SHAPES = [(769, 1024, 14026),   # 256x256 eight waves, no split
                    (385, 8320, 8329),    # 256x256 eight waves, K slices
                    (513, 6976, 13393),   # 256x256 three-stage ring, no split
                    (535, 512, 13175),    # 256x192, no split
                    (129, 9472, 11072),   # 256x192, K slices
                    (161, 960, 100),      # 128x128 four waves, K slices
                    (161, 64, 100)]       # 128x128 four waves of 64x64, no split


# (M, K, N) -> small-M plans (waves per workgroup, column tiles per workgroup, K slices,
# aligned K or not) that the small shapes of test_gpu_gemm.py leave out, for both schemes
SMALL_PLAN_SHAPES = [(3, 2624, 413),     # four waves, K slices, aligned K
                     (7, 100, 1207),     # eight waves, no split, ragged K
                     (11, 100, 2398),    # four waves, no split, ragged K
                     (13, 1727, 413),    # eight waves, K slices, ragged K
                     (16, 1000, 1207),   # four waves, K slices, ragged K
                     # several 16-column tiles per workgroup (the last group holds fewer);
                     # tiles x waves for W8A16 / INT8 W8A8 / FP8 W8A8
                     (13, 64, 10338),    # 4 x 4 / 2 x 4 / 4 x 4
                     (14, 704, 10338),   # 4 x 8 / 2 x 8 / 4 x 4
                     (12, 1024, 10338),  # 4 x 16 / 2 x 8 / 4 x 8
                     (13, 1984, 5177),   # 2 x 16 / 2 x 8 / 2 x 8
                     (13, 1984, 10338),  # 4 x 16 / 2 x 8 / 4 x 16
                     (2, 4160, 5177),    # 2 x 16 / 2 x 8 / 2 x 8 at M = 2 (K from 4096 to 8192)
                     # K slices x waves for W8A16 / INT8 W8A8 / FP8 W8A8
                     (1, 8256, 2100),    # 2 x 16 / 2 x 16 / 2 x 8 (fewer than 192 column tiles)
                     (2, 8192, 4100),    # 4 x 4 / 4 x 4 (257 column tiles, deep K) / 1 x 4
                     (3, 4160, 3080),    # 1 x 8 / 1 x 16 / 1 x 8
                     (1, 4224, 16),      # 2 x 8 / 2 x 8 / 1 x 8 (one column tile)
                     (1, 6464, 16),      # 2 x 8 / 2 x 8 / 2 x 4
                     # batched decode: 16-row groups (the last one partial) x slices x waves x tiles
                     (17, 2112, 16), (17, 4160, 16), (17, 8576, 1014),     # K slices, one column
                     (17, 64, 5127), (17, 64, 10611), (17, 512, 5127),     # two and four column tiles
                     (17, 960, 10611), (17, 960, 5127), (33, 4160, 1604),  # up to 16 waves, three groups
                     (17, 4544, 1014), (17, 4096, 2385), (20, 6464, 16),    # K slices, 4 / 8 waves
                     (100, 1024, 500), (128, 4096, 100),                    # narrow: 7 and 8 groups
                     (80, 1024, 2048),                                      # 128 column tiles, 5 groups
                     # two row groups per workgroup (deep or wide weights): K slices or not, 4 to
                     # 16 waves; three groups (the second pair's second group past M)
                     (17, 8576, 2385), (17, 8576, 3299), (17, 8576, 4213), (17, 64, 3299),
                     (33, 8384, 16), (33, 8384, 413), (33, 8384, 1604),
                     # three groups in one workgroup of four (deep weights, 128 column tiles;
                     # 64 column tiles over deeper weights, with K slices)
                     (33, 8384, 2047), (47, 8192, 2040), (40, 16384, 2048),
                     (35, 14336, 1010), (48, 28672, 1024), (40, 8192, 1500), (47, 12288, 1920)]


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("MKN", W8A16_PLAN_SHAPES + SMALL_PLAN_SHAPES)
def test_w8a16_plan_parity(qtype, MKN):
    M, K, N = MKN
    plan = qlq.gemm_plan("w8a16", M, K, N, qtype)
    print(f"w8a16 {qtype} M={M} K={K} N={N} plan {plan}", flush=True)
    assert plan["kind"] == (0 if MKN in SMALL_PLAN_SHAPES else 2)
    _, _, x, qw, q_ref, s_ref = _prep(4000 + M * 7 + K + N, M, K, N, qtype)
    y = qlq.qlinear_w8a16(bf16_to_gpu(x), qw)
    ref = oracle.qlinear_w8a16(x, q_ref, s_ref, qtype)
    check_close(bits_to_f64(bf16_bits(y)), bits_to_f64(ref), f"w8a16 {qtype} {MKN}")


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("MKN", W8A8_PLAN_SHAPES + SMALL_PLAN_SHAPES)
def test_w8a8_plan_parity(qtype, MKN):
    M, K, N = MKN
    plan = qlq.gemm_plan("w8a8_static", M, K, N, qtype)
    print(f"w8a8 {qtype} M={M} K={K} N={N} plan {plan}", flush=True)
    assert plan["kind"] == (0 if MKN in SMALL_PLAN_SHAPES else 2)
    _, calib, x, qw, q_ref, s_ref = _prep(5000 + M * 7 + K + N, M, K, N, qtype)
    sx = oracle.calibrate_input_scale(calib, qtype)
    xq_ref = oracle.quantize_act_static(x, sx, qtype)
    xq = qlq.quantize_act_static(bf16_to_gpu(x), float(sx), qtype)
    assert np.array_equal(codes(xq), xq_ref.view(np.uint8))
    acc = qlq.qlinear_w8a8_static(xq, float(sx), qw, "acc").cpu().numpy()
    acc_ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, qtype, out="acc")
    y = bf16_bits(qlq.qlinear_w8a8_static(xq, float(sx), qw, "bf16"))
    y_ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, qtype)
    if qtype == "int8":                                   # exact int32 accumulators
        assert np.array_equal(acc, acc_ref)
        assert np.array_equal(y, y_ref)
    else:
        check_close(acc, acc_ref, f"fp8 acc {MKN}")
        check_close(bits_to_f64(y), bits_to_f64(y_ref), f"fp8 y {MKN}")
