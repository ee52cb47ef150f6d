"""GPU INT8 W8A8 at the largest K its int32 accumulator admits (127 * 127 * K < 2^31, so
K <= 133144), with worst-case magnitudes: every code is +-127 and some output sums reach
127 * 127 * K.  Each kernel family runs at that K -- the small-M kernel with a deep split
(aligned and generic loads), the direct-to-LDS kernel (K % 64 == 0) and the register-staged
kernel (any other K) -- and its int32 accumulators and bf16 outputs must equal the oracle's
exact sums bit for bit.
"""
import numpy as np
import pytest

import oracle
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_bits, bf16_to_gpu, f32_to_gpu

pytestmark = pytest.mark.gpu

K_ALIGNED = 64 * 2080          # 133120
K_RAGGED = 133141              # not a multiple of 64; 127 * 127 * K = 2 147 431 189 < 2^31


@pytest.mark.parametrize("K", [K_ALIGNED, K_RAGGED])
@pytest.mark.parametrize("M", [1, 16, 40])
def test_int8_w8a8_largest_k_worst_case(M, K):
    print(f"int8 w8a8 largest K: M={M} K={K}", flush=True)
    N = 48
    rng = np.random.default_rng(9000 + M + K)
    # +-1 weights: every row's absmax is 1, so its scale is fp32(1/127) and every code is +-127
    w = rng.choice(np.array([-1.0, 1.0], np.float32), size=(N, K))
    w[:8] = 1.0
    w[8:16] = -1.0
    # +-1 activations (bf16 exact); row 0 all +1 meets the constant weight rows at +-127 * 127 * K
    x = rng.choice(np.array([-1.0, 1.0], np.float32), size=(M, K))
    x[0] = 1.0
    xb = oracle.f32_to_bf16_bits(x)
    sx = oracle.calibrate_input_scale(xb, "int8")
    xq_ref = oracle.quantize_act_static(xb, sx, "int8")
    q_ref, s_ref = oracle.quantize_weight(w, "int8")
    assert np.all(np.abs(xq_ref.astype(np.int32)) == 127) and np.all(np.abs(q_ref.astype(np.int32)) == 127)
    acc_ref = oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, "int8", out="acc")
    assert int(acc_ref[0, 0]) == 127 * 127 * K and int(acc_ref[0, 8]) == -127 * 127 * K

    qw = qlq.quantize_weight(f32_to_gpu(w), "int8")
    xq = qlq.quantize_act_static(bf16_to_gpu(xb), float(sx), "int8")
    acc = qlq.qlinear_w8a8_static(xq, float(sx), qw, "acc").cpu().numpy()
    assert np.array_equal(acc, acc_ref)
    y = bf16_bits(qlq.qlinear_w8a8_static(xq, float(sx), qw, "bf16"))
    assert np.array_equal(y, oracle.qlinear_w8a8_static(xq_ref, sx, q_ref, s_ref, "int8"))
