"""The allocation-free W8A16 entry point (split-K scratch in a device array inside
the library) against qlq_qlinear_w8a16 with a caller's workspace, through the C ABI.

Two calls in a row on the shared array, the second with a smaller input, each
compared with the workspace call on the same inputs; the outputs are also held to
the oracle's tolerance.  A plan above the array's size is rejected and writes
nothing."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_bits, bf16_to_gpu, bits_to_f64, check_close, dev, f32_to_gpu

pytestmark = pytest.mark.gpu

MAX_SCRATCH = 32 * 1024 * 1024 + 4096


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _call_noalloc(x, qw, y):
    L = qlq.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return L.qlq_qlinear_w8a16_noalloc(_p(x), x.shape[0], qw.K, qw.N, _p(qw.packed), _p(qw.scale),
                                       qw.scale.numel(), qlq.QTYPES[qw.qtype], _p(y), stream)


def _case(seed, M, K, N, qtype):
    w, _, x = synth.small_inputs(seed, M, K, N)
    return w, x, qlq.quantize_weight(f32_to_gpu(w), qtype)


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    # 1: a split-K plan that fills the array (1024 x 11008 -> 2048: four K slices of
    #    128 x 256 tiles, 32 MiB of partials); 2: a smaller split plan (small-M kernel)
    #    on the same array; 3: a plan without split-K.
    cases = [(5, 1024, 11008, 2048, "int8"), (6, 16, 11008, 2048, "fp8_e4m3fn"), (7, 1, 2048, 2048, "int8")]
    plans = [qlq.gemm_plan("w8a16", M, K, N, q) for _, M, K, N, q in cases]
    assert plans[0]["split_k"] > 1 and plans[0]["workspace_bytes"] <= MAX_SCRATCH
    assert plans[1]["split_k"] > 1 and plans[1]["kind"] == 0 and plans[2]["workspace_bytes"] == 0
    for seed, M, K, N, qtype in cases:
        print(f"noalloc {qtype} M={M} K={K} N={N}", flush=True)
        w, x, qw = _case(seed, M, K, N, qtype)
        xg = bf16_to_gpu(x)
        y_na = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
        st = _call_noalloc(xg, qw, y_na)
        assert st == 0, qlq.lib().qlq_last_error().decode()
        y_ws = qlq.qlinear_w8a16(xg, qw)                     # workspace call, same plan and kernels
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y_na), bf16_bits(y_ws)), (M, K, N, qtype)
        if M <= 16:
            q_ref, s_ref = oracle.quantize_weight(w, qtype)
            check_close(bits_to_f64(bf16_bits(y_na)), bits_to_f64(oracle.qlinear_w8a16(x, q_ref, s_ref, qtype)),
                        f"noalloc {qtype} M={M}")
    # the first case again after the smaller ones: the array's leftovers do not leak in
    seed, M, K, N, qtype = cases[0]
    _, x, qw = _case(seed, M, K, N, qtype)
    xg = bf16_to_gpu(x)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    assert _call_noalloc(xg, qw, y1) == 0
    assert torch.equal(y1, qlq.qlinear_w8a16(xg, qw))


def test_noalloc_rejects_a_plan_above_its_scratch():
    M, K, N = 2048, 11008, 2048                              # needs 64 MiB of partials
    assert qlq.gemm_plan("w8a16", M, K, N, "int8")["workspace_bytes"] > MAX_SCRATCH
    _, x, qw = _case(8, 64, K, N, "int8")
    xg = torch.zeros((M, K), dtype=torch.bfloat16, device=dev())
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=dev())
    st = _call_noalloc(xg, qw, y)
    assert st == 1 and "scratch" in qlq.lib().qlq_last_error().decode()
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
