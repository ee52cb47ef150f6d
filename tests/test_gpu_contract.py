"""A rejected call enqueues nothing (the C ABI's error contract), with real device
buffers: the workspace and the output keep a sentinel fill after the fused static
call and the routed Linear reject an argument that only the GEMM step checks."""
import ctypes

import pytest
import torch

import synth
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_to_gpu, dev, f32_to_gpu

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("qtype", ["int8", "fp8_e4m3fn"])
@pytest.mark.parametrize("M", [4, 300])
def test_rejected_multi_kernel_calls_leave_buffers_untouched(qtype, M):
    K, N = 256, 96
    print(f"contract {qtype} M={M}", flush=True)
    w, _, x = synth.small_inputs(11, M, K, N)
    qw = qlq.quantize_weight(f32_to_gpu(w), qtype)
    xg = bf16_to_gpu(x)
    L = qlq.lib()
    qt = qlq.QTYPES[qtype]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    need = max(qlq.workspace_bytes("w8a8_static_fused", M, K, N, qtype),
               qlq.linear_workspace_bytes("w8a8_dynamic", M, K, N, qtype))
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=dev())
    y = torch.full((M, N), 0x3F80, dtype=torch.int16, device=dev())
    y_misaligned = torch.full((M * N + 8,), 0x3F80, dtype=torch.int16, device=dev())
    cases = [
        ("fused, w_scale_numel", lambda: L.qlq_qlinear_w8a8_static_fused(
            _p(xg), 0.05, M, K, N, _p(qw.packed), _p(qw.scale), 3, qt, 0, _p(y), _p(ws), need, stream)),
        ("fused, misaligned y", lambda: L.qlq_qlinear_w8a8_static_fused(
            _p(xg), 0.05, M, K, N, _p(qw.packed), _p(qw.scale), N, qt, 0,
            ctypes.c_void_p(y_misaligned.data_ptr() + 1), _p(ws), need, stream)),
    ]
    for scheme in (1, 3):
        cases.append((f"linear {scheme}, w_scale_numel", lambda s=scheme: L.qlq_linear(
            s, _p(xg), M, K, N, _p(qw.packed), _p(qw.scale), 3, qt, 0.05, None, 0, _p(y), _p(ws), need, stream)))
        cases.append((f"linear {scheme}, misaligned bias", lambda s=scheme: L.qlq_linear(
            s, _p(xg), M, K, N, _p(qw.packed), _p(qw.scale), N, qt, 0.05,
            ctypes.c_void_p(y_misaligned.data_ptr() + 1), 0, _p(y), _p(ws), need, stream)))
    for what, call in cases:
        st = call()
        assert st == 1, (what, st, L.qlq_last_error())
    torch.cuda.synchronize()
    assert bool((ws == 0x5A).all()), "workspace written by a rejected call"
    assert bool((y == 0x3F80).all()), "output written by a rejected call"
    assert bool((y_misaligned == 0x3F80).all())
