"""The C ABI library loads, exports what include/qlq.h declares, and validates
its arguments on the host (CPU only: every call here is rejected before any
kernel is enqueued)."""
import ctypes
import os
import re

import pytest

import weight_quantized_linear_qlinear_amd as qlq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlq.h")
FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced: validation fails first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls_and_helpers():
    names = _declared()
    for n in ["qlq_quantize_weight", "qlq_qlinear_w8a16", "qlq_quantize_act_static", "qlq_qlinear_w8a8_static",
              "qlq_calibrate_input_scale", "qlq_unpack_weight", "qlq_packed_weight_bytes",
              "qlq_workspace_bytes", "qlq_status_string", "qlq_last_error", "qlq_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(qlq.library_path())
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_signatures_cover_the_header():
    from weight_quantized_linear_qlinear_amd import binding
    assert sorted(binding._SIGNATURES) == _declared()


def test_version_and_status_strings():
    L = qlq.lib()
    assert L.qlq_version().decode().startswith("qlq")
    assert [L.qlq_status_string(i).decode() for i in range(4)] == \
        ["QLQ_OK", "QLQ_ERR_INVALID_ARG", "QLQ_ERR_UNSUPPORTED", "QLQ_ERR_HIP"]


def test_packed_bytes_is_tile_padded_and_about_half_of_bf16():
    assert qlq.packed_weight_bytes(16, 64) == 1024
    assert qlq.packed_weight_bytes(1, 1) == 1024
    assert qlq.packed_weight_bytes(17, 65) == 32 * 128
    assert qlq.packed_weight_bytes(0, 5) == 0
    # INT8 table of the Nano-vLLM-MOE mirror: weight memory ~0.5x of BF16
    for N, K in [(2048, 2048), (11008, 2048), (2048, 11008)]:
        assert qlq.packed_weight_bytes(N, K) == N * K == (2 * N * K) // 2


def test_workspace_sizes():
    assert qlq.workspace_bytes("w8a16", 16, 2048, 11008, "fp8_e4m3fn") == 0      # enough column blocks
    assert qlq.workspace_bytes("w8a16", 1, 2048, 2048, "int8") == 0              # waves split K in one workgroup
    assert qlq.gemm_plan("w8a16", 1, 2048, 1024, "int8")["split_k"] == 1          # narrow N, 32 units of K: one slice
    assert qlq.workspace_bytes("w8a16", 1, 2048, 1024, "int8") > 0               # (unaligned x: generic path, split)
    assert qlq.workspace_bytes("w8a16", 1, 14336, 1024, "int8") > 0              # narrow N, deep K: split over K
    assert qlq.workspace_bytes("w8a16", 1, 13824, 5120, "int8") > 0              # 320 column tiles, deep K: split
    assert qlq.workspace_bytes("w8a8_static", 1024, 2048, 11008, "fp8_e4m3fn") == 0
    assert qlq.workspace_bytes("w8a8_static", 256, 11008, 2048, "int8") > 0
    assert qlq.workspace_bytes("w8a16", 0, 64, 64, "int8") == 0


def _status(fn, *args):
    return fn(*args), qlq.lib().qlq_last_error().decode()


def test_validation_null_pointers_and_sizes():
    L = qlq.lib()
    st, msg = _status(L.qlq_qlinear_w8a16, None, 1, 64, 16, FAKE, FAKE, 16, 0, FAKE, None, 0, None)
    assert st == 1 and "null" in msg
    st, msg = _status(L.qlq_qlinear_w8a16, FAKE, 0, 64, 16, FAKE, FAKE, 16, 0, FAKE, None, 0, None)
    assert st == 1 and ">= 1" in msg
    st, _ = _status(L.qlq_quantize_weight, FAKE, 0, 16, -1, 0, 0, FAKE, FAKE, None)
    assert st == 1
    # every dimension in range but M * N beyond 2^40 outputs: rejected before any launch
    big = 1 << 24
    st, msg = _status(L.qlq_qlinear_w8a16, FAKE, big, 64, big, FAKE, FAKE, big, 0, FAKE, None, 0, None)
    assert st == 2 and "2^40" in msg
    st, _ = _status(L.qlq_calibrate_input_scale, FAKE, 0, 0, FAKE, None)
    assert st == 1


def test_validation_enums_scales_and_workspace():
    L = qlq.lib()
    st, _ = _status(L.qlq_qlinear_w8a16, FAKE, 1, 64, 16, FAKE, FAKE, 16, 7, FAKE, None, 0, None)
    assert st == 2
    st, _ = _status(L.qlq_quantize_weight, FAKE, 0, 16, 64, 0, 5, FAKE, FAKE, None)
    assert st == 2
    st, msg = _status(L.qlq_qlinear_w8a16, FAKE, 1, 64, 16, FAKE, FAKE, 3, 0, FAKE, None, 0, None)
    assert st == 1 and "w_scale_numel" in msg
    for bad in [0.0, -1.0, float("inf"), float("nan")]:
        st, msg = _status(L.qlq_quantize_act_static, FAKE, 4, 64, bad, 0, FAKE, None)
        assert st == 1 and "input_scale" in msg
        st, _ = _status(L.qlq_qlinear_w8a8_static, FAKE, bad, 4, 64, 16, FAKE, FAKE, 16, 0, 0, FAKE, None, 0, None)
        assert st == 1
    st, _ = _status(L.qlq_qlinear_w8a8_static, FAKE, 1.0, 4, 64, 16, FAKE, FAKE, 16, 0, 9, FAKE, None, 0, None)
    assert st == 2
    # INT8 accumulator bound: K <= 133144
    st, msg = _status(L.qlq_qlinear_w8a8_static, FAKE, 1.0, 4, 133145, 16, FAKE, FAKE, 16, 0, 0, FAKE, None, 0, None)
    assert st == 1 and "133144" in msg
    # a split-K plan needs its workspace
    need = qlq.workspace_bytes("w8a16", 1, 14336, 1024, "int8")
    assert need > 0
    st, msg = _status(L.qlq_qlinear_w8a16, FAKE, 1, 14336, 1024, FAKE, FAKE, 1024, 0, FAKE, None, 0, None)
    assert st == 1 and "workspace" in msg
    st, msg = _status(L.qlq_qlinear_w8a16, FAKE, 1, 14336, 1024, FAKE, FAKE, 1024, 0, FAKE, FAKE, need - 1, None)
    assert st == 1 and "workspace" in msg
    # misaligned packed weights
    st, msg = _status(L.qlq_qlinear_w8a16, FAKE, 1, 64, 16, ctypes.c_void_p(0x10008), FAKE, 16, 0, FAKE, None, 0,
                      None)
    assert st == 1 and "aligned" in msg


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        qlq.quantize_weight(torch.zeros(4, 4), "int8")


def test_header_declares_the_next_rows():
    names = _declared()
    for n in ["qlq_quantize_act_dynamic", "qlq_qlinear_w8a8_dynamic", "qlq_qlinear_w8a8_static_fused"]:
        assert n in names


def test_fused_and_dynamic_workspace_sizes():
    for M, K, N in [(1, 2048, 2048), (16, 2048, 11008), (1, 11008, 2048), (17, 64, 16), (256, 11008, 2048),
                    (1024, 2048, 11008)]:
        for qtype in ["int8", "fp8_e4m3fn"]:
            g = qlq.workspace_bytes("w8a8_static", M, K, N, qtype)
            assert qlq.workspace_bytes("w8a8_dynamic", M, K, N, qtype) == g
            # the codes live after the GEMM's region and never below the 4 KiB counter region
            f = qlq.workspace_bytes("w8a8_static_fused", M, K, N, qtype)
            assert f >= max(g, 4096) + M * K and f - M * K >= 4096 and (f - M * K) % 256 == 0


def test_validation_of_the_next_rows():
    L = qlq.lib()
    st, msg = _status(L.qlq_quantize_act_dynamic, FAKE, 4, 64, 0, FAKE, None, None)
    assert st == 1 and "null" in msg
    st, _ = _status(L.qlq_quantize_act_dynamic, FAKE, 0, 64, 0, FAKE, FAKE, None)
    assert st == 1
    st, _ = _status(L.qlq_quantize_act_dynamic, FAKE, 4, 64, 3, FAKE, FAKE, None)
    assert st == 2
    st, msg = _status(L.qlq_qlinear_w8a8_dynamic, FAKE, None, 4, 64, 16, FAKE, FAKE, 16, 0, 0, FAKE, None, 0, None)
    assert st == 1 and "null" in msg
    st, msg = _status(L.qlq_qlinear_w8a8_dynamic, FAKE, FAKE, 4, 133145, 16, FAKE, FAKE, 16, 0, 0, FAKE, None, 0,
                      None)
    assert st == 1 and "133144" in msg
    st, _ = _status(L.qlq_qlinear_w8a8_dynamic, FAKE, FAKE, 4, 64, 16, FAKE, FAKE, 16, 0, 5, FAKE, None, 0, None)
    assert st == 2
    for bad in [0.0, -2.0, float("nan")]:
        st, msg = _status(L.qlq_qlinear_w8a8_static_fused, FAKE, bad, 4, 64, 16, FAKE, FAKE, 16, 0, 0, FAKE, None,
                          0, None)
        assert st == 1 and "input_scale" in msg
    # the fused call keeps its codes in the workspace
    need = qlq.workspace_bytes("w8a8_static_fused", 64, 128, 32, "int8")
    st, msg = _status(L.qlq_qlinear_w8a8_static_fused, FAKE, 1.0, 64, 128, 32, FAKE, FAKE, 32, 0, 0, FAKE, FAKE,
                      need - 1, None)
    assert st == 1 and "workspace" in msg
    st, msg = _status(L.qlq_qlinear_w8a8_static_fused, FAKE, 1.0, 64, 128, 32, FAKE, FAKE, 32, 0, 0, FAKE,
                      ctypes.c_void_p(0x10010), need, None)
    assert st == 1 and "256-byte" in msg


def test_validation_of_the_kv_codec():
    L = qlq.lib()
    assert "qlq_kv_quantize" in _declared() and "qlq_kv_dequantize" in _declared()
    st, msg = _status(L.qlq_kv_quantize, FAKE, FAKE, 4, 2, 100, FAKE, FAKE, FAKE, FAKE, None)
    assert st == 1 and "multiple of 32" in msg
    st, msg = _status(L.qlq_kv_quantize, FAKE, None, 4, 2, 128, FAKE, FAKE, FAKE, FAKE, None)
    assert st == 1 and "null" in msg
    st, _ = _status(L.qlq_kv_quantize, FAKE, FAKE, 0, 2, 128, FAKE, FAKE, FAKE, FAKE, None)
    assert st == 1
    st, msg = _status(L.qlq_kv_dequantize, FAKE, FAKE, FAKE, FAKE, 4, 2, 2048, FAKE, FAKE, None)
    assert st == 1 and "1024" in msg
    st, msg = _status(L.qlq_kv_dequantize, FAKE, FAKE, FAKE, FAKE, 4, 2, 128, ctypes.c_void_p(0x10008), FAKE, None)
    assert st == 1 and "aligned" in msg


def test_validation_of_the_routed_linear():
    L = qlq.lib()
    for n in ["qlq_linear", "qlq_linear_workspace_bytes"]:
        assert n in _declared()
    st, msg = _status(L.qlq_linear, 2, FAKE, 4, 64, 16, FAKE, FAKE, 16, 0, 1.0, None, 0, FAKE, None, 0, None)
    assert st == 2 and "scheme" in msg
    st, msg = _status(L.qlq_linear, 1, FAKE, 4, 64, 16, FAKE, FAKE, 16, 0, 1.0, None, -1, FAKE, None, 0, None)
    assert st == 1 and "fallback" in msg
    st, msg = _status(L.qlq_linear, 1, FAKE, 4, 64, 16, FAKE, FAKE, 16, 0, float("nan"), None, 0, FAKE, None, 0, None)
    assert st == 1 and "input_scale" in msg
    need = qlq.linear_workspace_bytes("w8a8_dynamic", 4, 64, 16, "int8")
    st, msg = _status(L.qlq_linear, 3, FAKE, 4, 64, 16, FAKE, FAKE, 16, 0, 1.0, None, 0, FAKE, FAKE, need - 1, None)
    assert st == 1 and "workspace" in msg
    st, msg = _status(L.qlq_linear, 0, FAKE, 4, 64, 16, FAKE, FAKE, 16, 0, 1.0, ctypes.c_void_p(0x10001), 0, FAKE,
                      None, 0, None)
    assert st == 1 and "aligned" in msg


def test_routed_linear_workspace_sizes():
    for M, K, N in [(1, 2048, 2048), (16, 2048, 11008), (256, 11008, 2048), (1024, 2048, 11008)]:
        assert qlq.linear_workspace_bytes("w8a16", M, K, N, "int8") == qlq.workspace_bytes("w8a16", M, K, N, "int8")
        s = qlq.linear_workspace_bytes("w8a8_static", M, K, N, "int8")
        d = qlq.linear_workspace_bytes("w8a8_dynamic", M, K, N, "int8")
        assert s >= qlq.workspace_bytes("w8a8_static", M, K, N, "int8") + M * K and d >= s + 4 * M
        assert s >= qlq.workspace_bytes("w8a16", M, K, N, "int8")          # the fallback fits too


def test_validation_of_the_requant_call():
    L = qlq.lib()
    f = L.qlq_qlinear_w8a8_static_requant
    for bad in [0.0, -2.0, float("inf"), float("nan")]:
        st, msg = _status(f, FAKE, 1.0, 4, 64, 16, FAKE, FAKE, 16, 0, bad, FAKE, FAKE, None, 0, None)
        assert st == 1 and "next_scale" in msg
        st, msg = _status(f, FAKE, bad, 4, 64, 16, FAKE, FAKE, 16, 0, 1.0, FAKE, FAKE, None, 0, None)
        assert st == 1 and "input_scale" in msg
    st, msg = _status(f, FAKE, 1.0, 4, 64, 16, FAKE, FAKE, 16, 0, 1.0, FAKE, None, None, 0, None)
    assert st == 1 and "null" in msg
    st, msg = _status(f, FAKE, 1.0, 4, 64, 16, FAKE, FAKE, 16, 0, 1.0, FAKE, ctypes.c_void_p(0x10008), None, 0, None)
    assert st == 1 and "aligned" in msg
    st, msg = _status(f, FAKE, 1.0, 4, 133145, 16, FAKE, FAKE, 16, 0, 1.0, FAKE, FAKE, None, 0, None)
    assert st == 1 and "133144" in msg
    st, _ = _status(f, FAKE, 1.0, 4, 64, 16, FAKE, FAKE, 16, 5, 1.0, FAKE, FAKE, None, 0, None)
    assert st == 2


def test_multi_kernel_calls_validate_everything_before_the_first_launch():
    """The fused static call and the routed Linear enqueue a quantization kernel and
    then the GEMM.  Every check of the GEMM runs before the first launch: on this
    host (no GPU) a launch would fail with QLQ_ERR_HIP, so QLQ_ERR_INVALID_ARG with
    the GEMM's own message shows that nothing was enqueued."""
    L = qlq.lib()
    M, K, N = 4, 64, 16
    mis = ctypes.c_void_p(0x10001)
    for qtype in (0, 1):
        need = qlq.workspace_bytes("w8a8_static_fused", M, K, N, "int8" if qtype == 0 else "fp8_e4m3fn")
        fused = L.qlq_qlinear_w8a8_static_fused
        st, msg = _status(fused, FAKE, 1.0, M, K, N, FAKE, FAKE, 3, qtype, 0, FAKE, FAKE, need, None)
        assert st == 1 and "w_scale_numel" in msg, msg
        st, msg = _status(fused, FAKE, 1.0, M, K, N, FAKE, FAKE, N, qtype, 0, mis, FAKE, need, None)
        assert st == 1 and "aligned" in msg, msg
        st, msg = _status(fused, FAKE, 1.0, M, K, N, ctypes.c_void_p(0x10008), FAKE, N, qtype, 0, FAKE, FAKE, need,
                          None)
        assert st == 1 and "aligned" in msg, msg
        st, msg = _status(fused, FAKE, 1.0, 1 << 24, K, 1 << 24, FAKE, FAKE, 1, qtype, 0, FAKE, FAKE, 1 << 62, None)
        assert st == 2 and "2^40" in msg, msg
        for scheme, name in ((1, "w8a8_static"), (3, "w8a8_dynamic")):
            need = qlq.linear_workspace_bytes(name, M, K, N, "int8" if qtype == 0 else "fp8_e4m3fn")
            st, msg = _status(L.qlq_linear, scheme, FAKE, M, K, N, FAKE, FAKE, 3, qtype, 1.0, None, 0, FAKE, FAKE,
                              need, None)
            assert st == 1 and "w_scale_numel" in msg, msg
            st, msg = _status(L.qlq_linear, scheme, FAKE, M, K, N, FAKE, FAKE, N, qtype, 1.0, mis, 0, FAKE, FAKE,
                              need, None)
            assert st == 1 and "aligned" in msg, msg
            st, msg = _status(L.qlq_linear, scheme, FAKE, M, K, N, FAKE, FAKE, N, qtype, 1.0, None, 0, mis, FAKE,
                              need, None)
            assert st == 1 and "aligned" in msg, msg


def _bf16_positive_finite():
    import numpy as np
    bits = np.arange(1, 0x7F80, dtype=np.uint32)            # +denormals .. largest finite
    return (bits << 16).view(np.float32)


def _calibrated_by_definition(s):
    """s = fp32(a / qmax) for some positive finite bf16 a and qmax in {127, 448}, and s >= 2^-100
    (brute force over every such a)."""
    import numpy as np
    a = _bf16_positive_finite()
    s = np.float32(s)
    if not np.isfinite(s) or not s >= np.float32(2.0 ** -100):
        return False
    return any(bool(np.any((a / np.float32(q)).astype(np.float32) == s)) for q in (127.0, 448.0))


def test_scale_classifier_accepts_exactly_the_calibrated_scales():
    import numpy as np
    rng = np.random.default_rng(5)
    a = _bf16_positive_finite()
    picks = np.concatenate([a[rng.integers(0, a.size, 300)], a[:5], a[-5:],
                            np.array([1.0, 3.0, 0.5, 2.0 ** -110, 2.0 ** -90], np.float32)])
    accepted = rejected = 0
    for q in (127.0, 448.0):
        for ai in picks:
            s = np.float32(ai) / np.float32(q)
            cand = [s, np.nextafter(s, np.float32(np.inf)), np.nextafter(s, np.float32(0.0)),
                    np.float32(s * np.float32(1.5))]
            for c in cand:
                want = _calibrated_by_definition(c)
                assert qlq.scale_is_calibrated(float(c)) == want, (float(ai), q, float(c))
                accepted += want
                rejected += not want
    for bad in [0.0, -1.0 / 127, float("inf"), float("nan"), 2.0 ** -101, 0.1, 1e-3]:
        assert qlq.scale_is_calibrated(bad) == _calibrated_by_definition(np.float32(bad))
    assert accepted > 500 and rejected > 500


def test_plan_hook_reports_the_kernel_families():
    p = qlq.gemm_plan("w8a16", 1, 2048, 2048, "int8")
    assert p["kind"] == 0 and p["tile_n"] == 16 and p["waves"] in (4, 8, 16) and p["cfg"] == -1
    p = qlq.gemm_plan("w8a16", 1024, 2048, 11008, "int8")
    assert p["kind"] == 2 and p["cfg"] >= 0 and p["tile_m"] in (128, 256)
    p = qlq.gemm_plan("w8a8_static", 300, 2000, 300, "int8")
    assert p["kind"] == 1
    p = qlq.gemm_plan("w8a8_static", 256, 11008, 2048, "int8")
    assert p["split_k"] > 1 and 0 < p["workspace_bytes"] <= qlq.workspace_bytes("w8a8_static", 256, 11008, 2048, "int8")
    with pytest.raises(qlq.QlqError):
        qlq.gemm_plan("w8a16", 0, 64, 64, "int8")


def test_requant_parity_shapes_reach_every_plan_of_the_stack_chain():
    """Every launch plan (kernel family, tile configuration, split or not, waves, tile
    width) that
    the 3B-scale stack's W8A8 chain takes is also taken by a requantizing-epilogue
    parity shape, so a planner refit cannot leave a timed plan without an oracle
    comparison of its code-writing epilogue."""
    import synth
    from tests.test_gpu_requant import SHAPES

    def key(p):
        return p["kind"], p["cfg"], p["split_k"] > 1, p["waves"], p["tile_n"]

    for qtype in ("int8", "fp8_e4m3fn"):
        tested = {key(qlq.gemm_plan("w8a8_static", *mkn, qtype)) for mkn in SHAPES}
        for M in synth.STACK_M:
            for name, K, N in synth.STACK_PROJS:
                k = key(qlq.gemm_plan("w8a8_static", M, K, N, qtype))
                assert k in tested, (qtype, M, name, k)


def test_parity_shapes_reach_every_launch_plan():
    """Every launch plan the planner chooses over a grid of shapes, for both schemes and
    qtypes, is taken by a GPU parity shape (test_gpu_gemm.py's or test_gpu_plans.py's),
    so no kernel instantiation the library can launch goes without an oracle comparison.
    A plan is, for large M, the kernel (direct-to-LDS for K a multiple of 64, else
    register-staged), its tile configuration and whether K is split; for small M, the
    waves per workgroup, the 16-column tiles per workgroup, whether K is split, whether
    K is a multiple of 64 (the aligned path) and whether there are several 16-row groups."""
    from tests.test_gpu_gemm import PAIR_SHAPES, SHAPES
    from tests.test_gpu_plans import SMALL_PLAN_SHAPES, W8A16_PLAN_SHAPES, W8A8_PLAN_SHAPES

    def key(mkn, p):
        if p["kind"] == 0:
            return 0, p["waves"], p["split_k"] > 1, mkn[1] % 64 == 0, p["tile_n"], mkn[0] > 16, p["tile_m"]
        return p["kind"], p["cfg"], p["split_k"] > 1

    grid = [(M, K, N) for M in range(17, 1100, 48) for K in range(64, 11100, 64 * 7)
            for N in range(100, 15000, 457)]
    grid += [(M, K, N) for M in (17, 300, 1000) for K in (100, 1000, 1727, 5000) for N in (100, 2000, 11000)]
    grid += [(M, K, N) for M in (1, 2, 5, 16, 20, 33, 64) for K in list(range(64, 16400, 320)) + [100, 1000, 1727]
             for N in range(16, 15000, 397)]
    for scheme, extra in (("w8a16", W8A16_PLAN_SHAPES), ("w8a8_static", W8A8_PLAN_SHAPES)):
        for qtype in ("int8", "fp8_e4m3fn"):
            tested = {key(mkn, qlq.gemm_plan(scheme, *mkn, qtype))
                      for mkn in list(SHAPES) + list(PAIR_SHAPES) + list(extra) + list(SMALL_PLAN_SHAPES)}
            for mkn in grid:
                p = qlq.gemm_plan(scheme, *mkn, qtype)
                assert key(mkn, p) in tested, (scheme, qtype, mkn, p)


def test_noalloc_call_validates_on_the_host():
    """The allocation-free W8A16 call checks its arguments, and that its plan fits the
    library's scratch array, before it looks up a device (no GPU here)."""
    L = qlq.lib()
    f = L.qlq_qlinear_w8a16_noalloc
    st, msg = _status(f, None, 1, 64, 16, FAKE, FAKE, 16, 0, FAKE, None)
    assert st == 1 and "null" in msg
    st, msg = _status(f, FAKE, 1, 64, 16, FAKE, FAKE, 3, 0, FAKE, None)
    assert st == 1 and "w_scale_numel" in msg
    assert qlq.gemm_plan("w8a16", 2048, 11008, 2048, "int8")["workspace_bytes"] > 32 * 1024 * 1024 + 4096
    st, msg = _status(f, FAKE, 2048, 11008, 2048, FAKE, FAKE, 2048, 0, FAKE, None)
    assert st == 1 and "scratch" in msg


def test_small_m_column_tile_plans_keep_their_invariants():
    """Small-M plans over a grid of decode shapes: several 16-column tiles per workgroup
    only on the aligned path (K a multiple of 64) without K slices and from 320 column
    tiles (below M = 6 / 12 only with 4096 <= K < 8192), the grid is one
    workgroup per group of tiles (and K slice), W8A8 stays at 8 waves with two tiles (FP8
    with one too), and wide outputs at M = 16 take several tiles for every scheme."""
    wide = set()
    for sch in ("w8a16", "w8a8_static"):
        for qt in ("int8", "fp8_e4m3fn"):
            for M in (1, 2, 5, 6, 8, 12, 16):
                for K in (64, 100, 704, 2048, 4096, 11008, 14336):
                    for N in (100, 2048, 5120, 5177, 10240, 11008, 14336, 28672):
                        p = qlq.gemm_plan(sch, M, K, N, qt)
                        assert p["kind"] == 0, (sch, qt, M, K, N, p)
                        ct = p["tile_n"] // 16
                        assert ct in (1, 2, 4) and p["tile_n"] == 16 * ct
                        assert p["waves"] in (4, 8, 16)
                        NT = -(-N // 16)
                        assert p["grid"] == -(-NT // ct) * p["split_k"], (sch, qt, M, K, N, p)
                        if ct > 1:
                            assert p["split_k"] == 1 and K % 64 == 0, (sch, qt, M, K, N, p)
                            k_mid = 4096 <= K < 8192
                            assert NT >= 320 and (M >= (6 if sch == "w8a16" else 12) or k_mid)
                            if M == 16 and K == 2048 and N == 11008:
                                wide.add((sch, qt))
                        if sch == "w8a8_static" and (ct == 2 or (qt == "fp8_e4m3fn" and ct == 1)):
                            assert p["waves"] <= 8, (M, K, N, p)
    assert len(wide) == 4, wide


def test_batched_decode_plans_take_row_groups():
    """From 17 to 128 rows on aligned K, the small-M kernel runs one workgroup per 16-row
    group when it measured faster than the direct-to-LDS kernel: up to 64 rows always for
    outputs of fewer than 128 column tiles, otherwise two groups below K = 12288, three for
    weights of at most 20M codes (over K <= 8192: 28M, for W8A8 on at most 512 column
    tiles), four for at most 12M (W8A16 over K = 2048: 24M); from 65 to 128 rows narrow
    outputs over K <= 4096 and weights of at most 4M codes on at most 128 column tiles;
    ragged K and larger M keep the large-M kernels.  With one column tile per workgroup, two
    groups share a workgroup (tile_m 32) on 192 or more column tiles, or on at least 128
    over K >= 8192, and three groups take a pair and a single (the pair's second group
    past M) on fewer than 128 column tiles over K >= 8192; on exactly 128 column tiles over
    K >= 8192, on 64 column tiles over K >= 14336 (FP8 W8A8: K >= 28672) and, in W8A8, on 80
    to 127 column tiles over K >= 8192 (FP8 up to 24M weight codes, INT8 below K = 10240),
    three groups take one workgroup of four (tile_m 64).  The grid and workspace count
    every group, and K slices keep one arrival counter per (group, column tile) inside the
    counter region."""
    def cdiv(a, b):
        return -(-a // b)

    for sch in ("w8a16", "w8a8_static"):
        for qt in ("int8", "fp8_e4m3fn"):
            for M in (16, 17, 24, 32, 33, 48, 64, 65, 100, 128, 129):
                for K in (64, 1000, 2048, 3072, 4096, 8192, 11008, 12288, 14336, 28672):
                    for N in (16, 1000, 1024, 1536, 2048, 4096, 5632, 8192, 11008):
                        p = qlq.gemm_plan(sch, M, K, N, qt)
                        where = (sch, qt, M, K, N, p)
                        nrg = cdiv(M, 16)
                        w16 = sch == "w8a16"
                        by_size = {3: N * K <= 20 << 20 or (K <= 8192 and N * K <= 28 << 20 and
                                                              (w16 or cdiv(N, 16) <= 512)) or
                                      (K >= 8192 and cdiv(N, 16) == 128),
                                   4: N * K <= 12 << 20 or (w16 and K <= 2048 and N * K <= 24 << 20)}
                        narrow = cdiv(N, 16) < 128
                        if M <= 16:
                            small = True
                        elif K % 64 or M > 128:
                            small = False
                        elif nrg > 4:
                            small = (narrow and K <= 4096) or (cdiv(N, 16) <= 128 and N * K <= 4 << 20)
                        else:
                            small = narrow or (K < 12288 if nrg <= 2 else by_size[nrg])
                        assert (p["kind"] == 0) == small, where
                        if p["kind"] != 0:
                            continue
                        NT, ct, S, rw = cdiv(N, 16), p["tile_n"] // 16, p["split_k"], p["tile_m"] // 16
                        pair = ct == 1 and ((nrg == 2 and (NT >= 192 or (K >= 8192 and NT >= 128))) or
                                            (nrg == 3 and NT < 128 and K >= 8192))
                        if sch != "w8a16" and qt == "fp8_e4m3fn" and p["waves"] == 16:
                            pair = False                  # no 16-wave FP8 W8A8 pair build
                        fp8_w8a8 = sch != "w8a16" and qt == "fp8_e4m3fn"
                        quad = nrg == 3 and ((K >= 8192 and NT == 128) or
                                             (NT == 64 and K >= 14336 and (not fp8_w8a8 or K >= 28672)) or
                                             (sch != "w8a16" and 80 <= NT < 128 and K >= 8192 and
                                              (N * K <= 24 << 20 if fp8_w8a8 else K < 10240)))
                        assert ct == 1 or not quad, where
                        assert rw == (4 if quad else 2 if pair else 1), where
                        assert p["grid"] == cdiv(NT, ct) * S * cdiv(nrg, rw), where
                        if S > 1:
                            assert NT * nrg <= 1024 and p["workspace_bytes"] >= S * nrg * NT * 1024, where


def test_small_m_k_slice_plans_keep_their_invariants():
    """K slices of small-M plans: narrow outputs (fewer than 128 column tiles) on aligned K
    take about 64 units of 64 inputs per slice (48 two-tile units for FP8 W8A8, 32 for
    W8A16 above M = 8) on at most 256 workgroups (ragged K: up to 128 workgroups of at
    least 8 units); 128 to 191 tiles take two slices over 64 units or more; wider outputs
    are split only with one column tile per workgroup, 257 to 1024 tiles, deep weights
    (128 units; FP8 W8A8 96 two-tile units) and the busiest CU above 1.2 times the mean,
    into the 2 to 4 slices with the best spread (four waves each)."""
    def cdiv(a, b):
        return -(-a // b)

    def spread(g):
        return cdiv(g, 256) / (g / 256)

    for sch in ("w8a16", "w8a8_static"):
        for qt in ("int8", "fp8_e4m3fn"):
            tpu = 2 if (sch == "w8a8_static" and qt == "fp8_e4m3fn") else 1
            for M in (1, 4, 8, 16):
                for K in (100, 2048, 4096, 8192, 11008, 13824, 14336, 28672, 100000):
                    for N in (16, 100, 1024, 2047, 2048, 3000, 4100, 5120, 6144, 11008, 16400, 17000):
                        p = qlq.gemm_plan(sch, M, K, N, qt)
                        NT, KU = cdiv(N, 16), cdiv(cdiv(K, 64), tpu)
                        S, ct = p["split_k"], p["tile_n"] // 16
                        where = (sch, qt, M, K, N, p)
                        assert 1 <= S <= KU and S * NT <= 1024 * 256, where
                        if S > 1:
                            assert p["workspace_bytes"] >= S * NT * 1024, where
                        if NT < 128 and K % 64 == 0:
                            target = 48 if tpu == 2 else (32 if sch == "w8a16" and M > 8 else 64)
                            s0 = max(1, min(cdiv(256, NT), cdiv(KU, target)))
                            assert S == cdiv(KU, cdiv(KU, s0)), where      # equal slices of whole units
                            assert cdiv(KU, S) <= target or S * NT >= 256, where
                        elif NT < 128:                                       # generic path: the first rule
                            s0 = min(cdiv(128, NT), max(1, KU // 8))
                            assert S == cdiv(KU, cdiv(KU, s0)), where
                        elif NT < 192:
                            assert S == (2 if KU >= 64 else 1), where
                        elif S > 1:
                            assert ct == 1 and 256 < NT <= 1024 and KU >= (96 if tpu == 2 else 128), where
                            assert spread(NT) > 1.2 and p["waves"] == 4, where
                            best = min(range(2, 5), key=lambda s: (round(spread(NT * s), 9), s))
                            assert S == cdiv(KU, cdiv(KU, best)), where
                        elif NT > 1024 or KU < (96 if tpu == 2 else 128):
                            assert S == 1, where
