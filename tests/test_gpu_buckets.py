"""Decode-batch graph buckets (GraphBuckets): a batch of M rows runs in the graph
captured for the next bucket size, padded with zero rows.

Per bucket, at a batch size that is not itself a bucket (except 1 and 2), the
bucketed result equals the oracle at the real M: INT8 W8A8 bit for bit, bf16/fp32
paths within relL2 <= 4e-3 and |err| <= 8e-3 (|ref| + rms(ref)).  A three-projection
chain through the buckets equals the same calls made eagerly at the real M
(bit-exact where both sizes take the same launch plan, M <= 16)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_bits, bf16_to_gpu, bits_to_f64, check_close, dev, f32_to_gpu

pytestmark = pytest.mark.gpu

# one non-bucket batch size per bucket: b // 2 + 1 (b itself for the buckets 1 and 2)
M_PER_BUCKET = [b if b <= 2 else b // 2 + 1 for b in qlq.DEFAULT_BUCKETS]


@pytest.mark.parametrize("scheme", ["int8_w8a16", "fp8_w8a8_static", "int8_w8a8_dynamic"])
def test_every_bucket_matches_the_oracle_at_the_real_batch(scheme):
    K, N = 2048, 2048
    print(f"graph buckets {scheme}", flush=True)
    w, calib, x_all = synth.small_inputs(91, max(M_PER_BUCKET), K, N)
    qtype, gran = {"int8_w8a16": ("int8", "per_channel"), "fp8_w8a8_static": ("fp8_e4m3fn", "per_tensor"),
                   "int8_w8a8_dynamic": ("int8", "per_channel")}[scheme]
    qw = qlq.quantize_weight(f32_to_gpu(w), qtype, gran)
    q_ref, s_ref = oracle.quantize_weight(w, qtype, gran)
    sx = oracle.calibrate_input_scale(calib, qtype)
    Mmax = max(qlq.DEFAULT_BUCKETS)
    lin = {"int8_w8a16": "w8a16", "fp8_w8a8_static": "w8a8_static", "int8_w8a8_dynamic": "w8a8_dynamic"}[scheme]
    ws = torch.zeros(max(qlq.linear_workspace_bytes(lin, m, K, N, qtype) for m in qlq.DEFAULT_BUCKETS) + 256,
                     dtype=torch.uint8, device=dev())

    def fn(x, y):
        qlq.linear(lin, x, qw, input_scale=float(sx), out=y, workspace=ws)

    gb = qlq.GraphBuckets(fn, K, N)
    for M in M_PER_BUCKET:
        b = gb.bucket_for(M)
        x = x_all[:M]
        y = bf16_bits(gb(bf16_to_gpu(x)))
        y_ref = oracle.linear(lin, x, q_ref, s_ref, qtype, input_scale=sx)
        if scheme == "int8_w8a8_dynamic":
            assert np.array_equal(y, y_ref), f"M={M} bucket {b}"
        else:
            check_close(bits_to_f64(y), bits_to_f64(y_ref), f"{scheme} M={M} bucket {b}")
    assert Mmax == 512


@pytest.mark.parametrize("M", [1, 13, 30, 100, 300])
def test_chain_through_buckets_matches_eager_calls(M):
    """q -> up -> down of the 3B-scale stack's first layer (INT8 W8A16), bucketed and eager."""
    print(f"bucketed chain M={M}", flush=True)
    ws_b = torch.zeros(64 << 20, dtype=torch.uint8, device=dev())
    qws = [qlq.quantize_weight(synth.stack_weight(0, 0, p, dev()), "int8") for p in range(3)]
    mids = {}

    def fn(x, y):
        b = x.shape[0]
        h1 = mids.setdefault((b, 1), torch.empty((b, synth.HIDDEN), dtype=torch.bfloat16, device=dev()))
        h2 = mids.setdefault((b, 2), torch.empty((b, synth.INTERMEDIATE), dtype=torch.bfloat16, device=dev()))
        qlq.qlinear_w8a16(x, qws[0], out=h1, workspace=ws_b)
        qlq.qlinear_w8a16(h1, qws[1], out=h2, workspace=ws_b)
        qlq.qlinear_w8a16(h2, qws[2], out=y, workspace=ws_b)

    gb = qlq.GraphBuckets(fn, synth.HIDDEN, synth.HIDDEN)
    _, x = synth.stack_inputs(0, M)
    xg = bf16_to_gpu(x)
    got = gb(xg).clone()
    h = xg
    for qw in qws:
        h = qlq.qlinear_w8a16(h, qw)
    torch.cuda.synchronize()
    b = gb.bucket_for(M)
    same_plan = all(qlq.gemm_plan("w8a16", M, K, N, "int8") == qlq.gemm_plan("w8a16", b, K, N, "int8")
                    for _, K, N in synth.STACK_PROJS)
    if M <= 64 and same_plan:                           # same small-M plan at M and at its bucket
        assert torch.equal(got, h)
    else:
        check_close(bits_to_f64(bf16_bits(got)), bits_to_f64(bf16_bits(h)), f"chain M={M}")
    # replaying the same bucket again gives the same rows
    again = gb(xg)
    assert torch.equal(again, got)
