"""Exhaustive check of the activation quantizers' division on the GPU.

The static quantizer, the requantizing epilogue, the per-token quantizer and the
KV codec divide by their scale with a reciprocal refined by one Newton step and
one correction of the product, where the host finds the scale to be of the kind
this was shown for; the codes must be those of the IEEE fp32 quotient
(sat(RNE(x / s))) that the oracle computes.  Here every case of those domains is
run through the library calls themselves:

* static (any x): every scale s = fp32(a / qmax) for every positive finite bf16 a
  and qmax 127 and 448, both code types, every finite bf16 x;
* per-token (|x| <= the row's absmax a): every positive finite bf16 a, both code
  types, every finite bf16 x with |x| <= a, and the row scale itself;
* KV codec (fp16 scales): every positive finite bf16 a as the absmax of a K group
  and of a V row, every finite bf16 x with |x| <= a.

The expected codes are the IEEE quotient's, computed with torch on the GPU
(fp32 division, round-half-even, clamp, cast to e4m3fn); that reference is itself
checked against the oracle on a strided subset of the scales.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_quantized_linear_qlinear_amd as qlq
from oracle import kvcache
from tests.gpu_util import dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

QTYPES = ["int8", "fp8_e4m3fn"]
QMAX = {"int8": 127.0, "fp8_e4m3fn": 448.0}


def _finite_bf16_bits():
    b = np.arange(0, 1 << 16, dtype=np.uint32)
    finite = (b & 0x7F80) != 0x7F80
    return b[finite].astype(np.uint16)                        # 65280 patterns, both zeros included


def _positive_finite_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    return (bits << 16).view(np.float32)                     # 32639 values, denormals to the largest


def _ref_codes(xf: torch.Tensor, s: torch.Tensor, qtype: str) -> torch.Tensor:
    """sat(RNE(x / s)) in fp32 on the GPU: the IEEE quotient's code bytes (uint8)."""
    q = xf / s
    if qtype == "int8":
        return torch.clamp(torch.round(q), -127.0, 127.0).to(torch.int8).view(torch.uint8)
    return torch.clamp(q, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def test_static_quantizer_every_calibrated_scale_every_x():
    xb = _finite_bf16_bits()
    x = torch.from_numpy(xb.view(np.int16)).to(dev()).view(torch.bfloat16).reshape(1, -1)
    xf = x.float()
    a = _positive_finite_bf16()
    B = 512
    checked = 0
    for qmax in (127.0, 448.0):
        scales = (a / np.float32(qmax)).astype(np.float32)
        assert np.all(scales > 0)
        for qtype in QTYPES:
            print(f"static division: qmax {qmax:g}, {qtype}, {scales.size} scales", flush=True)
            out = torch.empty((B, x.shape[1]), dtype=torch.uint8, device=dev())
            for b0 in range(0, scales.size, B):
                sb = scales[b0:b0 + B]
                for i, s in enumerate(sb):
                    qlq.quantize_act_static(x, float(s), qtype, out=out[i:i + 1])
                ref = _ref_codes(xf, torch.from_numpy(sb).to(dev()).reshape(-1, 1), qtype)
                got = out[:sb.size]
                if not torch.equal(got, ref):
                    bad = (got != ref).nonzero()[0].tolist()
                    s = float(sb[bad[0]])
                    raise AssertionError(f"qmax {qmax} {qtype}: scale {s!r} (calibrated="
                                         f"{qlq.scale_is_calibrated(s)}) x {float(xf[0, bad[1]])!r}: "
                                         f"code {int(got[bad[0], bad[1]])} != {int(ref[bad[0], bad[1]])}")
                checked += sb.size * x.shape[1]
            # the torch reference is the oracle's quantizer on a strided subset of the scales
            for s in scales[::997]:
                want = oracle.quantize_act_static(xb.reshape(1, -1), s, qtype).view(np.uint8)
                got = _ref_codes(xf, torch.tensor(float(s), device=dev()), qtype).cpu().numpy()
                assert np.array_equal(got, want), (qmax, qtype, float(s))
    assert checked == 2 * 2 * a.size * xb.size


def test_per_token_quantizer_every_absmax_every_x_within_it():
    xb = _finite_bf16_bits()
    x_all = torch.from_numpy(xb.view(np.int16)).to(dev()).view(torch.bfloat16)
    xf_all = x_all.float()
    a = _positive_finite_bf16()
    ag = torch.from_numpy(a).to(dev())
    B = 1024
    for qtype in QTYPES:
        print(f"per-token division: {qtype}, {a.size} row absmax values", flush=True)
        for b0 in range(0, a.size, B):
            ab = ag[b0:b0 + B].reshape(-1, 1)
            keep = xf_all.abs().reshape(1, -1) <= ab                # every x within the row's absmax
            X = torch.where(keep, x_all.reshape(1, -1), torch.zeros((), dtype=torch.bfloat16, device=dev()))
            xq, xs = qlq.quantize_act_dynamic(X, qtype)
            want_s = torch.from_numpy((a[b0:b0 + B] / np.float32(QMAX[qtype])).astype(np.float32)).to(dev())
            assert torch.equal(xs, want_s), f"{qtype}: row scales from absmax index {b0}"
            ref = _ref_codes(X.float(), xs.reshape(-1, 1), qtype)
            assert torch.equal(xq.view(torch.uint8), ref), f"{qtype}: codes of rows from absmax index {b0}"
            if b0 % (16 * B) == 0:                             # reference against the oracle
                r = 7
                Xr = X[r:r + 1].cpu().view(torch.int16).numpy().view(np.uint16)
                cq, cs = oracle.quantize_act_dynamic(Xr, qtype)
                assert np.float32(cs[0]) == np.float32(xs[r].item())
                assert np.array_equal(ref[r:r + 1].cpu().numpy(), cq.view(np.uint8))


def test_kv_codec_every_absmax_every_x_within_it():
    """Rows of D = 1024 channels: 32 K groups that each start with the absmax a and
    hold 31 values |x| <= a, so a is the absmax of every K group and of the V row."""
    xb = _finite_bf16_bits()
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    order = np.argsort(np.abs(xf), kind="stable")
    by_abs = torch.from_numpy(xb[order].view(np.int16)).to(dev())
    absf = np.abs(xf[order])
    a = _positive_finite_bf16()
    n_a = np.searchsorted(absf, a, side="right")               # values with |x| <= a (a itself included)
    per_row = 32 * 31
    rows_a = -(-n_a // per_row)
    # fp16 scales the codec must store for absmax a (oracle's rule)
    k_scale = kvcache.fp16_encode((a / np.float32(127.0)).astype(np.float32))
    v_scale = kvcache.fp16_encode((a / np.float32(448.0)).astype(np.float32))
    k_scale = np.where(k_scale == 0, 1, k_scale).astype(np.uint16)   # 2^-24 for a positive absmax
    v_scale = np.where(v_scale == 0, 1, v_scale).astype(np.uint16)
    A_CHUNK = 2048
    print(f"KV division: {a.size} absmax values, {int(rows_a.sum())} rows of 1024", flush=True)
    for c0 in range(0, a.size, A_CHUNK):
        sl = slice(c0, c0 + A_CHUNK)
        ra = torch.from_numpy(rows_a[sl]).to(dev())
        owner = torch.repeat_interleave(torch.arange(ra.numel(), device=dev()), ra)     # chunk-local a index
        first = torch.cumsum(ra, 0) - ra
        local_row = torch.arange(owner.numel(), device=dev()) - first[owner]
        e = torch.arange(per_row, device=dev())
        idx = local_row.reshape(-1, 1) * per_row + e.reshape(1, -1)                 # index into the prefix
        na = torch.from_numpy(n_a[sl]).to(dev())[owner].reshape(-1, 1)
        vals = torch.where(idx < na, by_abs[torch.clamp(idx, max=by_abs.numel() - 1)],
                           torch.zeros((), dtype=torch.int16, device=dev()))
        abits = torch.from_numpy((a[sl].view(np.uint32) >> 16).astype(np.int16)).to(dev())[owner]
        rows = torch.cat([abits.reshape(-1, 1, 1).expand(-1, 32, 1), vals.reshape(-1, 32, 31)], dim=2)
        kv = rows.reshape(-1, 1, 1024).view(torch.bfloat16).contiguous()
        q = qlq.kv_quantize(kv, kv)
        ks = torch.from_numpy(k_scale[sl].view(np.int16)).to(dev())[owner]
        vs = torch.from_numpy(v_scale[sl].view(np.int16)).to(dev())[owner]
        assert torch.equal(q.k_scales.view(torch.int16).reshape(-1, 32), ks.reshape(-1, 1).expand(-1, 32)), c0
        assert torch.equal(q.v_scales.view(torch.int16).reshape(-1), vs), c0
        kf = kv.float().reshape(-1, 32, 32)
        kref = _ref_codes(kf, q.k_scales.float().reshape(-1, 32, 1), "int8").reshape(-1, 1, 1024)
        assert torch.equal(q.k_codes.view(torch.uint8), kref), f"K codes, absmax chunk {c0}"
        vref = _ref_codes(kv.float().reshape(-1, 1024), q.v_scales.float().reshape(-1, 1), "fp8_e4m3fn")
        assert torch.equal(q.v_codes.reshape(-1, 1024), vref), f"V codes, absmax chunk {c0}"
        if c0 % (4 * A_CHUNK) == 0:                             # reference against the oracle
            r = int(rows_a[sl][:3].sum())                       # first row of the chunk's 4th absmax
            sample = kv[r:r + 1].cpu().view(torch.int16).numpy().view(np.uint16)
            kq_o, ks_o, vq_o, vs_o = oracle.kv_quantize(sample, sample)
            assert np.array_equal(q.k_codes[r:r + 1].cpu().numpy().view(np.int8), kq_o.view(np.int8))
            assert np.array_equal(q.v_codes[r:r + 1].cpu().numpy(), vq_o.view(np.uint8))
