"""GPU KV-cache codec against the oracle: codes, fp16 scale bits and decoded bf16
values are all compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import weight_quantized_linear_qlinear_amd as qlq
from tests.gpu_util import bf16_bits, bf16_to_gpu, dev

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 32), (3, 2, 64), (7, 4, 128), (5, 3, 96), (2, 2, 256), (1, 1, 1024), (1024, 4, 128),
          (333, 8, 128), (16, 28, 64)]


def _inputs(seed, T, H, D):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, H, D)).astype(np.float32) * (2.0 ** rng.integers(-8, 9, size=(T, H, 1))).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32) * (2.0 ** rng.integers(-8, 9, size=(T, H, 1))).astype(np.float32)
    if T * H > 2:
        k[0, 0, :32] = 0.0                            # zero group: scale 1
        v[-1, -1, :] = 0.0                            # zero row
        k[-1, 0, -32:] *= np.float32(1e-10)           # scale underflows fp16 -> 2^-24
        k[T // 2, -1, :32] *= np.float32(1e6)         # scale saturates at 65504, codes clamp
    return oracle.f32_to_bf16_bits(k), oracle.f32_to_bf16_bits(v)


def _u16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("THD", SHAPES)
def test_kv_quantize_bit_exact(THD):
    T, H, D = THD
    print(f"kv quantize T={T} H={H} D={D}", flush=True)
    kb, vb = _inputs(T * 131 + H * 7 + D, T, H, D)
    q = qlq.kv_quantize(bf16_to_gpu(kb), bf16_to_gpu(vb))
    kq, ks, vq, vs = oracle.kv_quantize(kb, vb)
    assert np.array_equal(q.k_codes.cpu().numpy(), kq)
    assert np.array_equal(_u16(q.k_scales), ks)
    assert np.array_equal(q.v_codes.cpu().numpy(), vq)
    assert np.array_equal(_u16(q.v_scales), vs)
    # decoding the GPU's entries equals decoding the oracle's
    kd, vd = qlq.kv_dequantize(q)
    kd_ref, vd_ref = oracle.kv_dequantize(kq, ks, vq, vs)
    assert np.array_equal(bf16_bits(kd), kd_ref)
    assert np.array_equal(bf16_bits(vd), vd_ref)


def test_kv_dequantize_all_codes_and_scales():
    # every int8 / e4m3fn code with a spread of fp16 scales, decoded exactly as the oracle does
    T, H, D = 64, 2, 256
    rng = np.random.default_rng(7)
    kq = rng.integers(-127, 128, size=(T, H, D)).astype(np.int8)
    kq.reshape(-1)[:255] = np.arange(-127, 128)
    vq = np.arange(T * H * D, dtype=np.int64).astype(np.uint8).reshape(T, H, D)
    vq[(vq & 0x7F) == 0x7F] = 0x00                   # no NaN codes
    ks = oracle.fp16_encode((2.0 ** rng.uniform(-24, 15, size=(T, H, D // 32))).astype(np.float32))
    vs = oracle.fp16_encode((2.0 ** rng.uniform(-24, 15, size=(T, H))).astype(np.float32))
    to = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).view(dt).to(dev())
    q = qlq.QuantizedKV(to(kq, torch.int8), to(ks.view(np.int16), torch.float16), to(vq, torch.uint8),
                        to(vs.view(np.int16), torch.float16))
    kd, vd = qlq.kv_dequantize(q)
    kd_ref, vd_ref = oracle.kv_dequantize(kq, ks, vq, vs)
    assert np.array_equal(bf16_bits(kd), kd_ref)
    assert np.array_equal(bf16_bits(vd), vd_ref)


def _rows_below(abits: int) -> np.ndarray:
    """bf16 rows of 128 whose four 32-channel groups and whole row all have absmax a (the bf16
    value with bits `abits`), together holding every bf16 x with |x| <= a, both signs."""
    mags = np.arange(0, abits + 1, dtype=np.uint16)
    xs = np.concatenate([mags, mags | np.uint16(0x8000)])
    per_row = 4 * 31
    n = -(-xs.size // per_row)
    fill = np.zeros(n * per_row, np.uint16)
    fill[:xs.size] = xs
    fill = fill.reshape(n, 4, 31)
    rows = np.empty((n, 4, 32), np.uint16)
    rows[:, :, 0] = abits                             # each group's and the row's absmax
    rows[:, :, 1:] = fill
    return rows.reshape(n, 128)


@pytest.mark.parametrize("part", range(4))
def test_kv_quantize_every_bf16_below_absmax(part):
    # The quantizer's division (x / s with the stored fp16 scale) against the oracle's IEEE
    # division on every bf16 x with |x| <= absmax, for absmax values across the bf16 range:
    # subnormals, every binade, the largest finite value, and values whose scale saturates
    # fp16 or rounds to a tie.
    exps = list(range(0, 255, 4))
    abits_all = [0x0001, 0x0003, 0x007F] + [(e << 7) | m for e in exps if e > 0 for m in (0x00, 0x2B, 0x7F)] + [0x7F7F]
    abits = abits_all[part::4]
    print(f"kv quantize every x below absmax: part {part}, {len(abits)} absmax values", flush=True)
    rows = np.concatenate([_rows_below(a) for a in abits])
    kb = rows.reshape(-1, 1, 128)
    vb = kb[::-1].copy()
    q = qlq.kv_quantize(bf16_to_gpu(kb), bf16_to_gpu(vb))
    kq, ks, vq, vs = oracle.kv_quantize(kb, vb)
    assert np.array_equal(_u16(q.k_scales), ks)
    assert np.array_equal(_u16(q.v_scales), vs)
    assert np.array_equal(q.k_codes.cpu().numpy(), kq)
    assert np.array_equal(q.v_codes.cpu().numpy(), vq)
