// KV-cache codec: K as int8 with a scale per group of 32 channels, V as FP8
// with a scale per token and head, both computed at run time ("Nano-vLLM-MoE"
// README, section "KV cache compression", its Setup list: float16 scales).
//
// K and V are bf16 [T, H, D] (token, KV head, head_dim; D % 32 == 0).
//   K: per (t, h, group of 32 channels): s = fp16(absmax / 127) (an fp32
//      division, then round to nearest even into binary16, saturating at 65504;
//      1 for an all-zero group; 2^-24 if a positive absmax would round to 0),
//      codes q = clamp(rint(k / fp32(s)), -127, 127) -- division by the stored
//      scale, so decoding with it inverts the step taken.
//   V: per (t, h): s = fp16(absmax / 448), codes = e4m3fn_sat(v / fp32(s)).
//   Decoding: bf16(fp32(q) * fp32(s)), the W8A16 dequantization rule.
//   The divisions go through RcpDiv (qlq_device.h): same codes, fewer instructions.
// Stored per (t, h) with D = 128: 128 + 8 bytes of K, 128 + 2 of V, 0.5195 of
// bf16 -- the bytes-per-block figure of the pages.
//
// Quantizer, head_dim a power of two from 32 to 512 (the common case): each
// thread owns 8 consecutive elements of a row (one 16-byte load of K and of V,
// one 8-byte store of each's codes), so a wave streams 1 KiB of K and of V per
// instruction; a K group is 4 neighbouring lanes and a row D / 8 lanes, both
// reduced with xor-shuffles.  Its loads and stores are non-temporal: each input
// is read once and the codes go to the cache for later steps (measured on the 7B
// shape, 28 layers: 8.4 -> 6.7 us per layer at 8192 tokens, 23.1 -> 21.9 at
// 32768).  The dequantizer keeps ordinary stores: its output is read right away
// by attention, and a scratch output reused layer after layer stays in the cache.  Any other head_dim takes a wave per (t, h) row
// (lane l owns elements l + 64 j; a K group is a half-wave for one j).
// Dequantizer: 8 elements per thread (one 8-byte code load, one 16-byte store),
// the 8 sharing one K group and one V scale.  All are HBM-bound streams.
#include "qlq_device.h"
#include "qlq_launch.h"

namespace qlq {

namespace {

__device__ __forceinline__ uint32_t f32_to_f16_bits_sat(float x) {
  const float c = __builtin_amdgcn_fmed3f(x, 65504.0f, -65504.0f);
  const _Float16 h = (_Float16)c;                           // v_cvt_f16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);    // exact
}

__device__ __forceinline__ uint32_t kv_scale_bits(float absmax, float qmax) {
  if (absmax == 0.0f) return 0x3C00u;                         // 1.0
  const uint32_t s = f32_to_f16_bits_sat(absmax / qmax);
  return s == 0u ? 1u : s;                                    // 2^-24 instead of a zero scale
}

__device__ __forceinline__ float half_max(float v) {          // max over the 32 lanes of a half-wave
  for (int off = 16; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

template <int JN>
__global__ __launch_bounds__(256) void kv_quantize_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                          int rows, int D, uint8_t* __restrict__ kq,
                                                          uint16_t* __restrict__ ks, uint8_t* __restrict__ vq,
                                                          uint16_t* __restrict__ vs) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;                                    // whole wave leaves together
  const int64_t base = (int64_t)row * D;
  const int G = D / 32;
  float kf[JN], vf[JN];
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    const int e = lane + 64 * j;
    kf[j] = e < D ? bf16_bits_to_f32(k[base + e]) : 0.0f;
    vf[j] = e < D ? bf16_bits_to_f32(v[base + e]) : 0.0f;
  }
  // K: group 2 j + lane / 32 is the half-wave holding elements 64 j + 32 (lane / 32) + 0..31
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    const float am = half_max(fabsf(kf[j]));
    const int e = lane + 64 * j;
    if (64 * j + (lane & 32) < D) {                           // the group exists (D % 32 == 0)
      const uint32_t sb = kv_scale_bits(am, 127.0f);
      if ((lane & 31) == 0) ks[(int64_t)row * G + 2 * j + (lane >> 5)] = (uint16_t)sb;
      kq[base + e] = (uint8_t)f32_to_i8_sat(RcpDiv(f16_bits_to_f32(sb))(kf[j]));
    }
  }
  // V: one scale for the whole row
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < JN; ++j) am = fmaxf(am, fabsf(vf[j]));
  for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
  const uint32_t sb = kv_scale_bits(am, 448.0f);
  if (lane == 0) vs[row] = (uint16_t)sb;
  const RcpDiv dv(f16_bits_to_f32(sb));
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    const int e = lane + 64 * j;
    if (e < D) vq[base + e] = (uint8_t)f32_to_e4m3_sat(dv(vf[j]));
  }
}

// 8 consecutive elements per thread; TPR = D / 8 threads per (t, h) row.
template <int TPR>
__global__ __launch_bounds__(256) void kv_quantize8_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                           int64_t n8, uint8_t* __restrict__ kq,
                                                           uint16_t* __restrict__ ks, uint8_t* __restrict__ vq,
                                                           uint16_t* __restrict__ vs) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int lane = threadIdx.x & 63;
  // every lane of a wave runs the same number of iterations (n8 is padded to whole waves
  // by the launcher's grid; the tail is masked, not skipped), so the shuffles see all lanes
  const int64_t iters = (n8 + stride - 1) / stride;
  for (int64_t it = 0; it < iters; ++it) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x + it * stride;
    const bool live = i < n8;
    const u32x4 kc = live ? ld16_stream(k + i * 8) : (u32x4){0u, 0u, 0u, 0u};
    const u32x4 vc = live ? ld16_stream(v + i * 8) : (u32x4){0u, 0u, 0u, 0u};
    const uint32_t kd[4] = {kc.x, kc.y, kc.z, kc.w}, vd[4] = {vc.x, vc.y, vc.z, vc.w};
    float ka = 0.0f, va = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ka = fmaxf(ka, fmaxf(fabsf(bf16_bits_to_f32(kd[c] & 0xFFFF)), fabsf(bf16_bits_to_f32(kd[c] >> 16))));
      va = fmaxf(va, fmaxf(fabsf(bf16_bits_to_f32(vd[c] & 0xFFFF)), fabsf(bf16_bits_to_f32(vd[c] >> 16))));
    }
    ka = fmaxf(ka, __shfl_xor(ka, 1, 64));                    // K group: 4 lanes
    ka = fmaxf(ka, __shfl_xor(ka, 2, 64));
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) va = fmaxf(va, __shfl_xor(va, off, 64));   // V row: TPR lanes
    if (!live) continue;
    const uint32_t kb = kv_scale_bits(ka, 127.0f), vb = kv_scale_bits(va, 448.0f);
    const RcpDiv dk(f16_bits_to_f32(kb)), dv(f16_bits_to_f32(vb));
    uint32_t kw[2], vw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t a = kd[2 * h], b = kd[2 * h + 1];
      kw[h] = f32_to_i8_sat(dk(bf16_bits_to_f32(a & 0xFFFF))) | (f32_to_i8_sat(dk(bf16_bits_to_f32(a >> 16))) << 8) |
              (f32_to_i8_sat(dk(bf16_bits_to_f32(b & 0xFFFF))) << 16) |
              (f32_to_i8_sat(dk(bf16_bits_to_f32(b >> 16))) << 24);
      const uint32_t c = vd[2 * h], d = vd[2 * h + 1];
      vw[h] = f32x4_to_e4m3x4_sat(dv(bf16_bits_to_f32(c & 0xFFFF)), dv(bf16_bits_to_f32(c >> 16)),
                                  dv(bf16_bits_to_f32(d & 0xFFFF)), dv(bf16_bits_to_f32(d >> 16)));
    }
    __builtin_nontemporal_store((u32x2){kw[0], kw[1]}, reinterpret_cast<u32x2*>(kq + i * 8));
    __builtin_nontemporal_store((u32x2){vw[0], vw[1]}, reinterpret_cast<u32x2*>(vq + i * 8));
    if ((lane & 3) == 0) ks[i / 4] = (uint16_t)kb;            // chunk i starts group i / 4
    if ((lane & (TPR - 1)) == 0) vs[i / TPR] = (uint16_t)vb;  // chunk i starts row i / TPR
  }
}

// 8 consecutive elements per thread: codes [8 i, 8 i + 8) of the flattened [T, H, D].
__global__ __launch_bounds__(256) void kv_dequantize_kernel(const uint8_t* __restrict__ kq,
                                                            const uint16_t* __restrict__ ks,
                                                            const uint8_t* __restrict__ vq,
                                                            const uint16_t* __restrict__ vs, int64_t n8, int D,
                                                            uint16_t* __restrict__ ko, uint16_t* __restrict__ vo) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int G = D / 32;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const int64_t e0 = i * 8;
    const int64_t row = e0 / D;
    const int c = (int)(e0 % D);
    const float sk = f16_bits_to_f32(ks[row * G + c / 32]);
    const float sv = f16_bits_to_f32(vs[row]);
    const u32x2 kc = *reinterpret_cast<const u32x2*>(kq + e0);
    const u32x2 vc = *reinterpret_cast<const u32x2*>(vq + e0);
    st16(ko + e0, __builtin_bit_cast(u32x4, dequant8<kInt8>(kc.x, kc.y, sk, -128.0f * sk)));
    st16(vo + e0, __builtin_bit_cast(u32x4, dequant8<kFp8>(vc.x, vc.y, sv, -128.0f * sv)));
  }
}

}  // namespace

hipError_t launch_kv_quantize(const void* k, const void* v, int64_t rows, int D, void* kq, void* ks, void* vq,
                              void* vs, hipStream_t st) {
  const uint16_t* kb = static_cast<const uint16_t*>(k);
  const uint16_t* vb = static_cast<const uint16_t*>(v);
  uint8_t* kqb = static_cast<uint8_t*>(kq);
  uint8_t* vqb = static_cast<uint8_t*>(vq);
  uint16_t* ksb = static_cast<uint16_t*>(ks);
  uint16_t* vsb = static_cast<uint16_t*>(vs);
  const bool pow2 = D >= 32 && D <= 512 && (D & (D - 1)) == 0;
  const bool vec = ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15) == 0 &&
                   ((reinterpret_cast<uintptr_t>(kq) | reinterpret_cast<uintptr_t>(vq)) & 7) == 0;
  if (pow2 && vec) {
    // a row's D / 8 threads sit in one wave (64 is a multiple of D / 8), so whole rows and
    // groups share a wave; the grid covers the chunks with at most 2048 workgroups
    const int64_t n8 = rows * (int64_t)D / 8;
    int64_t g = (n8 + 255) / 256;
    if (g > 2048) g = 2048;
    switch (D / 8) {
      case 4: kv_quantize8_kernel<4><<<(int)g, 256, 0, st>>>(kb, vb, n8, kqb, ksb, vqb, vsb); break;
      case 8: kv_quantize8_kernel<8><<<(int)g, 256, 0, st>>>(kb, vb, n8, kqb, ksb, vqb, vsb); break;
      case 16: kv_quantize8_kernel<16><<<(int)g, 256, 0, st>>>(kb, vb, n8, kqb, ksb, vqb, vsb); break;
      case 32: kv_quantize8_kernel<32><<<(int)g, 256, 0, st>>>(kb, vb, n8, kqb, ksb, vqb, vsb); break;
      default: kv_quantize8_kernel<64><<<(int)g, 256, 0, st>>>(kb, vb, n8, kqb, ksb, vqb, vsb); break;
    }
    return hipGetLastError();
  }
  const int grid = (int)((rows + 3) / 4);
  const int jn = (D + 63) / 64;
  if (jn <= 1) kv_quantize_kernel<1><<<grid, 256, 0, st>>>(kb, vb, (int)rows, D, kqb, ksb, vqb, vsb);
  else if (jn <= 2) kv_quantize_kernel<2><<<grid, 256, 0, st>>>(kb, vb, (int)rows, D, kqb, ksb, vqb, vsb);
  else if (jn <= 4) kv_quantize_kernel<4><<<grid, 256, 0, st>>>(kb, vb, (int)rows, D, kqb, ksb, vqb, vsb);
  else if (jn <= 8) kv_quantize_kernel<8><<<grid, 256, 0, st>>>(kb, vb, (int)rows, D, kqb, ksb, vqb, vsb);
  else kv_quantize_kernel<16><<<grid, 256, 0, st>>>(kb, vb, (int)rows, D, kqb, ksb, vqb, vsb);
  return hipGetLastError();
}

hipError_t launch_kv_dequantize(const void* kq, const void* ks, const void* vq, const void* vs, int64_t numel, int D,
                                void* ko, void* vo, hipStream_t st) {
  const int64_t n8 = numel / 8;
  int64_t g = (n8 + 255) / 256;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  kv_dequantize_kernel<<<(int)g, 256, 0, st>>>(static_cast<const uint8_t*>(kq), static_cast<const uint16_t*>(ks),
                                              static_cast<const uint8_t*>(vq), static_cast<const uint16_t*>(vs), n8, D,
                                              static_cast<uint16_t*>(ko), static_cast<uint16_t*>(vo));
  return hipGetLastError();
}

}  // namespace qlq
