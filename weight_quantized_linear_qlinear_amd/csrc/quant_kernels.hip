// Quantizers: weight absmax / scale / codes / packing, static activation
// calibration, static and dynamic (per-token) activation quantization.
//
// What they compute (symmetric, no zero point; "Nano-vLLM-MOE" README mirror,
// section "INT8 量化支持", scheme table and key-design list; "Nano-vLLM-MoE"
// README, sections "FP8 W8A16 weight-only quantization" and "FP8 W8A8 static
// quantization"):
//   scale = absmax / qmax (fp32 division; 1 when absmax is 0)
//   code  = sat(round-to-nearest-even(value / scale))  (fp32 division)
// These translation units must keep IEEE division: no fast-math flags.
#include "qlq_device.h"
#include "qlq_launch.h"

namespace qlq {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float load_w(const void* w, int is_bf16, int64_t idx) {
  if (is_bf16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(w)[idx]);
  return reinterpret_cast<const float*>(w)[idx];
}

__device__ __forceinline__ float scale_of(float absmax, float qmax) {
  return absmax == 0.0f ? 1.0f : absmax / qmax;
}

// ------------------------------------------------------------------ absmax reduction
// out_bits must hold 0 before the launch; |v| of finite floats compares like its
// bit pattern, so an unsigned atomic max is exact and order independent.
__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p) { *p = 0u; }

__global__ __launch_bounds__(256) void absmax_kernel(const void* src, int is_bf16, int64_t numel,
                                                     uint32_t* out_bits) {
  float m = 0.0f;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < numel; i += stride)
    m = fmaxf(m, fabsf(load_w(src, is_bf16, i)));
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(out_bits, __builtin_bit_cast(uint32_t, b));
  }
}

__global__ void finalize_scale_kernel(float* out, float qmax) {
  float am = __builtin_bit_cast(float, *reinterpret_cast<uint32_t*>(out));
  *out = scale_of(am, qmax);
}

// ------------------------------------------------------------------ weight packer
// One workgroup (256 threads) per 16-row block of W.  Phase 1: per-row absmax
// (per-channel) -> scale.  Phase 2: each wave produces whole 1 KiB tiles; lane
// `lane` writes the 16 codes of row (lane % 16), inputs 16 * (lane / 16) .. +15.
template <int QT>
__global__ __launch_bounds__(256) void pack_weight_kernel(const void* w, int is_bf16, int N, int K,
                                                          int KT, int per_tensor,
                                                          uint8_t* packed, float* w_scale) {
  const int nt = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float qmax = QT == kFp8 ? 448.0f : 127.0f;
  __shared__ float s_scale[16];

  if (per_tensor) {
    if (tid < 16) s_scale[tid] = w_scale[0];   // finalized by the absmax pass
  } else {
    // 4 waves x 4 rows each; a wave reduces one row at a time.
    for (int rr = 0; rr < 4; ++rr) {
      int r = wave * 4 + rr, n = nt * kTileN + r;
      float m = 0.0f;
      if (n < N)
        for (int k = lane; k < K; k += 64) m = fmaxf(m, fabsf(load_w(w, is_bf16, (int64_t)n * K + k)));
      m = wave_max(m);
      if (lane == 0) {
        float s = scale_of(m, qmax);
        s_scale[r] = s;
        if (n < N) w_scale[n] = s;
      }
    }
  }
  __syncthreads();

  const int r = lane & 15, g = lane >> 4;
  const int n = nt * kTileN + r;
  const float s = s_scale[r];
  for (int kt = wave; kt < KT; kt += 4) {
    uint32_t d[4];
    for (int c = 0; c < 4; ++c) {
      float v[4];
      for (int e = 0; e < 4; ++e) {
        int k = kt * kTileK + g * 16 + c * 4 + e;
        v[e] = (n < N && k < K) ? load_w(w, is_bf16, (int64_t)n * K + k) / s : 0.0f;
      }
      if constexpr (QT == kFp8) {
        d[c] = f32x4_to_e4m3x4_sat(v[0], v[1], v[2], v[3]);
      } else {
        d[c] = f32_to_i8_sat(v[0]) | (f32_to_i8_sat(v[1]) << 8) | (f32_to_i8_sat(v[2]) << 16) |
               (f32_to_i8_sat(v[3]) << 24);
      }
    }
    st16(packed + ((int64_t)nt * KT + kt) * kTileBytes + lane * 16, (u32x4){d[0], d[1], d[2], d[3]});
  }
}

__global__ __launch_bounds__(256) void unpack_weight_kernel(const uint8_t* packed, int N, int K, int KT,
                                                            uint8_t* out) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)N * K) return;
  int n = (int)(idx / K), k = (int)(idx % K);
  int lane = (n % kTileN) + 16 * ((k % kTileK) / 16);
  out[idx] = packed[((int64_t)(n / kTileN) * KT + k / kTileK) * kTileBytes + lane * 16 + (k % 16)];
}

// ------------------------------------------------------------------ activation quantizer
// Eight bf16 -> eight codes per thread on the vector path (16-byte load, 8-byte
// store); element by element for the tail or unaligned buffers.
template <int QT>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* x, int64_t numel, float s,
                                                        uint8_t* xq, int vec_ok, int rcp) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t nvec = vec_ok ? numel / 8 : 0;
  if (rcp) {                                                 // s of the kind RcpDivAny was checked for
    const RcpDivAny dv(s);
    for (int64_t i = tid; i < nvec; i += stride) {
      u32x4 v = ld16(x + i * 8);
      u32x2 o = {quant4_rcp<QT>(v.x, v.y, dv), quant4_rcp<QT>(v.z, v.w, dv)};
      *reinterpret_cast<u32x2*>(xq + i * 8) = o;
    }
  } else {
    for (int64_t i = tid; i < nvec; i += stride) {
      u32x4 v = ld16(x + i * 8);
      u32x2 o = {quant4<QT>(v.x, v.y, s), quant4<QT>(v.z, v.w, s)};
      *reinterpret_cast<u32x2*>(xq + i * 8) = o;
    }
  }
  for (int64_t i = nvec * 8 + tid; i < numel; i += stride) {
    float v = bf16_bits_to_f32(x[i]) / s;
    xq[i] = (uint8_t)(QT == kFp8 ? f32_to_e4m3_sat(v) : f32_to_i8_sat(v));
  }
}

// Dynamic per-token quantization.  RPW rows per workgroup, T = 256 / RPW threads
// per row.  Pass 1 reduces the row's absmax (x_scale[m] = absmax / qmax, 1 for
// an all-zero row: the weight rule); pass 2 writes the codes.  On the vector path
// (K % 8 == 0, 16-byte aligned rows) each thread keeps its first kCache 16-byte
// chunks of the row in registers between the passes and re-reads the rest.
template <int QT, int RPW>
__global__ __launch_bounds__(256) void quant_act_dynamic_kernel(const uint16_t* x, int M, int K, uint8_t* xq,
                                                                float* x_scale, int vec_ok) {
  constexpr int T = 256 / RPW, kCache = 8, WPR = T / 64;    // threads and waves per row
  const int tid = threadIdx.x, sub = tid / T, t = tid % T;
  const int m = blockIdx.x * RPW + sub;
  const bool live = m < M;
  const uint16_t* row = x + (int64_t)(live ? m : 0) * K;
  uint8_t* out = xq + (int64_t)(live ? m : 0) * K;
  const int nvec = (vec_ok && live) ? K / 8 : 0;
  u32x4 cache[kCache];
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < kCache; ++j) {
    const int i = t + j * T;
    cache[j] = i < nvec ? ld16(row + i * 8) : (u32x4){0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < kCache; ++j) {
    const uint32_t d[4] = {cache[j].x, cache[j].y, cache[j].z, cache[j].w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      am = fmaxf(am, fmaxf(fabsf(bf16_bits_to_f32(d[c] & 0xFFFF)), fabsf(bf16_bits_to_f32(d[c] >> 16))));
  }
  for (int i = t + kCache * T; i < nvec; i += T) {
    const u32x4 v = ld16(row + i * 8);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      am = fmaxf(am, fmaxf(fabsf(bf16_bits_to_f32(d[c] & 0xFFFF)), fabsf(bf16_bits_to_f32(d[c] >> 16))));
  }
  if (live)
    for (int k = nvec * 8 + t; k < K; k += T) am = fmaxf(am, fabsf(bf16_bits_to_f32(row[k])));
  am = wave_max(am);
  if constexpr (WPR > 1) {
    __shared__ float red[RPW][WPR];
    if ((tid & 63) == 0) red[sub][t >> 6] = am;
    __syncthreads();
    am = red[sub][0];
#pragma unroll
    for (int w = 1; w < WPR; ++w) am = fmaxf(am, red[sub][w]);
  }
  if (!live) return;
  const float s = scale_of(am, QT == kFp8 ? 448.0f : 127.0f);
  if (t == 0) x_scale[m] = s;
  // every x of the row is within its absmax, so RcpDiv gives the IEEE codes for
  // s >= 2^-100 (row-uniform branch; tinier rows keep the division)
  auto emit = [&](auto q4) {
#pragma unroll
    for (int j = 0; j < kCache; ++j) {
      const int i = t + j * T;
      if (i < nvec)
        *reinterpret_cast<u32x2*>(out + i * 8) = (u32x2){q4(cache[j].x, cache[j].y), q4(cache[j].z, cache[j].w)};
    }
    for (int i = t + kCache * T; i < nvec; i += T) {
      const u32x4 v = ld16(row + i * 8);
      *reinterpret_cast<u32x2*>(out + i * 8) = (u32x2){q4(v.x, v.y), q4(v.z, v.w)};
    }
  };
  if (s >= 0x1p-100f) {
    const RcpDiv dv(s);
    emit([&](uint32_t lo, uint32_t hi) { return quant4_rcp<QT>(lo, hi, dv); });
  } else {
    emit([&](uint32_t lo, uint32_t hi) { return quant4<QT>(lo, hi, s); });
  }
  for (int k = nvec * 8 + t; k < K; k += T) {
    const float v = bf16_bits_to_f32(row[k]) / s;
    out[k] = (uint8_t)(QT == kFp8 ? f32_to_e4m3_sat(v) : f32_to_i8_sat(v));
  }
}

// ------------------------------------------------------------------ launchers

static int grid_for(int64_t work, int per_block, int cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

hipError_t launch_absmax_scale(const void* src, int is_bf16, int64_t numel, float qmax, float* out,
                               hipStream_t st) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(out);
  zero_u32_kernel<<<1, 1, 0, st>>>(bits);
  absmax_kernel<<<grid_for(numel, 256 * 8, 2048), 256, 0, st>>>(src, is_bf16, numel, bits);
  finalize_scale_kernel<<<1, 1, 0, st>>>(out, qmax);
  return hipGetLastError();
}

hipError_t launch_pack_weight(const void* w, int is_bf16, int N, int K, int qtype, int per_tensor,
                              uint8_t* packed, float* w_scale, hipStream_t st) {
  int NT = (N + kTileN - 1) / kTileN, KT = (K + kTileK - 1) / kTileK;
  if (per_tensor) {
    hipError_t e = launch_absmax_scale(w, is_bf16, (int64_t)N * K, qtype == kFp8 ? 448.0f : 127.0f,
                                       w_scale, st);
    if (e != hipSuccess) return e;
  }
  if (qtype == kFp8)
    pack_weight_kernel<kFp8><<<NT, 256, 0, st>>>(w, is_bf16, N, K, KT, per_tensor, packed, w_scale);
  else
    pack_weight_kernel<kInt8><<<NT, 256, 0, st>>>(w, is_bf16, N, K, KT, per_tensor, packed, w_scale);
  return hipGetLastError();
}

hipError_t launch_unpack_weight(const uint8_t* packed, int N, int K, uint8_t* out, hipStream_t st) {
  int KT = (K + kTileK - 1) / kTileK;
  int64_t total = (int64_t)N * K;
  unpack_weight_kernel<<<(int)((total + 255) / 256), 256, 0, st>>>(packed, N, K, KT, out);
  return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, int64_t numel, float s, int qtype, void* xq, hipStream_t st, bool rcp) {
  int vec_ok = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && ((reinterpret_cast<uintptr_t>(xq) & 7) == 0);
  int grid = grid_for(vec_ok ? numel / 8 + 1 : numel, 256, 8192);
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(x);
  uint8_t* out = reinterpret_cast<uint8_t*>(xq);
  if (qtype == kFp8)
    quant_act_kernel<kFp8><<<grid, 256, 0, st>>>(xs, numel, s, out, vec_ok, rcp ? 1 : 0);
  else
    quant_act_kernel<kInt8><<<grid, 256, 0, st>>>(xs, numel, s, out, vec_ok, rcp ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_quant_act_dynamic(const void* x, int M, int K, int qtype, void* xq, float* x_scale,
                                   hipStream_t st) {
  const int vec_ok = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(xq) & 7) == 0);
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(x);
  uint8_t* out = reinterpret_cast<uint8_t*>(xq);
  // Few rows: a whole workgroup per row.  Many rows: one wave per row, as long as a
  // row's 16-byte chunks fit the 8-chunk register cache of its 64 threads (K <= 4096),
  // else a whole workgroup per row again, so that no thread loops over its chunks or
  // reads them twice (1024 x 11008: 17.5 -> 7 us).
  if (M < 1024 || (int64_t)K > 64 * 8 * 8) {
    if (qtype == kFp8)
      quant_act_dynamic_kernel<kFp8, 1><<<M, 256, 0, st>>>(xs, M, K, out, x_scale, vec_ok);
    else
      quant_act_dynamic_kernel<kInt8, 1><<<M, 256, 0, st>>>(xs, M, K, out, x_scale, vec_ok);
  } else {
    const int grid = (M + 3) / 4;
    if (qtype == kFp8)
      quant_act_dynamic_kernel<kFp8, 4><<<grid, 256, 0, st>>>(xs, M, K, out, x_scale, vec_ok);
    else
      quant_act_dynamic_kernel<kInt8, 4><<<grid, 256, 0, st>>>(xs, M, K, out, x_scale, vec_ok);
  }
  return hipGetLastError();
}

}  // namespace qlq
