// Device-side building blocks shared by the qlq kernels (gfx950 only).
//
// Packed weight layout (the library's private format, written by the packer and
// read by every GEMM kernel): W[N, K] codes are cut into tiles of 16 output
// channels x 64 inputs, 1 KiB each.  Tile (nt, kt) lives at byte
// (nt * KT + kt) * 1024, KT = ceil(K / 64).  Inside a tile, byte
//     lane * 16 + i,   lane = (n % 16) + 16 * ((k % 64) / 16),   i = k % 16
// holds W[n, k].  So one 16-byte load by lane `lane` of a wave64 returns 16
// consecutive inputs of one output channel, a whole wave reads one contiguous
// KiB, and that register is exactly the per-lane B operand of a 16x16 MFMA
// (column n = lane % 16, k-group = lane / 16) for the int8 K=64 shape, half of
// it for the fp8 K=128 shape, and two bf16 K=32 operands after dequantization.
// Pad rows (n >= N) and pad inputs (k >= K) hold code 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTileN = 16;
constexpr int kTileK = 64;
constexpr int kTileBytes = 1024;

enum QType : int { kInt8 = 0, kFp8 = 1 };

// ---------------------------------------------------------------- conversions

// Two fp32 -> packed bf16x2 (round to nearest even: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

// fp32 -> e4m3fn code, round to nearest even, saturating at +-448 (the clamp runs
// first so the hardware convert never sees a value it would turn into NaN).
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float v) {
  float c = __builtin_amdgcn_fmed3f(v, 448.0f, -448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// Four fp32 -> four e4m3fn codes packed in a dword (byte i = value i).
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4_sat(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, 448.0f, -448.0f);
  b = __builtin_amdgcn_fmed3f(b, 448.0f, -448.0f);
  c = __builtin_amdgcn_fmed3f(c, 448.0f, -448.0f);
  d = __builtin_amdgcn_fmed3f(d, 448.0f, -448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// fp32 -> int8 code: round to nearest even, clamp to +-127.
__device__ __forceinline__ uint32_t f32_to_i8_sat(float v) {
  float r = __builtin_rintf(v);
  r = __builtin_amdgcn_fmed3f(r, 127.0f, -127.0f);
  return (uint32_t)((int)r) & 0xFFu;
}

// Epilogue bias: fp32(v + b[n]) for a bf16 bias, a separately rounded add (no
// contraction with the product that formed v).  No bias: v.
__device__ __forceinline__ float add_bias(float v, const uint16_t* bias, int n) {
#pragma clang fp contract(off)
  return bias ? v + bf16_bits_to_f32(bias[n]) : v;
}

__device__ __forceinline__ float add_bias_value(float v, float b) {
#pragma clang fp contract(off)
  return v + b;
}

// Activation codes: four bf16 (two dwords) -> four codes of sat(RNE(x / s)), an
// IEEE fp32 division per value (callers must not build with fast-math).
template <int QT>
__device__ __forceinline__ uint32_t quant4(uint32_t lo, uint32_t hi, float s) {
  float a = bf16_bits_to_f32(lo & 0xFFFF) / s, b = bf16_bits_to_f32(lo >> 16) / s;
  float c = bf16_bits_to_f32(hi & 0xFFFF) / s, d = bf16_bits_to_f32(hi >> 16) / s;
  if constexpr (QT == kFp8) return f32x4_to_e4m3x4_sat(a, b, c, d);
  return f32_to_i8_sat(a) | (f32_to_i8_sat(b) << 8) | (f32_to_i8_sat(c) << 16) | (f32_to_i8_sat(d) << 24);
}

// x / s through a reciprocal refined by one Newton step and one correction of the
// product (sign kept for zeros; a non-finite x keeps the plain product, inf or NaN
// as the division gives): about half the IEEE division's instructions.  Exhaustive
// runs on gfx950 found the int8 and e4m3 codes identical to the IEEE quotient's
// for every positive finite bf16 a and every bf16 x with |x| <= a, for the scales
// s = fp16(a / qmax) the KV codec stores (qmax 127 and 448) and s = fp32(a / qmax)
// >= 2^-100 (how the per-token quantizer and calibration form scales).  With
// ANY_X, quotients of magnitude >= 1024 (they saturate either code) keep the plain
// product, and the codes matched for every finite bf16 x whatever its magnitude,
// for the second kind of scale: the static quantizer and the requantizing epilogue
// use it when the host finds the caller's scale to be of that kind.
template <bool ANY_X>
struct RcpDivT {
  float s, r;
  __device__ __forceinline__ explicit RcpDivT(float s_) : s(s_) {
    const float r0 = __builtin_amdgcn_rcpf(s_);
    r = __builtin_fmaf(__builtin_fmaf(-s_, r0, 1.0f), r0, r0);
  }
  __device__ __forceinline__ float operator()(float x) const {
    const float q0 = x * r;
    const float rem = __builtin_fmaf(-s, q0, x);
    const float q1 = __builtin_copysignf(__builtin_fmaf(rem, r, q0), x);
    if constexpr (ANY_X) return (rem == rem && __builtin_fabsf(q0) < 1024.0f) ? q1 : q0;
    return rem == rem ? q1 : q0;
  }
};
using RcpDiv = RcpDivT<false>;
using RcpDivAny = RcpDivT<true>;

// quant4 with the division above (same codes within its checked domain).
template <int QT, class DIV>
__device__ __forceinline__ uint32_t quant4_rcp(uint32_t lo, uint32_t hi, const DIV& dv) {
  float a = dv(bf16_bits_to_f32(lo & 0xFFFF)), b = dv(bf16_bits_to_f32(lo >> 16));
  float c = dv(bf16_bits_to_f32(hi & 0xFFFF)), d = dv(bf16_bits_to_f32(hi >> 16));
  if constexpr (QT == kFp8) return f32x4_to_e4m3x4_sat(a, b, c, d);
  return f32_to_i8_sat(a) | (f32_to_i8_sat(b) << 8) | (f32_to_i8_sat(c) << 16) | (f32_to_i8_sat(d) << 24);
}

// One bf16 (bits) -> its activation code sat(RNE(x / s)), as quant4.
template <int QT>
__device__ __forceinline__ uint32_t quant1(uint32_t b, float s) {
  const float v = bf16_bits_to_f32(b) / s;
  if constexpr (QT == kFp8) return f32x4_to_e4m3x4_sat(v, 0.0f, 0.0f, 0.0f) & 0xFFu;
  return f32_to_i8_sat(v);
}

// bf16 output element y[o] = bf16(val) and, with a code buffer, codes[o] = the
// activation code of that bf16 value at scale s (requantization for the next layer),
// through RcpDivAny when `rcp` is set (s of the checked kind).
template <int QT>
__device__ __forceinline__ void store_bf16_requant(void* y, uint8_t* codes, int64_t o, float val, float s,
                                                   bool rcp = false) {
  const __bf16 h = (__bf16)val;
  reinterpret_cast<__bf16*>(y)[o] = h;
  if (codes) {
    const uint32_t b = __builtin_bit_cast(uint16_t, h);
    if (rcp) {
      const float v = RcpDivAny(s)(bf16_bits_to_f32(b));
      codes[o] = (uint8_t)(QT == kFp8 ? (f32x4_to_e4m3x4_sat(v, 0.0f, 0.0f, 0.0f) & 0xFFu) : f32_to_i8_sat(v));
    } else {
      codes[o] = (uint8_t)quant1<QT>(b, s);
    }
  }
}

// Dequantize 8 codes (two dwords) to 8 bf16 = bf16(fp32(q) * s), one fp32
// rounding for the product and one for the bf16 cast.
template <int QT>
__device__ __forceinline__ bf16x8 dequant8(uint32_t d0, uint32_t d1, float s, float s_m128) {
  u32x4 r;
  if constexpr (QT == kFp8) {
    f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)d0, false);
    f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)d0, true);
    f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)d1, false);
    f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)d1, true);
    r.x = pack_bf16x2(a.x * s, a.y * s);
    r.y = pack_bf16x2(b.x * s, b.y * s);
    r.z = pack_bf16x2(c.x * s, c.y * s);
    r.w = pack_bf16x2(d.x * s, d.y * s);
  } else {
    // Flip the sign bit of every byte: u = q + 128 in [1, 255] converts with
    // v_cvt_f32_ubyteN; then fma(u, s, -128 s) = q * s with a single rounding
    // (-128 s is exact, and fma rounds the exact u*s - 128 s once).
    uint32_t e0 = d0 ^ 0x80808080u, e1 = d1 ^ 0x80808080u;
    float f0 = (float)(e0 & 0xFF), f1 = (float)((e0 >> 8) & 0xFF);
    float f2 = (float)((e0 >> 16) & 0xFF), f3 = (float)(e0 >> 24);
    float f4 = (float)(e1 & 0xFF), f5 = (float)((e1 >> 8) & 0xFF);
    float f6 = (float)((e1 >> 16) & 0xFF), f7 = (float)(e1 >> 24);
    r.x = pack_bf16x2(__builtin_fmaf(f0, s, s_m128), __builtin_fmaf(f1, s, s_m128));
    r.y = pack_bf16x2(__builtin_fmaf(f2, s, s_m128), __builtin_fmaf(f3, s, s_m128));
    r.z = pack_bf16x2(__builtin_fmaf(f4, s, s_m128), __builtin_fmaf(f5, s, s_m128));
    r.w = pack_bf16x2(__builtin_fmaf(f6, s, s_m128), __builtin_fmaf(f7, s, s_m128));
  }
  return __builtin_bit_cast(bf16x8, r);
}

// ---------------------------------------------------------------- MFMA wrappers
// 16x16 output tiles; lane l holds D[4*(l/16) + j][l % 16], j = 0..3.
// A operand: row l % 16, B operand: column l % 16; both carry the same k slots,
// so any assignment of real k indices to slots that A and B share is valid.

__device__ __forceinline__ f32x4 mfma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i32x4 mfma_i8_k64(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// fp8 (e4m3) x fp8 (e4m3), K = 128: format selectors 0/0, no block scaling.
__device__ __forceinline__ f32x4 mfma_fp8_k128(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x4 c) {
  i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ---------------------------------------------------------------- memory helpers

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ---------------------------------------------------------------- split-K handoff
// Partial sums of one output tile, written by several workgroups, are read back
// by the last one to arrive.  Workgroups of one launch may sit on different XCDs,
// each with its own L2, so the partials travel through agent-coherent accesses
// (16-byte buffer stores and loads with the sc1 cache policy, write-through /
// coherent across XCDs) instead of a device-wide fence, which would write back
// and invalidate a whole L2 per workgroup.  Order: partial stores -> wait until
// they are performed -> increment the arrival counter (a device atomic).
// The buffer descriptor's record count is the partial region's size, so the
// hardware range check drops any access outside it.

constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr int kCachePolicySc1 = 16;       // sc1: coherent at agent scope
constexpr int kCachePolicyNt = 2;         // nt: streaming (non-temporal)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, kBufferWord3);
}

// f32x4 index -> byte offset (the partial region is below 2^31 bytes)
__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t r, int64_t idx, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)(idx * 16), 0, kCachePolicySc1);
}

__device__ __forceinline__ f32x4 load_partial(__amdgpu_buffer_rsrc_t r, int64_t idx) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(idx * 16), 0, kCachePolicySc1));
}

// Waits until this thread's earlier stores are performed (vmcnt = 0).
__device__ __forceinline__ void wait_stores_performed() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ uint32_t arrive(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void reset_counter(uint32_t* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup -> logical index remap so that consecutive logical indices land on
// the same XCD (dispatch sends workgroup b to XCD b % 8).  Bijective on [0, T).
__device__ __forceinline__ int xcd_remap(int b, int T) {
  constexpr int kXcd = 8;
  int q = T / kXcd, r = T % kXcd;
  int x = b % kXcd, li = b / kXcd;
  int start = x * q + (x < r ? x : r);
  return start + li;
}

}  // namespace qlq
