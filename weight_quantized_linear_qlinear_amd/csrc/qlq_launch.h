// Host-side interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <atomic>
#include <stddef.h>
#include <stdint.h>

namespace qlq {

enum Scheme : int { kW8A16 = 0, kW8A8 = 1 };

// How one GEMM call is cut into workgroups.
struct GemmPlan {
  int kind = 0;             // 0: small-M family (16-row groups), 1: large-M register-staged
                            // (any K), 2: large-M direct-to-LDS (K % 64 == 0)
  int cfg = 0;              // kind 2: tile configuration (see gemm_mfma.hip)
  int S = 1;                // split-K factor (workgroups sharing one output tile)
  int units_per_split = 0;  // K units per split (small-M: 64/128 inputs; kind 2: LDS stages)
  int units_per_wave = 0;   // small-M: K units per wave
  int waves = 4;            // small-M: waves per workgroup (4, 8 or 16)
  int ct = 1;               // small-M: 16-column tiles per workgroup (1, 2 or 4)
  int rw = 1;               // small-M: 16-row groups per workgroup (1 or 2)
  int BM = 0, BN = 0;       // large-M: workgroup tile
  int tiles = 0;            // output tiles (small: 16-column blocks)
  int grid = 0;             // workgroups launched
  size_t ws_bytes = 0;      // workspace: counters + split-K partials
  size_t ws_counter_bytes = 0;
};

// `fast`: K % 64 == 0 and x 16-byte aligned (enables kind 2).
GemmPlan plan_gemm(int scheme, int qtype, int64_t M, int64_t K, int64_t N, bool fast);

// Arguments every GEMM kernel receives (plain pointers and sizes).
struct GemmArgs {
  const void* x;            // bf16 [M,K] (W8A16) or 1-byte codes [M,K] (W8A8)
  const uint8_t* w;         // packed weight tiles
  const float* w_scale;     // [N] or [1]
  int scale_per_tensor;
  void* y;                  // bf16 [M,N], or int32/fp32 [M,N] accumulators
  uint32_t* counters;       // [tiles] arrival counters (split-K only)
  float* partials;          // split-K partial sums
  uint32_t partials_bytes;  // size of the partial region
  int M, K, N, KT, NT;
  float input_scale;
  const float* row_scale;   // W8A8 per-token activation scales [M], or null (static input_scale)
  const uint16_t* bias;     // bf16 bias [N] added before the bf16 rounding, or null
  uint8_t* y_codes;         // W8A8: codes [M,N] of the bf16 output at next_scale (the next
  float next_scale;         //   layer's static activation quantization), or null
  int next_scale_rcp = 0;   // next_scale is fp32(a / qmax) for a bf16 a: RcpDivAny is exact
  int out_acc;
  int fast;                 // K % 64 == 0 and 16-byte aligned rows/pointers
};

hipError_t launch_gemm_small(int scheme, int qtype, const GemmPlan& plan, const GemmArgs& a,
                             hipStream_t st);
hipError_t launch_gemm_large(int scheme, int qtype, const GemmPlan& plan, const GemmArgs& a,
                             hipStream_t st);
hipError_t launch_gemm_mfma(int scheme, int qtype, const GemmPlan& plan, const GemmArgs& a,
                            hipStream_t st);
int mfma_cfg_tile_m(int cfg);
int mfma_cfg_tile_n(int cfg);
int mfma_cfg_bkt(int cfg);
int mfma_num_cfgs();
bool mfma_cfg_valid(int scheme, int cfg);

hipError_t launch_absmax_scale(const void* src, int is_bf16, int64_t numel, float qmax, float* out,
                               hipStream_t st);
hipError_t launch_pack_weight(const void* w, int is_bf16, int N, int K, int qtype, int per_tensor,
                              uint8_t* packed, float* w_scale, hipStream_t st);
hipError_t launch_unpack_weight(const uint8_t* packed, int N, int K, uint8_t* out, hipStream_t st);
hipError_t launch_quant_act(const void* x, int64_t numel, float s, int qtype, void* xq, hipStream_t st,
                            bool rcp = false);
hipError_t launch_kv_quantize(const void* k, const void* v, int64_t rows, int D, void* kq, void* ks, void* vq,
                              void* vs, hipStream_t st);
hipError_t launch_kv_dequantize(const void* kq, const void* ks, const void* vq, const void* vs, int64_t numel, int D,
                                void* ko, void* vo, hipStream_t st);
hipError_t launch_quant_act_dynamic(const void* x, int M, int K, int qtype, void* xq, float* x_scale,
                                   hipStream_t st);

// Raises kernel k's dynamic-LDS limit to `bytes` on the current device, once per
// device (bit d of `done` records device d; devices past 63 set it every call).
inline hipError_t set_lds_limit(const void* k, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_relaxed);
  return e;
}

}  // namespace qlq
