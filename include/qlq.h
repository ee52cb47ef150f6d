/*
 * qlq.h -- C ABI of the MI355X (gfx950) quantized linear layer library (libqlq.so).
 *
 * The operations are the ones the pages describe for a quantized nn.Linear in an
 * LLM serving engine:
 *  - "Nano-vLLM-MoE" README (GitHub), section "FP8 W8A16 weight-only quantization"
 *    (Setup: FP8 weights dequantized to BF16 inside the GEMM, bf16 x bf16 dot with
 *    fp32 accumulation, bf16 out) and section "FP8 W8A8 static quantization"
 *    (offline-calibrated activation scales; a scaled FP8 GEMM with a custom epilogue).
 *  - "Nano-vLLM-MOE" README mirror, section "INT8 量化支持" (INT8 quantization
 *    support): scheme table (int8_w8a16, int8_w8a8_static) and key-design list
 *    (W8A16 dequantizes int8 weights to BF16 for a standard matmul; W8A8 static
 *    quantizes activations with one fixed, offline-calibrated scalar per layer and
 *    runs an INT8 GEMM with int32 accumulation).
 *
 * Notation: x is [M, K] (tokens x in-features), W is [N, K] (out x in), y = x W^T is
 * [M, N]; every matrix is row-major and densely packed (row stride = its column count).
 *
 * Conventions common to every call:
 *  - Pointers are DEVICE pointers (memory of the current HIP device) unless stated.
 *    The caller owns every buffer; the library never allocates, frees or
 *    synchronizes inside these calls.
 *  - Calls are asynchronous: they validate their arguments on the host, enqueue
 *    kernels on `stream` (0 = the null stream) and return.  A kernel fault shows
 *    up at the caller's next synchronization.  Nothing here blocks the host, so
 *    the calls may be recorded into a HIP graph.
 *  - Errors: QLQ_ERR_INVALID_ARG for a null pointer where one is required, a size
 *    below 1, a non-finite or non-positive scale, a scale count that is neither 1
 *    nor N, or a workspace that is too small; QLQ_ERR_UNSUPPORTED for an enum value
 *    the call does not know; QLQ_ERR_HIP when a launch fails.  Every argument is
 *    checked before the first kernel of a call is enqueued, so after
 *    QLQ_ERR_INVALID_ARG or QLQ_ERR_UNSUPPORTED nothing is enqueued; after
 *    QLQ_ERR_HIP, kernels the same call enqueued before the failed launch may
 *    still run.  qlq_last_error() returns a message (thread-local).
 *  - Numbers: bf16 and OCP FP8 e4m3fn (1-4-3, bias 7, max 448, no infinities;
 *    not the "fnuz" variant).  Non-finite inputs are not supported.
 */
#ifndef QLQ_H_
#define QLQ_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLQ_OK = 0,
  QLQ_ERR_INVALID_ARG = 1,
  QLQ_ERR_UNSUPPORTED = 2,
  QLQ_ERR_HIP = 3
} qlq_status;

/* Code type of quantized weights and activations. */
typedef enum {
  QLQ_INT8 = 0,        /* signed 8-bit integer codes in [-127, 127], qmax = 127 */
  QLQ_FP8_E4M3FN = 1   /* OCP e4m3fn codes, qmax = 448 */
} qlq_qtype;

/* Weight scale granularity. */
typedef enum {
  QLQ_PER_CHANNEL = 0, /* one fp32 scale per output channel n: w_scale[N] */
  QLQ_PER_TENSOR = 1   /* one fp32 scale for the whole matrix: w_scale[1] */
} qlq_granularity;

/* Output of qlq_qlinear_w8a8_static. */
typedef enum {
  QLQ_OUT_BF16 = 0,    /* y bf16 [M, N] after the scale epilogue */
  QLQ_OUT_ACC = 1      /* raw accumulators, no epilogue: int32 [M, N] for INT8,
                          fp32 [M, N] for FP8 */
} qlq_out;

/* Which GEMM a workspace is sized for. */
typedef enum {
  QLQ_SCHEME_W8A16 = 0,               /* qlq_qlinear_w8a16 */
  QLQ_SCHEME_W8A8_STATIC = 1,         /* qlq_qlinear_w8a8_static */
  QLQ_SCHEME_W8A8_STATIC_FUSED = 2,   /* qlq_qlinear_w8a8_static_fused */
  QLQ_SCHEME_W8A8_DYNAMIC = 3         /* qlq_qlinear_w8a8_dynamic */
} qlq_scheme;

/* ------------------------------------------------------------------ sizing */

/* Bytes of the packed weight buffer for an [N, K] weight: N and K are rounded up
 * to the tile grid (16 output channels x 64 inputs, 1 KiB per tile).  About N*K,
 * i.e. half of the bf16 weight ("~0.5GB (-50%)" in the INT8 performance table of
 * the "Nano-vLLM-MOE" mirror).  Returns 0 for N or K below 1. */
size_t qlq_packed_weight_bytes(int64_t N, int64_t K);

/* Bytes of workspace a GEMM call with these sizes needs (0 when the call needs
 * none).  The workspace holds split-K partial sums and arrival counters.  It must
 * be zero-filled before its first use; every completed call leaves the counters
 * at zero again, so one buffer can serve every later call on the same stream.
 * Calls that overlap in time (different streams) need separate workspaces. */
size_t qlq_workspace_bytes(qlq_scheme scheme, int64_t M, int64_t K, int64_t N, qlq_qtype qtype);

/* ------------------------------------------------------------------ weights */

/* Symmetric weight quantization and packing ("--scheme fp8_w8a16 / int8_w8a16 /
 * *_w8a8_static" export step of both nano-vllm-moe READMEs).
 *   w          [N, K] row-major, fp32 (w_is_bf16 = 0) or bf16 (w_is_bf16 = 1)
 *   scale      per channel: s[n] = absmax_k |w[n,k]| / qmax; per tensor: one s over
 *              all of W; fp32, correctly rounded division; an all-zero row
 *              (tensor) gets s = 1
 *   codes      q = round-to-nearest-even(w / s) (IEEE fp32 division), clamped to
 *              +-127 (INT8) or saturated to +-448 (e4m3fn)
 *   wq_packed  out, qlq_packed_weight_bytes(N, K) bytes, tiled layout private to
 *              the library (pad entries are code 0); 256-byte aligned
 *   w_scale    out, fp32 [N] (per channel) or [1] (per tensor)
 * Per tensor, the call runs a reduction before the packing kernel; both are
 * enqueued on `stream`. */
qlq_status qlq_quantize_weight(const void* w, int w_is_bf16, int64_t N, int64_t K,
                               qlq_qtype qtype, qlq_granularity granularity,
                               void* wq_packed, float* w_scale, hipStream_t stream);

/* Test hook: unpacks wq_packed into row-major 1-byte codes wq_rowmajor [N, K]. */
qlq_status qlq_unpack_weight(const void* wq_packed, int64_t N, int64_t K,
                             void* wq_rowmajor, hipStream_t stream);

/* --------------------------------------------------------------- activations */

/* Offline static calibration (the "--calib-samples 64 --calib-seqlen 512" step of
 * the INT8 section of the "Nano-vLLM-MOE" mirror): input_scale_out[0] =
 * absmax(x_calib) / qmax in fp32 (1 if x_calib is all zero).  x_calib is bf16 with
 * `numel` elements; input_scale_out is a device float. */
qlq_status qlq_calibrate_input_scale(const void* x_calib_bf16, int64_t numel, qlq_qtype qtype,
                                     float* input_scale_out, hipStream_t stream);

/* Static activation quantization with one fixed fp32 scalar (key-design list of
 * the INT8 section: no per-token reduction at run time):
 *   xq[m,k] = sat(round-to-nearest-even(x[m,k] / input_scale))
 * x bf16 [M, K]; xq [M, K] one byte per code; input_scale is a host value. */
qlq_status qlq_quantize_act_static(const void* x_bf16, int64_t M, int64_t K, float input_scale,
                                   qlq_qtype qtype, void* xq, hipStream_t stream);

/* Dynamic per-token activation quantization, the run-time alternative that the
 * key-design list of the INT8 section contrasts with static scaling (one more
 * reduction per call).  For every row m, with qmax = 127 (INT8) or 448 (e4m3fn):
 *   x_scale[m] = absmax_k |x[m,k]| / qmax   (fp32 division; 1 for an all-zero row)
 *   xq[m,k]    = sat(round-to-nearest-even(x[m,k] / x_scale[m]))   (fp32 division)
 * i.e. the weight quantizer's per-channel rule applied to each row of x.
 * x bf16 [M, K]; xq [M, K] one byte per code; x_scale fp32 [M] (device). */
qlq_status qlq_quantize_act_dynamic(const void* x_bf16, int64_t M, int64_t K, qlq_qtype qtype,
                                    void* xq, float* x_scale, hipStream_t stream);

/* -------------------------------------------------------------------- GEMMs */

/* Weight-only quantized linear (W8A16):
 *   y[m,n] = bf16( sum_k x[m,k] * bf16(fp32(q[n,k]) * s[n]) ), fp32 accumulation.
 * x bf16 [M, K]; wq_packed/w_scale from qlq_quantize_weight with the same N, K and
 * qtype; w_scale_numel is 1 (per tensor) or N (per channel); y bf16 [M, N].
 * workspace may be NULL when qlq_workspace_bytes(QLQ_SCHEME_W8A16, ...) is 0. */
qlq_status qlq_qlinear_w8a16(const void* x_bf16, int64_t M, int64_t K, int64_t N,
                             const void* wq_packed, const float* w_scale, int64_t w_scale_numel,
                             qlq_qtype qtype, void* y_bf16,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Allocation-free W8A16, for callers that cannot allocate or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, kernels and result as qlq_qlinear_w8a16, without the workspace:
 * the split-K partial sums and arrival counters live in a device array inside the
 * library (QLQ_NOALLOC_MAX_SCRATCH_BYTES, one copy per GPU, held until the process
 * ends).  The call allocates and frees nothing; its first call on a device looks up
 * that device's copy of the array.  The counters a call uses are cleared by a small
 * kernel before its GEMM, on `stream`.  Every call on one GPU shares that GPU's array,
 * so calls that may overlap in time on one GPU (different streams) race; serialize
 * them or use qlq_qlinear_w8a16 with separate workspaces.  A plan that needs more
 * scratch than the array holds is rejected with QLQ_ERR_INVALID_ARG (the 3B-scale
 * stack's shapes need at most 32 MiB + 4 KiB up to M = 1024). */
#define QLQ_NOALLOC_MAX_SCRATCH_BYTES ((size_t)32 * 1024 * 1024 + 4096)
qlq_status qlq_qlinear_w8a16_noalloc(const void* x_bf16, int64_t M, int64_t K, int64_t N,
                                     const void* wq_packed, const float* w_scale, int64_t w_scale_numel,
                                     qlq_qtype qtype, void* y_bf16, hipStream_t stream);

/* W8A8 static quantized linear on codes from qlq_quantize_act_static:
 *   acc[m,n] = sum_k xq[m,k] * q[n,k]   (INT8: exact int32; FP8: fp32)
 *   y[m,n]   = bf16( fp32(acc[m,n]) * fp32(input_scale * s[n]) )
 * out = QLQ_OUT_ACC writes acc itself (int32 or fp32 [M, N]) to y instead.
 * INT8 requires K <= 133144 so that |acc| < 2^31. */
qlq_status qlq_qlinear_w8a8_static(const void* xq, float input_scale,
                                   int64_t M, int64_t K, int64_t N,
                                   const void* wq_packed, const float* w_scale,
                                   int64_t w_scale_numel, qlq_qtype qtype, qlq_out out,
                                   void* y, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* W8A8 static with the next layer's static activation quantization in the
 * epilogue.  y is exactly what qlq_qlinear_w8a8_static writes with QLQ_OUT_BF16,
 * and in the same pass
 *   y_codes[m,n] = sat(round-to-nearest-even(fp32(y[m,n]) / next_scale))
 * (the bf16 value rounded first), i.e. the codes qlq_quantize_act_static(y,
 * next_scale, qtype) would write.  It serves a chain of projections whose next
 * layer is a static W8A8 layer with input scale next_scale (the key-design list
 * of the INT8 section of the "Nano-vLLM-MOE" mirror: one fixed scalar per layer,
 * no reduction at run time), so the next layer's quantization costs no extra
 * pass over y.  y bf16 [M, N]; y_codes [M, N] one byte per code, 16-byte
 * aligned.  The workspace is the one of qlq_qlinear_w8a8_static (size it with
 * QLQ_SCHEME_W8A8_STATIC).  Errors: those of qlq_qlinear_w8a8_static, plus a
 * non-finite or <= 0 next_scale and a null or misaligned y_codes
 * (QLQ_ERR_INVALID_ARG). */
qlq_status qlq_qlinear_w8a8_static_requant(const void* xq, float input_scale,
                                           int64_t M, int64_t K, int64_t N,
                                           const void* wq_packed, const float* w_scale,
                                           int64_t w_scale_numel, qlq_qtype qtype, float next_scale,
                                           void* y, void* y_codes, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream);

/* W8A8 static from bf16 activations: the same result as qlq_quantize_act_static
 * followed by qlq_qlinear_w8a8_static (identical codes, accumulators and
 * outputs), as one call.  The codes go through the workspace: one quantization
 * pass writes them, the GEMM reads them.  (Quantizing inside the GEMM kernels
 * measured slower on MI355X: the small-M kernel would divide every x element
 * once per workgroup of 16 to 64 output columns, and bf16 x tiles would double
 * the bytes each CU streams through the large-M main loop.)  Size the workspace with
 * qlq_workspace_bytes(QLQ_SCHEME_W8A8_STATIC_FUSED, ...); it follows the same
 * zero-fill rule as every other workspace. */
qlq_status qlq_qlinear_w8a8_static_fused(const void* x_bf16, float input_scale,
                                         int64_t M, int64_t K, int64_t N,
                                         const void* wq_packed, const float* w_scale,
                                         int64_t w_scale_numel, qlq_qtype qtype, qlq_out out,
                                         void* y, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/* W8A8 with per-token activation scales (codes and scales from
 * qlq_quantize_act_dynamic):
 *   acc[m,n] = sum_k xq[m,k] * q[n,k]   (as in qlq_qlinear_w8a8_static)
 *   y[m,n]   = bf16( fp32(acc[m,n]) * fp32(x_scale[m] * s[n]) )
 * x_scale fp32 [M] (device).  out, workspace and the INT8 K bound as for the
 * static call; size the workspace with QLQ_SCHEME_W8A8_DYNAMIC. */
qlq_status qlq_qlinear_w8a8_dynamic(const void* xq, const float* x_scale,
                                    int64_t M, int64_t K, int64_t N,
                                    const void* wq_packed, const float* w_scale,
                                    int64_t w_scale_numel, qlq_qtype qtype, qlq_out out,
                                    void* y, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* ------------------------------------------------------------ routed Linear */

/* The quantized Linear as a serving engine routes it by its checkpoint's scheme
 * (the quantization_type routing of the INT8 section's quick-start): y bf16 [M, N]
 * from bf16 x [M, K], with an optional bias and the opt-in small-batch fallback.
 *   scheme QLQ_SCHEME_W8A16         qlq_qlinear_w8a16
 *          QLQ_SCHEME_W8A8_STATIC   quantize with input_scale, then the static GEMM
 *          QLQ_SCHEME_W8A8_DYNAMIC  per-token quantization, then the dynamic GEMM
 *   bias_bf16            bf16 [N] or NULL: y = bf16(fp32(v + bias[n])), v the fp32
 *                        value the scale epilogue would round (added in fp32, not fused
 *                        with the product)
 *   bf16_fallback_max_m  W8A8 schemes: M <= this skips activation quantization and
 *                        computes the W8A16 result on the same weight codes and
 *                        scales (the key-design list's BF16 fallback for small
 *                        batches, 32 there); it changes the numerics, so 0 (off) is
 *                        the neutral value
 * The activation codes (and per-token scales) live in the workspace; size it with
 * qlq_linear_workspace_bytes (zero-fill rule as for every workspace). */
qlq_status qlq_linear(qlq_scheme scheme, const void* x_bf16, int64_t M, int64_t K, int64_t N,
                      const void* wq_packed, const float* w_scale, int64_t w_scale_numel,
                      qlq_qtype qtype, float input_scale, const void* bias_bf16,
                      int64_t bf16_fallback_max_m, void* y_bf16, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of qlq_linear for these sizes (covers the fallback too). */
size_t qlq_linear_workspace_bytes(qlq_scheme scheme, int64_t M, int64_t K, int64_t N, qlq_qtype qtype);

/* ---------------------------------------------------------------- KV cache */

/* KV-cache codec: K as int8 with a scale per group of 32 channels, V as FP8 with a scale
 * per token and head, both computed at run time ("Nano-vLLM-MoE" README, section "KV cache
 * compression", its Setup list: float16 scales).  K and V are bf16 [T, H, D] (tokens, KV heads, head_dim), D a multiple of
 * 32 (at most 1024).  Scales are IEEE binary16 bit patterns.
 *   K, per (t, h, group g of channels 32g .. 32g+31):
 *     k_scales[t,h,g] = fp16(absmax / 127)  (fp32 division, round to nearest even,
 *                       saturating at 65504; 1 for an all-zero group; 2^-24 when a
 *                       positive absmax would round to 0)
 *     k_codes[t,h,d]  = clamp(round-to-nearest-even(k / fp32(k_scales)), -127, 127)
 *   V, per (t, h): v_scales[t,h] = fp16(absmax_d |v[t,h,d]| / 448) (same rules),
 *     v_codes[t,h,d] = e4m3fn_sat(round-to-nearest-even(v / fp32(v_scales)))
 * k_codes int8 [T,H,D], k_scales [T,H,D/32], v_codes e4m3fn [T,H,D], v_scales [T,H].
 * Per (t, h) this stores 2D + D/16 + 2 bytes: 0.5195 of bf16 at D = 128. */
qlq_status qlq_kv_quantize(const void* k_bf16, const void* v_bf16, int64_t T, int64_t H, int64_t D,
                           void* k_codes, void* k_scales, void* v_codes, void* v_scales,
                           hipStream_t stream);

/* Decoding for attention: k[t,h,d] = bf16(fp32(k_code) * fp32(k_scale of its group)),
 * v[t,h,d] = bf16(fp32(v_code) * fp32(v_scale[t,h])).  Code buffers must be 8-byte
 * aligned and the bf16 outputs 16-byte aligned. */
qlq_status qlq_kv_dequantize(const void* k_codes, const void* k_scales, const void* v_codes,
                             const void* v_scales, int64_t T, int64_t H, int64_t D,
                             void* k_bf16, void* v_bf16, hipStream_t stream);

/* ------------------------------------------------------------- test hooks */

/* The launch plan a GEMM call takes for these sizes when x is 16-byte aligned (what
 * the tests use to show which kernel configuration a case reaches).  kind 0 is the
 * small-M family (M <= 16, or up to 128 rows with K a multiple of 64; tile_m = 16
 * rows per workgroup, tile_n = 16, 32 or 64 columns per workgroup, `waves` waves per
 * workgroup), 1 the register-staged large-M kernel
 * (K not a multiple of 64), 2 the direct-to-LDS large-M kernel with tile
 * configuration `cfg` (-1 otherwise).  split_k is the
 * number of K slices per output tile, grid the workgroups launched and
 * workspace_bytes what the call needs (0 without split-K).  Host only: nothing is
 * enqueued.  Errors as for the GEMM calls' size and enum checks. */
typedef struct {
  int32_t kind, cfg, split_k, tile_m, tile_n, waves, grid;
  int64_t workspace_bytes;
} qlq_plan_info;
qlq_status qlq_gemm_plan(qlq_scheme scheme, int64_t M, int64_t K, int64_t N, qlq_qtype qtype,
                         qlq_plan_info* info);

/* 1 when the activation quantizers divide by scale s with a reciprocal refined by
 * one Newton step and one correction of the product instead of the IEEE division:
 * s = fp32(a / qmax) for a positive finite bf16 a and qmax 127 or 448 (what
 * calibration and the per-token quantizer produce) and s >= 2^-100.  For those
 * scales the refined division gives the IEEE quotient's codes for every finite
 * bf16 x; every other scale keeps the IEEE division (returns 0).  Host only. */
int qlq_scale_is_calibrated(float s);

/* ------------------------------------------------------------------- errors */

const char* qlq_status_string(qlq_status status);
const char* qlq_last_error(void);

/* Library version string, e.g. "qlq 0.1.0 gfx950". */
const char* qlq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QLQ_H_ */
