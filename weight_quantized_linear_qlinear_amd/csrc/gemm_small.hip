// Small-M (decode, M <= 16; batched decode up to 128 rows in 16-row groups) quantized
// GEMM family.
//
// Decode is bound by reading the weights once ("Nano-vLLM-MoE" README, section
// "FP8 W8A16 weight-only quantization", Analysis: the FP8->BF16 dequant GEMM spends
// arithmetic to halve the weight bytes; "Nano-vLLM-MOE" mirror, Llama 3.1 8B section:
// decode leans on weight bandwidth).  So every weight byte is loaded exactly once
// with 16-byte coalesced loads (a wave reads one contiguous KiB tile per unit), a
// wave issues the loads of all its units before any arithmetic, each unit's
// arithmetic waits only for that unit's loads, and it runs on the matrix cores:
//   W8A16: codes -> bf16(fp32(q) * s[n]) in registers -> v_mfma_f32_16x16x32_bf16
//   W8A8 INT8: v_mfma_i32_16x16x64_i8 on the codes (exact int32)
//   W8A8 FP8:  v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3) on the codes
// The W8A8 epilogue takes a per-token scale per row when the call passes one.
// 16 rows fill the MFMA's 16-row A operand (rows >= M are zero).
//
// Work split: workgroup (rg, nt, s) owns rows [16 rg, 16 rg + 16 RW) (RW row groups),
// output columns [16 nt, 16 nt + 16 CT) (CT column tiles, see the kernel) and the s-th
// slice of K; its NW (4, 8 or 16) waves take consecutive sub-slices.  With several row
// groups (M > 16) the workgroups of one column tile and slice are consecutive in an
// XCD-grouped order, so they run together on one XCD and all but the first read the
// weights from its L2.  The
// wave accumulators are summed through LDS; with S > 1 slices per column block the
// partial sums go to the workspace and the last workgroup to arrive adds them
// in slice order (deterministic) and runs the epilogue.  The handoff uses
// agent-coherent partial stores and a device atomic counter (qlq_device.h).
#include "qlq_device.h"
#include "qlq_launch.h"

#include <type_traits>

namespace qlq {

namespace {

constexpr int kUnroll = 8;

template <int QT, int SCH>
struct SmallTraits {
  static constexpr int kTilesPerUnit = (SCH == kW8A8 && QT == kFp8) ? 2 : 1;
  static constexpr bool kIntAcc = (SCH == kW8A8 && QT == kInt8);
};

// 16 bf16 activations x[m, k .. k+15] (generic path: bounds-checked per element).
template <bool FAST>
__device__ __forceinline__ void load_x_bf16x16(const uint16_t* row, int k, int K, u32x4& lo, u32x4& hi) {
  if constexpr (FAST) {
    lo = ld16(row + k);
    hi = ld16(row + k + 8);
  } else {
    uint32_t v[8];
    for (int e = 0; e < 8; ++e) {
      uint32_t a = (k + 2 * e < K) ? row[k + 2 * e] : 0u;
      uint32_t b = (k + 2 * e + 1 < K) ? row[k + 2 * e + 1] : 0u;
      v[e] = a | (b << 16);
    }
    lo = (u32x4){v[0], v[1], v[2], v[3]};
    hi = (u32x4){v[4], v[5], v[6], v[7]};
  }
}

// 16 one-byte codes xq[m, k .. k+15].
template <bool FAST>
__device__ __forceinline__ u32x4 load_x_codes16(const uint8_t* row, int k, int K) {
  if constexpr (FAST) {
    return ld16(row + k);
  } else {
    uint32_t v[4];
    for (int e = 0; e < 4; ++e) {
      uint32_t d = 0;
      for (int b = 0; b < 4; ++b) {
        int kk = k + 4 * e + b;
        d |= (kk < K ? (uint32_t)row[kk] : 0u) << (8 * b);
      }
      v[e] = d;
    }
    return (u32x4){v[0], v[1], v[2], v[3]};
  }
}

// CT: 16-column tiles per workgroup (1, 2 or 4; more than one on the aligned path
// without K slices).  A wave's x fragments of a unit then serve all CT column tiles
// (each unit's CT weight loads are issued with its x loads), so every KiB of
// weights brings 1/CT as many x bytes through the vector memory path; at M = 16 in
// bf16 that is 2 KiB of x per KiB of weights with one tile.  A load batch holds
// 8 / CT units, so the registers in flight stay those of eight single-tile units.
// Four waves per SIMD (at most 128 registers per lane) let two 8-wave or four 4-wave
// workgroups share a CU (16 waves hold a CU alone); FP8 W8A8 with one tile keeps the
// registers its longer units take and runs three.
// RG: several 16-row groups (M > 16; aligned path).  A separate build, so that the
// single-group kernel keeps its code: the group arithmetic cost it 2-6 %.
// RW: row groups per workgroup (1, 2 or 4; more than one with one column tile).  Each unit's
// weights then serve every group (one load, RW MFMAs), and a load batch holds 8 / (CT RW) units
// so the registers in flight stay those of eight single-group units.
template <int QT, int SCH, bool FAST, int NW, int CT = 1, bool RG = false, int RW = 1>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(
    (NW == 16 || (SCH == kW8A8 && QT == kFp8 && CT == 1)) ? 1 : 4))) void gemm_small_kernel(GemmArgs a, int S, int ups,
                                                                                          int upw) {
  using T = SmallTraits<QT, SCH>;
  constexpr int TPU = T::kTilesPerUnit;
  constexpr int kU = kUnroll / (CT * RW);                  // units per load batch
  static_assert(RW == 1 || ((RW == 2 || RW == 4) && RG && CT == 1), "several row groups per workgroup: one column tile");
  static_assert(CT == 1 || ((CT == 2 || CT == 4) && FAST), "several column tiles on the aligned path only");
  static_assert(!RG || FAST, "several row groups on the aligned path only");
  // The wave index is uniform across the wave: reading it once keeps the unit range and
  // the loop control in scalar registers.  Chosen per build: it pays with one tile
  // except for 16-wave INT8 W8A16 (K-sliced down projections ran 3 % slower; the FP8
  // build spills without it), and with several tiles the register allocation spills
  // with it.
  constexpr bool kScalarWave = CT == 1 && (NW < 16 || SCH == kW8A8 || QT == kFp8);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = kScalarWave ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int NTG = (a.NT + CT - 1) / CT;                       // column-tile groups
  const int NRG = RG ? (a.M + 15) >> 4 : 1;                   // 16-row groups
  const int NRP = (NRG + RW - 1) / RW;                        // groups of RW row groups
  int rg = 0, nt, s;
  if constexpr (RG) {
    const int logical = xcd_remap(blockIdx.x, NTG * S * NRP);
    rg = logical % NRP * RW;
    nt = (logical / NRP % NTG) * CT;
    s = logical / NRP / NTG;
  } else {
    nt = (blockIdx.x % NTG) * CT;                             // first column tile of the group
    s = blockIdx.x / NTG;
  }
  const int m0 = rg * 16;                                     // first row of the group
  const int rows = RG ? (a.M - m0 < 16 ? a.M - m0 : 16) : a.M;
  // Rows of the second group of a pair (0 when the pair's first group is the last one).
  // Uniform; the clamp compiles to a vector instruction, so it is read back into a
  // scalar register for the buffer descriptor built from it.
  auto rows_of = [&](int q) {
    const int left = a.M - m0 - 16 * q;
    return __builtin_amdgcn_readfirstlane(left < 0 ? 0 : (left < 16 ? left : 16));
  };
  const int rows1 = RW >= 2 ? rows_of(1) : 0;
  const int rows2 = RW == 4 ? rows_of(2) : 0;
  const int rows3 = RW == 4 ? rows_of(3) : 0;
  const int KU = (a.KT + TPU - 1) / TPU;
  const int u_begin = s * ups + wave * upw;
  int u_end = u_begin + upw;
  if (u_end > (s + 1) * ups) u_end = (s + 1) * ups;
  if (u_end > KU) u_end = KU;

  const int r = lane & 15, g = lane >> 4;
  float sc[CT], sc_m128[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int nc = (nt + c) * kTileN + r;
    sc[c] = 0.0f;
    if (SCH == kW8A16) sc[c] = a.scale_per_tensor ? a.w_scale[0] : (nc < a.N ? a.w_scale[nc] : 0.0f);
    sc_m128[c] = -128.0f * sc[c];
  }

  // Row m0 + r of the A operand; rows >= M contribute zeros.
  const bool row_ok = r < rows;
  const uint8_t* wbase = a.w + (int64_t)nt * a.KT * kTileBytes + lane * 16;

  f32x4 accf[RW][CT];
  i32x4 acci[RW][CT];
#pragma unroll
  for (int q = 0; q < RW; ++q)
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      accf[q][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
      acci[q][c] = (i32x4){0, 0, 0, 0};
    }

  // A unit's arithmetic for column tile c: dequantize (W8A16) and feed the MFMA.
  auto unit_mma = [&](int c, const u32x4 (&wv)[TPU], const u32x4 (&xa)[RW][TPU], const u32x4 (&xb)[RW][TPU]) {
    if constexpr (SCH == kW8A16) {
      bf16x8 b0 = dequant8<QT>(wv[0].x, wv[0].y, sc[c], sc_m128[c]);
      bf16x8 b1 = dequant8<QT>(wv[0].z, wv[0].w, sc[c], sc_m128[c]);
#pragma unroll
      for (int q = 0; q < RW; ++q) {
        accf[q][c] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, xa[q][0]), b0, accf[q][c]);
        accf[q][c] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, xb[q][0]), b1, accf[q][c]);
      }
    } else if constexpr (QT == kInt8) {
#pragma unroll
      for (int q = 0; q < RW; ++q) acci[q][c] = mfma_i8_k64(xa[q][0], wv[0], acci[q][c]);
    } else {
#pragma unroll
      for (int q = 0; q < RW; ++q) accf[q][c] = mfma_fp8_k128(xa[q][0], xa[q][TPU - 1], wv[0], wv[TPU - 1], accf[q][c]);
    }
  };

  if constexpr (FAST) {
    // Aligned K and x: NU units (wave-uniform, 1..kUnroll) issue all their loads
    // with no branch in between, then run in order, so each unit's arithmetic waits
    // only for its own loads (the scheduling barriers keep issue order = unit
    // order).  A branch around a load would make the wait before the first unit a
    // wait for all of them.  The buffer range check returns zeros for activation
    // rows >= M and for the K tile past the end (odd tile count with two tiles per
    // unit); zero codes and zero activations add +0 to an accumulator that starts
    // at +0, so the sums are unchanged.  Offsets stay below 2^31: 16 rows of the
    // group and K <= 2^24 bound both buffers to 2^29 bytes.
    // The group's column tiles are consecutive in the packed weights; a tile past the
    // last one lies past the range and reads zeros.  With several column tiles the K
    // tile past the end of tile c would be the first K tile of tile c + 1, so that tile's
    // weight and x offsets are moved past both ranges instead.
    const int tiles_here = a.NT - nt < CT ? a.NT - nt : CT;
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.w) + (int64_t)nt * a.KT * kTileBytes, 0, tiles_here * a.KT * kTileBytes,
        kBufferWord3);
    constexpr int kEsz = SCH == kW8A16 ? 2 : 1;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.x)) + (int64_t)m0 * a.K * kEsz, 0,
        rows * a.K * kEsz, kBufferWord3);
    const uint32_t xrow = row_ok ? (uint32_t)((r * a.K + g * 16) * kEsz) : 0x80000000u;
    // Second group of a pair: named values rather than arrays, which the compiler
    // keeps in vector registers (every load then loops over the lanes' descriptors).
    // A group past the last row has an empty range: its loads return zeros.
    auto x_rsrc = [&](int q, int rq_rows) {
      return __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.x)) + (int64_t)(m0 + 16 * q) * a.K * kEsz, 0,
          rq_rows * a.K * kEsz, kBufferWord3);
    };
    const __amdgpu_buffer_rsrc_t xrs1 = RW == 1 ? xrs : x_rsrc(1, rows1);
    const __amdgpu_buffer_rsrc_t xrs2 = RW < 4 ? xrs : x_rsrc(2, rows2);
    const __amdgpu_buffer_rsrc_t xrs3 = RW < 4 ? xrs : x_rsrc(3, rows3);
    const uint32_t xrow1 = r < rows1 ? (uint32_t)((r * a.K + g * 16) * kEsz) : 0x80000000u;
    const uint32_t xrow2 = r < rows2 ? (uint32_t)((r * a.K + g * 16) * kEsz) : 0x80000000u;
    const uint32_t xrow3 = r < rows3 ? (uint32_t)((r * a.K + g * 16) * kEsz) : 0x80000000u;
    auto run = [&](int u0, auto nu) {
      constexpr int NU = decltype(nu)::value;
      u32x4 wv[NU][CT][TPU], xa[NU][RW][TPU], xb[NU][RW][TPU];
#pragma unroll
      for (int i = 0; i < NU; ++i) {
#pragma unroll
        for (int t = 0; t < TPU; ++t) {
          const int kt = (u0 + i) * TPU + t;
          const bool kt_in = TPU == 1 || CT == 1 || kt < a.KT;
          const uint32_t xo = kt_in ? xrow + (uint32_t)(kt * kTileK * kEsz) : 0x80000000u;
#pragma unroll
          for (int c = 0; c < CT; ++c)
            wv[i][c][t] = __builtin_amdgcn_raw_buffer_load_b128(
                wrs, kt_in ? (c * a.KT + kt) * kTileBytes + lane * 16 : (int)0x80000000u, 0, kCachePolicyNt);
          xa[i][0][t] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)xo, 0, 0);
          xb[i][0][t] = SCH == kW8A16 ? __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)(xo + 16), 0, 0)
                                      : (u32x4){0u, 0u, 0u, 0u};
          auto load_x = [&](int q, __amdgpu_buffer_rsrc_t rs, uint32_t xr) {
            const uint32_t xq = kt_in ? xr + (uint32_t)(kt * kTileK * kEsz) : 0x80000000u;
            xa[i][q][t] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)xq, 0, 0);
            xb[i][q][t] = SCH == kW8A16 ? __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(xq + 16), 0, 0)
                                        : (u32x4){0u, 0u, 0u, 0u};
          };
          if constexpr (RW >= 2) load_x(1, xrs1, xrow1);
          if constexpr (RW == 4) {
            load_x(2, xrs2, xrow2);
            load_x(3, xrs3, xrow3);
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // issue order = unit order
      }
#pragma unroll
      for (int i = 0; i < NU; ++i) {
#pragma unroll
        for (int c = 0; c < CT; ++c) unit_mma(c, wv[i][c], xa[i], xb[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int u0 = u_begin; u0 < u_end; u0 += kU) {
      const int nb = u_end - u0 < kU ? u_end - u0 : kU;
      if constexpr (kU == 2) {
        if (nb == 1) run(u0, std::integral_constant<int, 1>{});
        else run(u0, std::integral_constant<int, 2>{});
      } else if constexpr (kU == 8) {
        switch (nb) {
          case 1: run(u0, std::integral_constant<int, 1>{}); break;
          case 2: run(u0, std::integral_constant<int, 2>{}); break;
          case 3: run(u0, std::integral_constant<int, 3>{}); break;
          case 4: run(u0, std::integral_constant<int, 4>{}); break;
          case 5: run(u0, std::integral_constant<int, 5>{}); break;
          case 6: run(u0, std::integral_constant<int, 6>{}); break;
          case 7: run(u0, std::integral_constant<int, 7>{}); break;
          default: run(u0, std::integral_constant<int, 8>{}); break;
        }
      } else {
        switch (nb) {
          case 1: run(u0, std::integral_constant<int, 1>{}); break;
          case 2: run(u0, std::integral_constant<int, 2>{}); break;
          case 3: run(u0, std::integral_constant<int, 3>{}); break;
          default: run(u0, std::integral_constant<int, 4>{}); break;
        }
      }
    }
  } else {
    // Generic path: per-element bounds checks.
    for (int u0 = u_begin; u0 < u_end; u0 += kU) {
      u32x4 wv[kU][TPU];
      u32x4 xa[kU][RW][TPU];  // A operand bytes: 16 codes, or 8 bf16 (W8A16: values 0..7)
      u32x4 xb[kU][RW][TPU];  // W8A16: bf16 values 8 .. 15
#pragma unroll
      for (int i = 0; i < kU; ++i) {
        const bool live = u0 + i < u_end;
#pragma unroll
        for (int t = 0; t < TPU; ++t) {
          const int kt = (u0 + i) * TPU + t;
          const bool ok = live && kt < a.KT;
          wv[i][t] = ok ? ld16_stream(wbase + (int64_t)kt * kTileBytes) : (u32x4){0u, 0u, 0u, 0u};
          xa[i][0][t] = (u32x4){0u, 0u, 0u, 0u};
          xb[i][0][t] = (u32x4){0u, 0u, 0u, 0u};
          if constexpr (SCH == kW8A16) {
            if (ok && row_ok)
              load_x_bf16x16<FAST>(reinterpret_cast<const uint16_t*>(a.x) + (int64_t)(m0 + r) * a.K, kt * kTileK + g * 16,
                                   a.K, xa[i][0][t], xb[i][0][t]);
          } else {
            if (ok && row_ok)
              xa[i][0][t] = load_x_codes16<FAST>(reinterpret_cast<const uint8_t*>(a.x) + (int64_t)(m0 + r) * a.K,
                                                 kt * kTileK + g * 16, a.K);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kU; ++i) {
        if (u0 + i >= u_end) break;
        unit_mma(0, wv[i], xa[i], xb[i]);
      }
    }
  }

  // ---- sum the waves through LDS (wave c finishes column tile nt + c)
  __shared__ f32x4 red[RW * CT][NW][64];
#pragma unroll
  for (int q = 0; q < RW; ++q)
#pragma unroll
    for (int c = 0; c < CT; ++c)
      red[q * CT + c][wave][lane] = T::kIntAcc ? __builtin_bit_cast(f32x4, acci[q][c]) : accf[q][c];
  __syncthreads();
  // wave q * CT + c finishes column tile nt + c of row group rg + q (pairs have CT = 1)
  // (a group past M has nothing to finish)
  if (wave >= RW * CT || (RW == 1 && nt + wave >= a.NT) || (RW == 2 && wave == 1 && rows1 <= 0)) return;
  if (RW == 4 && wave > 0 && (wave == 1 ? rows1 : wave == 2 ? rows2 : rows3) <= 0) return;
  const int rq = RW == 1 ? 0 : wave;
  const int cw = CT == 1 ? 0 : wave;
  const int slot = rq * CT + cw;
  f32x4 tot;
  if constexpr (T::kIntAcc) {
    i32x4 t = __builtin_bit_cast(i32x4, red[slot][0][lane]);
    for (int w = 1; w < NW; ++w) t += __builtin_bit_cast(i32x4, red[slot][w][lane]);
    tot = __builtin_bit_cast(f32x4, t);
  } else {
    tot = red[slot][0][lane];
    for (int w = 1; w < NW; ++w) tot += red[slot][w][lane];
  }

  // ---- split-K (one column tile per workgroup): publish, count arrivals, last one
  // sums the slices in order
  if (CT == 1 && S > 1) {
    const __amdgpu_buffer_rsrc_t part = partial_rsrc(a.partials, a.partials_bytes);
    // partial of (slice, row group, column tile); one counter per (row group, column tile)
    const int64_t col = RG ? (int64_t)(rg + rq) * a.NT + nt : nt;
    const int64_t slice = RG ? (int64_t)NRG * a.NT : a.NT;
    store_partial(part, ((int64_t)s * slice + col) * 64 + lane, tot);
    wait_stores_performed();
    // The fences pin the order at the compiler level too: partial stores before the
    // arrival, partial loads after it (at workgroup scope they add no cache maintenance).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    uint32_t prev = 0;
    if (lane == 0) prev = arrive(&a.counters[col]);
    prev = __shfl(prev, 0, 64);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (prev != (uint32_t)(S - 1)) return;
    // slices summed in order 0..S-1, whichever workgroup arrived last (its own slice
    // from registers: one memory round trip less)
    if constexpr (T::kIntAcc) {
      i32x4 t = {0, 0, 0, 0};
      for (int q = 0; q < S; ++q)
        t += __builtin_bit_cast(i32x4, q == s ? tot : load_partial(part, ((int64_t)q * slice + col) * 64 + lane));
      tot = __builtin_bit_cast(f32x4, t);
    } else {
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q < S; ++q) t += q == s ? tot : load_partial(part, ((int64_t)q * slice + col) * 64 + lane);
      tot = t;
    }
    if (lane == 0) reset_counter(&a.counters[col]);
  }

  // ---- epilogue: lane holds D[4g + j][r] = y[m = m0 + 4g + j, n]
  const int n = (nt + cw) * kTileN + r;
  if (n >= a.N) return;
  float sw = 0.0f;
  if (SCH == kW8A8 && !a.out_acc) sw = a.scale_per_tensor ? a.w_scale[0] : a.w_scale[n];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 16 * rq + 4 * g + j;
    if (m >= a.M) break;
    const int64_t o = (int64_t)m * a.N + n;
    if constexpr (SCH == kW8A16) {
      reinterpret_cast<__bf16*>(a.y)[o] = (__bf16)add_bias(tot[j], a.bias, n);
    } else if (a.out_acc) {
      reinterpret_cast<float*>(a.y)[o] = tot[j];   // int32 bits or fp32
    } else {
      const float v = T::kIntAcc ? (float)__builtin_bit_cast(i32x4, tot)[j] : tot[j];
      const float comb = (a.row_scale ? a.row_scale[m] : a.input_scale) * sw;   // fp32(s_x * s_w[n])
      store_bf16_requant<QT>(a.y, a.y_codes, o, add_bias(v * comb, a.bias, n), a.next_scale, a.next_scale_rcp);
    }
  }
}

template <int QT, int SCH, int NW, bool RG>
hipError_t launch_small_rg(const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  // several row groups: planned for the aligned path only
  if (!a.fast) return hipErrorInvalidValue;
  if (p.ct == 1 && p.rw == 2) {
    // two row groups per workgroup: the weights loaded once for both
    if constexpr (SCH == kW8A8 && QT == kFp8 && NW == 16) return hipErrorInvalidValue;
    else gemm_small_kernel<QT, SCH, true, NW, 1, RG, 2><<<p.grid, NW * 64, 0, st>>>(a, p.S, p.units_per_split, p.units_per_wave);
  } else if (p.ct == 1 && p.rw == 4) {
    // four row groups per workgroup
    if constexpr (SCH == kW8A8 && QT == kFp8 && NW == 16) return hipErrorInvalidValue;
    else gemm_small_kernel<QT, SCH, true, NW, 1, RG, 4><<<p.grid, NW * 64, 0, st>>>(a, p.S, p.units_per_split, p.units_per_wave);
  } else if (p.rw != 1) {
    return hipErrorInvalidValue;
  } else if (p.ct == 2)
    gemm_small_kernel<QT, SCH, true, NW, 2, RG><<<p.grid, NW * 64, 0, st>>>(a, p.S, p.units_per_split, p.units_per_wave);
  else if (p.ct == 4)
    gemm_small_kernel<QT, SCH, true, NW, 4, RG><<<p.grid, NW * 64, 0, st>>>(a, p.S, p.units_per_split, p.units_per_wave);
  else if (p.ct != 1)
    return hipErrorInvalidValue;
  else if constexpr (SCH == kW8A8 && QT == kFp8 && NW == 16)
    return hipErrorInvalidValue;   // one FP8 W8A8 tile stops at 8 waves (16 would spill)
  else
    gemm_small_kernel<QT, SCH, true, NW, 1, RG><<<p.grid, NW * 64, 0, st>>>(a, p.S, p.units_per_split, p.units_per_wave);
  return hipGetLastError();
}

template <int QT, int SCH, int NW>
hipError_t launch_small_w(const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  if (a.M > 16) return launch_small_rg<QT, SCH, NW, true>(p, a, st);
  if (p.ct != 1) {
    // several column tiles per workgroup: planned for the aligned path without K slices only
    if (!a.fast || p.S != 1) return hipErrorInvalidValue;
    if (p.ct == 2)
      gemm_small_kernel<QT, SCH, true, NW, 2><<<p.grid, NW * 64, 0, st>>>(a, p.S, p.units_per_split, p.units_per_wave);
    else if (p.ct == 4)
      gemm_small_kernel<QT, SCH, true, NW, 4><<<p.grid, NW * 64, 0, st>>>(a, p.S, p.units_per_split, p.units_per_wave);
    else
      return hipErrorInvalidValue;
  } else if constexpr (SCH == kW8A8 && QT == kFp8 && NW == 16) {
    return hipErrorInvalidValue;   // one FP8 W8A8 tile stops at 8 waves (16 would spill)
  } else if (a.fast)
    gemm_small_kernel<QT, SCH, true, NW><<<p.grid, NW * 64, 0, st>>>(a, p.S, p.units_per_split, p.units_per_wave);
  else
    gemm_small_kernel<QT, SCH, false, NW><<<p.grid, NW * 64, 0, st>>>(a, p.S, p.units_per_split, p.units_per_wave);
  return hipGetLastError();
}

template <int QT, int SCH>
hipError_t launch_small_t(const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  switch (p.waves) {
    case 4: return launch_small_w<QT, SCH, 4>(p, a, st);
    case 8: return launch_small_w<QT, SCH, 8>(p, a, st);
    case 16: return launch_small_w<QT, SCH, 16>(p, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_small(int scheme, int qtype, const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  if (scheme == kW8A16)
    return qtype == kFp8 ? launch_small_t<kFp8, kW8A16>(p, a, st) : launch_small_t<kInt8, kW8A16>(p, a, st);
  return qtype == kFp8 ? launch_small_t<kFp8, kW8A8>(p, a, st) : launch_small_t<kInt8, kW8A8>(p, a, st);
}

}  // namespace qlq
