// Large-M (prefill) quantized GEMM family on the gfx950 matrix cores.
//
// Prefill is compute bound ("Nano-vLLM-MOE" mirror, Llama 3.1 8B section: prefill
// leans on compute; "tiny-vLLM" README, "Quantization Results": the quantized paths
// lose most of their ground at prefill), so each workgroup computes a BM x BN
// output tile with 16x16 MFMAs fed from LDS:
//   W8A16:     weight codes are dequantized once per workgroup while they are
//              staged (bf16(fp32(q) * s[n])), then v_mfma_f32_16x16x32_bf16
//   W8A8 INT8: codes staged as they are, v_mfma_i32_16x16x64_i8 (exact int32)
//   W8A8 FP8:  codes staged as they are, v_mfma_f32_16x16x128_f8f6f4
// LDS holds every operand fragment in "lane order" (fragment f, lane l at byte
// f * 1024 + l * 16), so each ds_read_b128 / ds_write_b128 of a wave touches one
// contiguous KiB: no bank conflicts and no swizzle.  Two LDS stages: the global
// loads of stage t+1 are issued before the MFMAs of stage t.
// Workgroups are renumbered so that tiles sharing weight columns run on the same
// XCD (one L2 per XCD).  With S > 1 K-slices per tile, slices publish partial
// sums to the workspace and the last to arrive adds them in slice order.
#include "qlq_device.h"
#include "qlq_launch.h"

namespace qlq {

namespace {

template <int QT, int SCH>
struct LargeTraits {
  static constexpr int kBKT = SCH == kW8A16 ? 1 : 2;          // 64-input tiles per stage
  static constexpr int kPlanes = SCH == kW8A16 ? 2 : 1;       // KiB fragments per 16 x 64 block
  static constexpr bool kIntAcc = (SCH == kW8A8 && QT == kInt8);
};

__device__ __forceinline__ u32x4 lds16(const uint8_t* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void sts16(uint8_t* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}

template <bool FAST>
__device__ __forceinline__ u32x4 load_bf16x8(const uint16_t* row, int k, int K) {
  if constexpr (FAST) {
    return ld16(row + k);
  } else {
    uint32_t v[4];
    for (int e = 0; e < 4; ++e) {
      uint32_t a = (k + 2 * e < K) ? row[k + 2 * e] : 0u;
      uint32_t b = (k + 2 * e + 1 < K) ? row[k + 2 * e + 1] : 0u;
      v[e] = a | (b << 16);
    }
    return (u32x4){v[0], v[1], v[2], v[3]};
  }
}

template <bool FAST>
__device__ __forceinline__ u32x4 load_codes16(const uint8_t* row, int k, int K) {
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

template <int QT, int SCH, int BM, int BN, bool FAST>
__global__ __launch_bounds__(256, 2) void gemm_large_kernel(GemmArgs a, int S, int ups, int tiles_m,
                                                            int tiles_n) {
  using T = LargeTraits<QT, SCH>;
  constexpr int BKT = T::kBKT, PL = T::kPlanes;
  constexpr int MB = BM / 16, NB = BN / 16;                  // 16-row / 16-col blocks
  constexpr int A_FRAGS = MB * BKT * PL, B_FRAGS = NB * BKT * PL;
  constexpr int STAGE_BYTES = (A_FRAGS + B_FRAGS) * 1024;
  constexpr int TM = MB / 2, TN = NB / 2;                    // per-wave blocks (2 x 2 waves)
  // global -> LDS work per stage, in wave-loads (one KiB each)
  constexpr int A_LOADS = MB * BKT * PL / 4;                 // per wave
  constexpr int B_LOADS = NB * BKT / 4;                      // per wave (code tiles)
  static_assert(MB * BKT * PL % 4 == 0 && NB * BKT % 4 == 0, "tile split");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, g = lane >> 4;

  // ---- tile coordinates: XCD-grouped, m fastest so that the tiles of one
  // weight column block (and one K slice) are neighbours on the same XCD.
  const int total = tiles_m * tiles_n * S;
  const int logical = xcd_remap(blockIdx.x, total);
  const int tm = logical % tiles_m;
  const int rest = logical / tiles_m;
  const int s = rest % S;
  const int tn = rest / S;
  const int m0 = tm * BM, nt0 = tn * NB;
  const int tile_id = tn * tiles_m + tm;

  const int KU = (a.KT + BKT - 1) / BKT;                     // stages over all of K
  const int st_begin = s * ups;
  int st_end = st_begin + ups;
  if (st_end > KU) st_end = KU;
  const int nst = st_end - st_begin;

  // ---- per-thread load assignments (fixed for the whole K loop)
  // A: wave-load q = wave * A_LOADS + i  ->  (m block, k tile, plane)
  // B: wave-load q = wave * B_LOADS + i  ->  (n block, k tile)
  float bscale[B_LOADS], bscale_m128[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int q = wave * B_LOADS + i;
    const int nb = q % NB;
    const int n = (nt0 + nb) * kTileN + r;
    float sc = 0.0f;
    if (SCH == kW8A16) sc = a.scale_per_tensor ? a.w_scale[0] : (n < a.N ? a.w_scale[n] : 0.0f);
    bscale[i] = sc;
    bscale_m128[i] = -128.0f * sc;
  }

  u32x4 ra[A_LOADS], rb[B_LOADS];

  auto load_stage = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int q = wave * A_LOADS + i;
      const int plane = q % PL;
      const int kt_l = (q / PL) % BKT;
      const int mb = q / (PL * BKT);
      const int m = m0 + mb * 16 + r;
      const int kt = st * BKT + kt_l;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m < a.M && kt < a.KT) {
        if constexpr (SCH == kW8A16) {
          const uint16_t* row = reinterpret_cast<const uint16_t*>(a.x) + (int64_t)m * a.K;
          v = load_bf16x8<FAST>(row, kt * kTileK + g * 16 + plane * 8, a.K);
        } else {
          const uint8_t* row = reinterpret_cast<const uint8_t*>(a.x) + (int64_t)m * a.K;
          v = load_codes16<FAST>(row, kt * kTileK + g * 16, a.K);
        }
      }
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int q = wave * B_LOADS + i;
      const int nb = q % NB, kt_l = q / NB;
      const int ntile = nt0 + nb, kt = st * BKT + kt_l;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ntile < a.NT && kt < a.KT)
        v = ld16(a.w + ((int64_t)ntile * a.KT + kt) * kTileBytes + lane * 16);
      rb[i] = v;
    }
  };

  auto store_stage = [&](uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int q = wave * A_LOADS + i;     // fragment index == q (mb, kt_l, plane order)
      sts16(buf, q * 1024 + lane * 16, ra[i]);
    }
    uint8_t* bbuf = buf + A_FRAGS * 1024;
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int q = wave * B_LOADS + i;
      const int nb = q % NB, kt_l = q / NB;
      const int f = (nb * BKT + kt_l) * PL;
      if constexpr (SCH == kW8A16) {
        bf16x8 lo = dequant8<QT>(rb[i].x, rb[i].y, bscale[i], bscale_m128[i]);
        bf16x8 hi = dequant8<QT>(rb[i].z, rb[i].w, bscale[i], bscale_m128[i]);
        sts16(bbuf, f * 1024 + lane * 16, __builtin_bit_cast(u32x4, lo));
        sts16(bbuf, (f + 1) * 1024 + lane * 16, __builtin_bit_cast(u32x4, hi));
      } else {
        sts16(bbuf, f * 1024 + lane * 16, rb[i]);
      }
    }
  };

  f32x4 accf[TM][TN];
  i32x4 acci[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      accf[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
      acci[i][j] = (i32x4){0, 0, 0, 0};
    }

  auto compute_stage = [&](const uint8_t* buf) {
    const uint8_t* abuf = buf;
    const uint8_t* bbuf = buf + A_FRAGS * 1024;
#pragma unroll
    for (int kt_l = 0; kt_l < (QT == kFp8 && SCH == kW8A8 ? 1 : BKT); ++kt_l) {
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) {
        u32x4 fa[TM], fb[TN], fa2[TM], fb2[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int mb = wm * TM + i;
          fa[i] = lds16(abuf, ((mb * BKT + kt_l) * PL + pl) * 1024 + lane * 16);
          if constexpr (SCH == kW8A8 && QT == kFp8) fa2[i] = lds16(abuf, ((mb * BKT + 1) * PL) * 1024 + lane * 16);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int nb = wn * TN + j;
          fb[j] = lds16(bbuf, ((nb * BKT + kt_l) * PL + pl) * 1024 + lane * 16);
          if constexpr (SCH == kW8A8 && QT == kFp8) fb2[j] = lds16(bbuf, ((nb * BKT + 1) * PL) * 1024 + lane * 16);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (SCH == kW8A16) {
              accf[i][j] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[j]),
                                         accf[i][j]);
            } else if constexpr (QT == kInt8) {
              acci[i][j] = mfma_i8_k64(fa[i], fb[j], acci[i][j]);
            } else {
              accf[i][j] = mfma_fp8_k128(fa[i], fa2[i], fb[j], fb2[j], accf[i][j]);
            }
          }
      }
    }
  };

  // ---- main loop: two LDS stages, one barrier per stage
  if (nst > 0) {
    load_stage(st_begin);
    store_stage(smem);
    __syncthreads();
    for (int t = 0; t < nst; ++t) {
      uint8_t* cur = smem + (t & 1) * STAGE_BYTES;
      uint8_t* nxt = smem + ((t + 1) & 1) * STAGE_BYTES;
      if (t + 1 < nst) load_stage(st_begin + t + 1);
      compute_stage(cur);
      if (t + 1 < nst) store_stage(nxt);
      __syncthreads();
    }
  }

  // ---- split-K: publish partials in register order, last arrival sums in order
  constexpr int NV = TM * TN;   // f32x4 values per thread
  if (S > 1) {
    const __amdgpu_buffer_rsrc_t part = partial_rsrc(a.partials, a.partials_bytes);
    const int64_t mine = ((int64_t)s * tiles_m * tiles_n + tile_id) * NV * 256;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        store_partial(part, mine + (i * TN + j) * 256 + tid,
                      T::kIntAcc ? __builtin_bit_cast(f32x4, acci[i][j]) : accf[i][j]);
    wait_stores_performed();
    __shared__ uint32_t s_prev;
    __syncthreads();
    if (tid == 0) s_prev = arrive(&a.counters[tile_id]);
    __syncthreads();
    if (s_prev != (uint32_t)(S - 1)) return;
    // slices summed in order 0..S-1 (deterministic), each slice loaded at once
    const int64_t slice = (int64_t)tiles_m * tiles_n * NV * 256;
    const int64_t base = (int64_t)tile_id * NV * 256;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        accf[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        acci[i][j] = (i32x4){0, 0, 0, 0};
      }
    for (int q = 0; q < S; ++q) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const f32x4 p = load_partial(part, base + q * slice + (i * TN + j) * 256 + tid);
          if constexpr (T::kIntAcc) acci[i][j] += __builtin_bit_cast(i32x4, p);
          else accf[i][j] += p;
        }
    }
    if (tid == 0) reset_counter(&a.counters[tile_id]);
  }

  // ---- epilogue: block (i, j), lane (r, g), value jj -> y[m, n]
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = (nt0 + wn * TN + j) * kTileN + r;
    if (n >= a.N) continue;
    float sw = 0.0f;
    if (SCH == kW8A8 && !a.out_acc) sw = a.scale_per_tensor ? a.w_scale[0] : a.w_scale[n];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int m = m0 + (wm * TM + i) * 16 + 4 * g + jj;
        if (m >= a.M) continue;
        const int64_t o = (int64_t)m * a.N + n;
        if constexpr (SCH == kW8A16) {
          reinterpret_cast<__bf16*>(a.y)[o] = (__bf16)add_bias(accf[i][j][jj], a.bias, n);
        } else if (a.out_acc) {
          if constexpr (T::kIntAcc) reinterpret_cast<int32_t*>(a.y)[o] = acci[i][j][jj];
          else reinterpret_cast<float*>(a.y)[o] = accf[i][j][jj];
        } else {
          const float v = T::kIntAcc ? (float)acci[i][j][jj] : accf[i][j][jj];
          const float comb = (a.row_scale ? a.row_scale[m] : a.input_scale) * sw;   // fp32(s_x * s_w[n])
          store_bf16_requant<QT>(a.y, a.y_codes, o, add_bias(v * comb, a.bias, n), a.next_scale, a.next_scale_rcp);
        }
      }
  }
}

template <int QT, int SCH, int BM, int BN>
hipError_t launch_large_t(const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  using T = LargeTraits<QT, SCH>;
  constexpr int STAGE = (BM / 16 + BN / 16) * T::kBKT * T::kPlanes * 1024;
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  auto k = a.fast ? gemm_large_kernel<QT, SCH, BM, BN, true> : gemm_large_kernel<QT, SCH, BM, BN, false>;
  static std::atomic<uint64_t> lds_set[2];       // per instantiation, per device
  {
    const hipError_t e = set_lds_limit((const void*)k, 2 * STAGE, lds_set[a.fast ? 1 : 0]);
    if (e != hipSuccess) return e;
  }
  k<<<p.grid, 256, 2 * STAGE, st>>>(a, p.S, p.units_per_split, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_large(int scheme, int qtype, const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  if (scheme == kW8A16)
    return qtype == kFp8 ? launch_large_t<kFp8, kW8A16, 128, 128>(p, a, st)
                         : launch_large_t<kInt8, kW8A16, 128, 128>(p, a, st);
  return qtype == kFp8 ? launch_large_t<kFp8, kW8A8, 128, 128>(p, a, st)
                       : launch_large_t<kInt8, kW8A8, 128, 128>(p, a, st);
}

}  // namespace qlq
