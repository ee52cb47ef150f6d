// Large-M (prefill) quantized GEMM on the gfx950 matrix cores, direct-to-LDS
// pipeline.  Used when K is a multiple of 64 and x is 16-byte aligned (every
// shape of the pages' models); other shapes take the register-staged kernel in
// gemm_large.hip.
//
// Prefill is compute bound ("Nano-vLLM-MOE" mirror, Llama 3.1 8B section: prefill
// leans on compute; "tiny-vLLM" README, "Quantization Results": the quantized paths
// lose most of their ground at prefill).  Design for gfx950, from measurements on
// the part (32x32 MFMA shapes run at twice the rate of the 16x16 ones for bf16
// and int8; LDS reads ~128 B/clk/CU; L2 -> LDS ~55 B/clk/CU):
//  * 32x32 MFMAs: v_mfma_f32_32x32x16_bf16 (W8A16), v_mfma_i32_32x32x32_i8 and
//    v_mfma_f32_32x32x64_f8f6f4 (W8A8);
//  * operands move global -> LDS with global_load_lds_dwordx4 (no VGPR staging)
//    into a ring of NSTAGE stages of 64 (or 128) inputs each; the loop body is
//    branch-free;
//  * the loop is software-pipelined by MFMA step (16 inputs for bf16, 32 for
//    int8, 64 for fp8): the LDS reads (and, for W8A16, the dequantization) of
//    step q+1 sit between the MFMAs of step q in a fixed order (sched_barrier
//    after each MFMA), and a stage's last step already prepares step 0 of the
//    next stage and issues the DMAs of the stage NSTAGE ahead, so the stage
//    barrier never leaves the matrix cores waiting on VALU or LDS;
//  * the bf16 output tile is staged through LDS so global stores are whole
//    16-byte chunks of rows;
//  * x rows that fill whole 128-byte lines per stage (bf16 x; 8-bit x with two
//    64-input tiles per stage) land in LDS row-major with the 16-byte chunks of
//    each line XOR-swizzled by the row, so every DMA instruction fetches 8 whole
//    lines (the vector L1 keeps a fixed number of requests in flight per CU, so
//    bytes per request set the streaming rate) and the MFMA reads hit distinct
//    banks; otherwise A fragments land in MFMA lane order.  B is the packed
//    weight tile copied verbatim (8 whole lines per instruction) and read with
//    per-lane addresses;
//  * W8A16 dequantizes B in registers after the LDS read, two codes after
//    each MFMA: bf16(fp32(q) * s[n]), the rounding the weight-only scheme prescribes;
//  * per-wave tiles of 128 rows (or 64 with 8 waves) keep LDS traffic within
//    budget; W8A16 tiles give each wave its own weight columns where they can,
//    so a column is dequantized once per workgroup (128x128 as 1 x 4 waves).
//
// K-slot convention (A and B agree, so the sum over k is unchanged): inside a
// 64-input tile, chunk c covers inputs 16c .. 16c+15.  For bf16 step (p, j)
// lane group kg (= lane / 32) holds inputs 16(2p + kg) + 8j .. +7; for int8 step
// p it holds chunk 2p + kg; for fp8 (one MFMA per 64-input tile) it holds chunks
// 2kg and 2kg + 1.
#include "qlq_device.h"
#include "qlq_launch.h"

#include <utility>

namespace qlq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 0x3) << 14));
}

// The same with every LDS read of the wave returned (lgkmcnt 0) as well.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds_reads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (((N >> 4) & 0x3) << 14));
}

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void*)g, (lds_void*)lds, 16, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// four fp32 -> four bf16 (RNE), first value in the lowest bytes
__device__ __forceinline__ u32x2 pack_bf16x4(f32x4 v) { return (u32x2){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}; }

template <int QT, int SCH>
struct MfmaTraits {
  static constexpr int kAElem = SCH == kW8A16 ? 2 : 1;       // bytes per x element
  // A fragments per 32-row block per stage (1 KiB each)
  static constexpr int kAFrags = SCH == kW8A16 ? 4 : 2;
  static constexpr bool kIntAcc = (SCH == kW8A8 && QT == kInt8);
};

// Dynamic LDS of one workgroup: the stage ring, or the staged bf16 output tile
// if that is larger (it reuses the ring after the main loop).
template <int QT, int SCH, int BM, int BN, int BKT, int NSTAGE>
constexpr int kLdsBytes() {
  constexpr int stage = ((BM / 32) * MfmaTraits<QT, SCH>::kAFrags + BN / 16) * BKT * 1024;
  constexpr int ring = NSTAGE * stage, out = BM * (BN * 2 + 16);
  return ring > out ? ring : out;
}

template <int QT, int SCH, int BM, int BN, int WM, int WN, int BKT, int NSTAGE, bool SPLIT>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 1) void gemm_mfma_kernel(GemmArgs a, int S, int ups, int tiles_m,
                                                                                 int tiles_n) {
  using T = MfmaTraits<QT, SCH>;
  constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  constexpr int NW = WAVES_M * WAVES_N, NT = NW * 64;         // waves, threads
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  constexpr int TM = WM / 32, TN = WN / 32;                 // 32x32 blocks per wave
  constexpr int A_FRAGS = (BM / 32) * T::kAFrags * BKT;      // per stage
  constexpr int B_TILES = (BN / 16) * BKT;                   // packed tiles per stage
  constexpr int STAGE = (A_FRAGS + B_TILES) * 1024;
  constexpr int A_PER_WAVE = A_FRAGS / NW, B_PER_WAVE = B_TILES / NW;
  constexpr int ROW_BYTES = kTileK * BKT * T::kAElem;        // bytes of one x row per stage
  constexpr bool LINE_A = ROW_BYTES >= 128;
  constexpr int LINES = ROW_BYTES / 128;
  static_assert(!LINE_A || (ROW_BYTES % 128 == 0 && A_FRAGS * 8 == BM * LINES), "A line layout");
  static_assert(LINE_A || SCH == kW8A8, "bf16 x always fills whole lines");
  constexpr int LOADS = A_PER_WAVE + B_PER_WAVE;             // DMA instructions per wave per stage
  static_assert(A_FRAGS % NW == 0 && B_TILES % NW == 0, "DMA split");
  static_assert(LOADS * (NSTAGE - 1) < 64, "vmcnt range");

  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int l32 = lane & 31, kg = lane >> 5;

  // tile coordinates: XCD-grouped, m fastest (tiles of one weight column block
  // and K slice are neighbours on one XCD)
  const int total = tiles_m * tiles_n * S;
  const int logical = xcd_remap(blockIdx.x, total);
  const int tm = logical % tiles_m;
  const int rest = logical / tiles_m;
  const int s = rest % S;
  const int tn = rest / S;
  const int m0 = tm * BM, nt0 = tn * (BN / 16);             // first 16-column weight tile
  const int tile_id = tn * tiles_m + tm;

  const int st_begin = s * ups;
  int st_end = st_begin + ups;
  const int KS = a.KT / BKT;                                 // stages over K (KT % BKT == 0)
  if (st_end > KS) st_end = KS;
  const int nst = st_end - st_begin;

  // ---- per-lane DMA source pointers (stage 0 of this slice); each stage adds 64 BKT inputs.
  // LINE_A (an x row of a stage spans whole 128-byte lines): the stage holds x
  // row-major, [row][line][8 chunks of 16 bytes].  One DMA instruction then
  // fetches 8 whole lines (one request per line).  The chunks are permuted so
  // that 16 consecutive rows reading the same chunk (one ds_read_b128 pass over
  // the 64 four-byte banks, 256 bytes) touch 16 distinct 16-byte bank groups:
  // with one line per row, even and odd rows sit in opposite bank halves and
  // chunk c of row r goes to position c ^ ((r / 2) % 8); with two or more lines
  // per row, rows 8..15 of each 16 swap lines 0 <-> 1 (and 2 <-> 3, ...) and
  // chunk c goes to position c ^ (r % 8).  Otherwise (8-bit x, one 64-input tile
  // per stage) A fragment f of a stage is f = (mb * BKT + kt) * kAFrags + q, in
  // MFMA lane order.
  const uint8_t* a_src[A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < A_PER_WAVE; ++i) {
    const int f = wave * A_PER_WAVE + i;                     // DMA instruction index in the stage
    if constexpr (LINE_A) {
      const int slot = f * 8 + (lane >> 3);                  // (row, line) slot, row-major
      const int r = slot / LINES;
      const int line = LINES == 1 ? 0 : (slot % LINES) ^ ((r >> 3) & 1);   // logical line held by this slot
      const int c = (lane & 7) ^ (LINES == 1 ? (r >> 1) & 7 : r & 7);     // chunk held by this position
      int row = m0 + r;
      row = row < a.M ? row : a.M - 1;                       // rows >= M: harmless duplicate
      a_src[i] = reinterpret_cast<const uint8_t*>(a.x) + ((int64_t)row * a.K + (int64_t)st_begin * BKT * kTileK) * T::kAElem +
                 line * 128 + c * 16;
    } else {
      const int mb = f / (T::kAFrags * BKT), kt = (f / T::kAFrags) % BKT, q = f % T::kAFrags;
      int row = m0 + mb * 32 + l32;
      row = row < a.M ? row : a.M - 1;
      int col;                                               // element offset inside the stage
      if constexpr (QT == kInt8) col = (2 * q + kg) * 16;    // step p = q
      else col = (2 * kg + q) * 16;                          // half h = q
      a_src[i] = reinterpret_cast<const uint8_t*>(a.x) +
                 ((int64_t)row * a.K + ((int64_t)st_begin * BKT + kt) * kTileK + col) * T::kAElem;
    }
  }
  // B tile b of a stage: b = nb16 * BKT + kt (16-column block, 64-input tile)
  const uint8_t* b_src[B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < B_PER_WAVE; ++i) {
    const int b = wave * B_PER_WAVE + i;
    int ntile = nt0 + b / BKT;
    ntile = ntile < a.NT ? ntile : a.NT - 1;                 // columns >= N: harmless duplicate
    b_src[i] = a.w + ((int64_t)ntile * a.KT + (int64_t)st_begin * BKT + b % BKT) * kTileBytes + lane * 16;
  }

  auto issue = [&](int st_local, int slot) {
    uint8_t* base = smem + slot * STAGE;
#pragma unroll
    for (int i = 0; i < A_PER_WAVE; ++i)
      dma16(a_src[i] + (int64_t)st_local * BKT * kTileK * T::kAElem, base + (wave * A_PER_WAVE + i) * 1024);
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i)
      dma16(b_src[i] + (int64_t)st_local * BKT * kTileBytes, base + (A_FRAGS + wave * B_PER_WAVE + i) * 1024);
  };

  // ---- per-lane column scales (W8A16)
  float sc[TN], sc_m128[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = nt0 * 16 + (wn * TN + j) * 32 + l32;
    float v = 0.0f;
    if (SCH == kW8A16) v = a.scale_per_tensor ? a.w_scale[0] : (n < a.N ? a.w_scale[n] : 0.0f);
    sc[j] = v;
    sc_m128[j] = -128.0f * v;
  }

  // W8A8 per-tensor weight scale, loaded before the main loop
  const float sw_t = (SCH == kW8A8 && a.scale_per_tensor) ? a.w_scale[0] : 1.0f;

  f32x16 accf[TM][TN];
  i32x16 acci[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      accf[i][j] = (f32x16){};
      acci[i][j] = (i32x16){};
    }

  // B read offset of lane (column l32 of the wave's 32-column block, 64-input tile kt, chunk c)
  auto b_off = [&](int nb32, int kt, int c) {
    const int col = nb32 * 32 + l32;                          // column inside the workgroup tile
    return (A_FRAGS + (col >> 4) * BKT + kt) * 1024 + ((col & 15) + 16 * c) * 16;
  };

  // LINE_A read offset of lane's row in row block i of this wave, 16-byte chunk c of the stage row
  auto a_off = [&](int i, int c) {
    const int r = (wm * TM + i) * 32 + l32;
    if constexpr (LINES == 1) return r * 128 + (((c & 7) ^ ((l32 >> 1) & 7)) << 4);
    else return (r * LINES + ((c >> 3) ^ ((l32 >> 3) & 1))) * 128 + (((c & 7) ^ (l32 & 7)) << 4);
  };

  // ---- W8A16 operand helpers for the software-pipelined loop below
  // DMA instruction idx (0 .. LOADS-1) of stage st_local into ring slot `slot`
  auto dma_one = [&](int st_local, int slot, int idx) {
    uint8_t* base = smem + slot * STAGE;
    if (idx < A_PER_WAVE)
      dma16(a_src[idx] + (int64_t)st_local * BKT * kTileK * T::kAElem, base + (wave * A_PER_WAVE + idx) * 1024);
    else
      dma16(b_src[idx - A_PER_WAVE] + (int64_t)st_local * BKT * kTileBytes,
            base + (A_FRAGS + wave * B_PER_WAVE + idx - A_PER_WAVE) * 1024);
  };
  // 16-input step q of a stage (q = 4 kt + 2 p + jj): A chunk of row block i, and
  // half h (4 inputs) of the B fragment of column block j from the stage's codes
  auto a_step = [&](const uint8_t* base, int q, int i) {
    return lds_read16(base + a_off(i, (q >> 2) * 8 + 4 * ((q >> 1) & 1) + 2 * kg + (q & 1)));
  };
  auto read_codes = [&](const uint8_t* base, u32x4 (&bc)[2 * BKT][TN]) {
#pragma unroll
    for (int h = 0; h < 2 * BKT; ++h)
#pragma unroll
      for (int j = 0; j < TN; ++j) bc[h][j] = lds_read16(base + b_off(wn * TN + j, h >> 1, 2 * (h & 1) + kg));
  };
  // Two codes of step q's B fragment of column block j (half h, pair e of its four
  // codes) -> two bf16 of fp32(q) * s, rounded as in dequant8.  INT8 flips the sign bits of
  // the word at pair 0 and keeps it for pair 1.
  uint32_t xw[TN][2];
  auto b_pair = [&](const u32x4 (&bc)[2 * BKT][TN], int q, int j, int h, int e) -> uint32_t {
    const u32x4 cw = bc[q >> 1][j];
    const uint32_t d = (q & 1) ? (h ? cw.w : cw.z) : (h ? cw.y : cw.x);
    if constexpr (QT == kFp8) {
      const f32x2 v = e ? __builtin_amdgcn_cvt_pk_f32_fp8((int)d, true) : __builtin_amdgcn_cvt_pk_f32_fp8((int)d, false);
      return pack_bf16x2(v.x * sc[j], v.y * sc[j]);
    } else {
      if (e == 0) xw[j][h] = d ^ 0x80808080u;
      const uint32_t x = xw[j][h] >> (16 * e);
      return pack_bf16x2(__builtin_fmaf((float)(x & 0xFF), sc[j], sc_m128[j]),
                         __builtin_fmaf((float)((x >> 8) & 0xFF), sc[j], sc_m128[j]));
    }
  };

  // ---- pipeline: NSTAGE-1 stages in flight ahead of the one being consumed.
  // The loop body is branch-free: the prefetch source is clamped to the last
  // stage, so past the end it re-reads a valid stage into a slot nobody reads,
  // and every iteration waits for the same vmcnt.
  if constexpr (SCH == kW8A16) {
    // W8A16: the dequantization (VALU) and LDS reads of step q+1 run between
    // the MFMAs of step q, in a fixed order (sched_barrier after each MFMA).
    // The stage barrier sits before a stage's last step: that step needs no
    // LDS of its own stage (its operands are already in registers), so it
    // reads and dequantizes step 0 of the next stage, and it issues the DMAs
    // of stage t + NSTAGE into the slot of stage t, whose last reader passed
    // the barrier.  Each stage's DMAs get NSTAGE - 1 whole stages to land.
    //
    // With one row of waves (WAVES_M == 1) every wave copies exactly the weight
    // tiles it reads (its own columns), so it may read the next stage's codes as
    // soon as its own DMAs of that stage are complete, one step before the
    // barrier, and dequantize the next stage's first step across all of the
    // last step's MFMAs.  With a two-stage ring that wait would come a step
    // sooner after the DMAs were issued, which measured slower, so two-stage
    // tiles keep the codes read after the barrier.
    constexpr int Q = 4 * BKT, NM = TM * TN, DPM = (LOADS + NM - 1) / NM, NP = 4 * TN;
    constexpr bool OWN_B = WAVES_M == 1 && NSTAGE >= 3;
    static_assert(!OWN_B || B_PER_WAVE == TN * 2 * BKT, "each wave copies the weight tiles of its own columns");
    static_assert(TM >= 2 && NM >= 3, "W8A16 pipeline shape: the last step schedules its work from MFMA 2 on");
    u32x4 bc[2 * BKT][TN], bcn[2 * BKT][TN];                  // codes of this stage and (OWN_B) the next
    u32x4 af[2][TM];
    uint32_t bq[2][TN][2][2];   // [buffer][column block][half][pair]: bf16x2 of the B operand
#pragma unroll
    for (int t = 0; t < NSTAGE; ++t) issue(t < nst ? t : nst - 1, t);
    wait_vmcnt<LOADS * (NSTAGE - 1)>();
    __syncthreads();
    read_codes(smem, bc);
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = a_step(smem, 0, i);
#pragma unroll
    for (int p = 0; p < NP; ++p) bq[0][p >> 2][(p >> 1) & 1][p & 1] = b_pair(bc, 0, p >> 2, (p >> 1) & 1, p & 1);
    for (int t = 0; t < nst; ++t) {
      const uint8_t* cur = smem + (t % NSTAGE) * STAGE;
      const uint8_t* nxt = smem + ((t + 1) % NSTAGE) * STAGE;   // past the end: a valid slot, unused
      const int pf = t + NSTAGE < nst ? t + NSTAGE : nst - 1;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int c = q & 1;
        if (OWN_B && q == Q - 2) wait_vmcnt<LOADS * (NSTAGE - 2)>();   // this wave's DMAs of stage t+1
        if (q == Q - 1) {
          // Stage t+1 visible, slot t free.  This wave's DMAs of stage t+1 are
          // complete (vmcnt) and its reads of slot t have returned (lgkmcnt),
          // so no release fence: one would also wait for the younger stages' DMAs.
          wait_vmcnt_lds_reads<LOADS * (NSTAGE - 2)>();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const int i = m / TN, j = m % TN;
          const u32x4 bv = (u32x4){bq[c][j][0][0], bq[c][j][0][1], bq[c][j][1][0], bq[c][j][1][1]};
          accf[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bv),
                                                                __builtin_bit_cast(bf16x8, af[c][i]), accf[i][j], 0, 0, 0);
          if (q + 1 < Q) {
            // step q+1's dequantization spread evenly over this step's MFMAs
#pragma unroll
            for (int p = 0; p < NP; ++p)
              if (m == p * NM / NP) bq[c ^ 1][p >> 2][(p >> 1) & 1][p & 1] = b_pair(bc, q + 1, p >> 2, (p >> 1) & 1, p & 1);
            if (m < TM) af[c ^ 1][m] = a_step(cur, q + 1, m);   // early in the step: ready by its end
            if (OWN_B && q == Q - 2 && m == 0) read_codes(nxt, bcn);
          } else {
#pragma unroll
            for (int d = 0; d < DPM; ++d)
              if (m * DPM + d < LOADS) dma_one(pf, t % NSTAGE, m * DPM + d);
            if (!OWN_B && m == 0) read_codes(nxt, bc);
            if (m == (OWN_B ? 0 : 1)) {
#pragma unroll
              for (int ii = 0; ii < TM; ++ii) af[c ^ 1][ii] = a_step(nxt, 0, ii);
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              if constexpr (OWN_B) {
                if (m == p * NM / NP) bq[c ^ 1][p >> 2][(p >> 1) & 1][p & 1] = b_pair(bcn, 0, p >> 2, (p >> 1) & 1, p & 1);
              } else {
                if (m == 2 + p * (NM - 2) / NP) bq[c ^ 1][p >> 2][(p >> 1) & 1][p & 1] = b_pair(bc, 0, p >> 2, (p >> 1) & 1, p & 1);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (OWN_B) {
#pragma unroll
        for (int h = 0; h < 2 * BKT; ++h)
#pragma unroll
          for (int j = 0; j < TN; ++j) bc[h][j] = bcn[h][j];
      }
    }
  } else {
    // W8A8: the same pipeline without dequantization.  A step is one MFMA
    // deep in K: 32 inputs (int8) or 64 (fp8, two 16-byte reads per operand).
    constexpr int Q = QT == kInt8 ? 2 * BKT : BKT, NM = TM * TN, NR = QT == kInt8 ? 1 : 2;
    constexpr int DPM = (LOADS + NM - 1) / NM;
    // operands of step q (int8: q = 2 kt + p, chunk 2p + kg; fp8: q = kt, chunks 2kg and 2kg + 1)
    auto read_a = [&](const uint8_t* base, int q, int i, u32x4 (&dst)[NR]) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int kt = QT == kInt8 ? q >> 1 : q;
        if constexpr (LINE_A) {
          dst[r] = lds_read16(base + a_off(i, QT == kInt8 ? kt * 4 + 2 * (q & 1) + kg : kt * 4 + 2 * kg + r));
        } else {
          const int f = ((wm * TM + i) * BKT + kt) * T::kAFrags + (QT == kInt8 ? (q & 1) : r);
          dst[r] = lds_read16(base + f * 1024 + lane * 16);
        }
      }
    };
    auto read_b = [&](const uint8_t* base, int q, int j, u32x4 (&dst)[NR]) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
        dst[r] = QT == kInt8 ? lds_read16(base + b_off(wn * TN + j, q >> 1, 2 * (q & 1) + kg))
                             : lds_read16(base + b_off(wn * TN + j, q, 2 * kg + r));
    };
    auto mma = [&](const u32x4 (&b)[NR], const u32x4 (&a)[NR], int i, int j) {
      if constexpr (QT == kInt8) {
        acci[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, b[0]), __builtin_bit_cast(i32x4, a[0]),
                                                           acci[i][j], 0, 0, 0);
      } else {
        const i32x8 bb = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w, (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
        const i32x8 aa = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w, (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
        accf[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bb, aa, accf[i][j], 0, 0, 0, 0, 0, 0);
      }
    };
    u32x4 af[2][TM][NR], bf[2][TN][NR];
#pragma unroll
    for (int t = 0; t < NSTAGE; ++t) issue(t < nst ? t : nst - 1, t);
    wait_vmcnt<LOADS * (NSTAGE - 1)>();
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TN; ++j) read_b(smem, 0, j, bf[0][j]);
#pragma unroll
    for (int i = 0; i < TM; ++i) read_a(smem, 0, i, af[0][i]);
    for (int t = 0; t < nst; ++t) {
      const uint8_t* cur = smem + (t % NSTAGE) * STAGE;
      const uint8_t* nxt = smem + ((t + 1) % NSTAGE) * STAGE;   // past the end: a valid slot, unused
      const int pf = t + NSTAGE < nst ? t + NSTAGE : nst - 1;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int c = q & 1;
        const uint8_t* src = q + 1 < Q ? cur : nxt;            // operands of the following step
        const int qn = q + 1 < Q ? q + 1 : 0;
        if (q == Q - 1) {                                      // as in the W8A16 loop
          wait_vmcnt_lds_reads<LOADS * (NSTAGE - 2)>();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          mma(bf[c][m % TN], af[c][m / TN], m / TN, m % TN);
          if (q == Q - 1) {
#pragma unroll
            for (int d = 0; d < DPM; ++d)
              if (m * DPM + d < LOADS) dma_one(pf, t % NSTAGE, m * DPM + d);
          }
          if (m == 0) {
#pragma unroll
            for (int j = 0; j < TN; ++j) read_b(src, qn, j, bf[c ^ 1][j]);
          }
          if (m % TN == TN - 1) read_a(src, qn, m / TN, af[c ^ 1][m / TN]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (Q & 1) {                                   // step 0 of the next stage landed in buffer 1
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < NR; ++r) af[0][i][r] = af[1][i][r];
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < NR; ++r) bf[0][j][r] = bf[1][j][r];
      }
    }
  }
  wait_vmcnt<0>();                                           // no DMA may outlive the loop

  // ---- split-K handoff (partials in register order)
  constexpr int NV = TM * TN * 4;                            // f32x4 per thread
  auto acc_vec = [&](int i, int j, int v) -> f32x4 {
    if constexpr (T::kIntAcc) {
      i32x16 c = acci[i][j];
      return __builtin_bit_cast(f32x4, (i32x4){c[4 * v], c[4 * v + 1], c[4 * v + 2], c[4 * v + 3]});
    } else {
      f32x16 c = accf[i][j];
      return (f32x4){c[4 * v], c[4 * v + 1], c[4 * v + 2], c[4 * v + 3]};
    }
  };
  if constexpr (SPLIT) {
    const __amdgpu_buffer_rsrc_t part = partial_rsrc(a.partials, a.partials_bytes);
    const int64_t slice = (int64_t)tiles_m * tiles_n * NV * NT;
    const int64_t base = (int64_t)tile_id * NV * NT;
    __shared__ uint32_t s_prev;
    // Publish, arrive, and the last to arrive sums.  Tiles with at most 16
    // accumulator vectors per thread (8 with eight waves) add the last workgroup's
    // own slice from registers instead of reading it back; larger tiles have no
    // registers for the second copy of the tile this takes (their main loop would
    // lose registers to it).
    constexpr bool kOwnInRegs = NV <= 16 && (NW == 4 || NV <= 8);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          store_partial(part, base + s * slice + ((i * TN + j) * 4 + v) * NT + tid, acc_vec(i, j, v));
    wait_stores_performed();
    __syncthreads();
    if (tid == 0) s_prev = arrive(&a.counters[tile_id]);
    __syncthreads();
    if (s_prev != (uint32_t)(S - 1)) return;
    // Sum the slices in slice order 0..S-1 from +0 (independent of which workgroup
    // is last, so the result is deterministic), each slice's values loaded together;
    // with kOwnInRegs slice s comes from registers.
    if constexpr (!kOwnInRegs) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          accf[i][j] = (f32x16){};
          acci[i][j] = (i32x16){};
        }
      for (int q = 0; q < S; ++q) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const f32x4 p = load_partial(part, base + q * slice + ((i * TN + j) * 4 + v) * NT + tid);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if constexpr (T::kIntAcc) acci[i][j][4 * v + e] += __builtin_bit_cast(i32x4, p)[e];
                else accf[i][j][4 * v + e] += p[e];
              }
            }
      }
    } else {
      f32x16 sumf[TM][TN];
      i32x16 sumi[TM][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          sumf[i][j] = (f32x16){};
          sumi[i][j] = (i32x16){};
        }
      for (int q = 0; q < S; ++q) {
        if (q == s) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              if constexpr (T::kIntAcc) sumi[i][j] += acci[i][j];
              else sumf[i][j] += accf[i][j];
            }
          continue;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const f32x4 p = load_partial(part, base + q * slice + ((i * TN + j) * 4 + v) * NT + tid);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if constexpr (T::kIntAcc) sumi[i][j][4 * v + e] += __builtin_bit_cast(i32x4, p)[e];
                else sumf[i][j][4 * v + e] += p[e];
              }
            }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          accf[i][j] = sumf[i][j];
          acci[i][j] = sumi[i][j];
        }
    }
    if (tid == 0) reset_counter(&a.counters[tile_id]);
  }

  // ---- epilogue.  The MFMAs take the weights as their first operand, so block
  // (i, j) holds the transposed product: lane l has output row l32 of block i and,
  // for value e, column 8 (e / 4) + 4 kg + (e % 4) of block j, i.e. four
  // consecutive columns per group of four values.  bf16 outputs go through LDS
  // (8-byte writes) so that global stores are whole 16-byte chunks of rows;
  // accumulator outputs and rows that are not 16-byte aligned are stored directly.
  const bool staged = !(SCH == kW8A8 && a.out_acc) && (a.N % 8 == 0);
  if (staged) {
    constexpr int PITCH = BN * 2 + 16;                       // bytes per staged row (padding spreads banks)
    static_assert(BM * PITCH <= kLdsBytes<QT, SCH, BM, BN, BKT, NSTAGE>(), "staging fits the LDS allocation");
    __syncthreads();                                         // every wave is done with the stage buffers
    // W8A8 scales for this lane's TN x 4 groups of four columns and TM rows: the
    // element scale is fp32(s_x * s_w[n]), s_x the static input scale or the
    // row's per-token scale.  All loads are issued before the first use
    // (N % 8 == 0 here, so n < N implies n + 3 < N).
    f32x4 sw[TN][4];
    float rf[TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        sw[j][g] = (f32x4){sw_t, sw_t, sw_t, sw_t};
        if (SCH == kW8A8 && !a.scale_per_tensor) {
          const int n = nt0 * 16 + (wn * TN + j) * 32 + 8 * g + 4 * kg;
          if (n < a.N) {
#pragma unroll
            for (int c = 0; c < 4; ++c) sw[j][g][c] = a.w_scale[n + c];
          }
        }
      }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + (wm * TM + i) * 32 + l32;
      rf[i] = a.input_scale;
      if (SCH == kW8A8 && a.row_scale) rf[i] = m < a.M ? a.row_scale[m] : 0.0f;
    }
    // bias of this lane's columns (bf16 -> fp32, exact); zero without a bias
    f32x4 bs[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bs[j][g] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        const int n = nt0 * 16 + (wn * TN + j) * 32 + 8 * g + 4 * kg;
        if (a.bias && n < a.N) {
#pragma unroll
          for (int c = 0; c < 4; ++c) bs[j][g][c] = bf16_bits_to_f32(a.bias[n + c]);
        }
      }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = (wn * TN + j) * 32 + 8 * g + 4 * kg;  // first of this lane's four columns
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          f32x4 v;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if constexpr (SCH == kW8A16) v[c] = accf[i][j][4 * g + c];
            else v[c] = (T::kIntAcc ? (float)acci[i][j][4 * g + c] : accf[i][j][4 * g + c]) * (rf[i] * sw[j][g][c]);
            if (a.bias) v[c] = add_bias_value(v[c], bs[j][g][c]);
          }
          const int row = (wm * TM + i) * 32 + l32;
          *reinterpret_cast<u32x2*>(smem + row * PITCH + col * 2) = pack_bf16x4(v);
        }
      }
    }
    __syncthreads();
    constexpr int CH = BN / 8;                               // 16-byte chunks per row
    const RcpDivAny dvn(a.next_scale_rcp ? a.next_scale : 1.0f);
#pragma unroll 4
    for (int c = tid; c < BM * CH; c += NT) {
      const int row = c / CH, ch = c % CH;
      const int m = m0 + row;
      const int n = nt0 * 16 + ch * 8;
      if (m < a.M && n < a.N) {
        u32x4 v = *reinterpret_cast<const u32x4*>(smem + row * PITCH + ch * 16);
        __bf16* dst = reinterpret_cast<__bf16*>(a.y) + (int64_t)m * a.N + n;
        if (n + 8 <= a.N) {
          st16(dst, v);
        } else {
          const __bf16* src = reinterpret_cast<const __bf16*>(&v);
          for (int e = 0; e < a.N - n; ++e) dst[e] = src[e];
        }
        if (SCH == kW8A8 && a.y_codes) {                     // next layer's codes of these 8 outputs
          const u32x2 q = a.next_scale_rcp ? (u32x2){quant4_rcp<QT>(v.x, v.y, dvn), quant4_rcp<QT>(v.z, v.w, dvn)}
                                           : (u32x2){quant4<QT>(v.x, v.y, a.next_scale), quant4<QT>(v.z, v.w, a.next_scale)};
          uint8_t* cdst = a.y_codes + (int64_t)m * a.N + n;
          if (n + 8 <= a.N) {
            *reinterpret_cast<u32x2*>(cdst) = q;
          } else {
            const uint8_t* src = reinterpret_cast<const uint8_t*>(&q);
            for (int e = 0; e < a.N - n; ++e) cdst[e] = src[e];
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + (wm * TM + i) * 32 + l32;
      if (m >= a.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int n = nt0 * 16 + (wn * TN + j) * 32 + 8 * (e >> 2) + 4 * kg + (e & 3);
          if (n >= a.N) continue;
          const int64_t o = (int64_t)m * a.N + n;
          if constexpr (SCH == kW8A16) {
            reinterpret_cast<__bf16*>(a.y)[o] = (__bf16)add_bias(accf[i][j][e], a.bias, n);
          } else if (a.out_acc) {
            if constexpr (T::kIntAcc) reinterpret_cast<int32_t*>(a.y)[o] = acci[i][j][e];
            else reinterpret_cast<float*>(a.y)[o] = accf[i][j][e];
          } else {
            const float sx = a.row_scale ? a.row_scale[m] : a.input_scale;
            const float comb = sx * (a.scale_per_tensor ? a.w_scale[0] : a.w_scale[n]);
            const float v = T::kIntAcc ? (float)acci[i][j][e] : accf[i][j][e];
            store_bf16_requant<QT>(a.y, a.y_codes, o, add_bias(v * comb, a.bias, n), a.next_scale, a.next_scale_rcp);
          }
        }
    }
  }
}

template <int QT, int SCH, int BM, int BN, int WM, int WN, int BKT, int NSTAGE>
hipError_t launch_t(const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  constexpr int LDS = kLdsBytes<QT, SCH, BM, BN, BKT, NSTAGE>();
  static_assert(LDS <= 160 * 1024, "LDS");
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  auto k = p.S > 1 ? gemm_mfma_kernel<QT, SCH, BM, BN, WM, WN, BKT, NSTAGE, true>
                   : gemm_mfma_kernel<QT, SCH, BM, BN, WM, WN, BKT, NSTAGE, false>;
  static std::atomic<uint64_t> lds_set[2];       // per instantiation, per device
  {
    const hipError_t e = set_lds_limit((const void*)k, LDS, lds_set[p.S > 1 ? 1 : 0]);
    if (e != hipSuccess) return e;
  }
  k<<<p.grid, (BM / WM) * (BN / WN) * 64, LDS, st>>>(a, p.S, p.units_per_split, tiles_m, tiles_n);
  return hipGetLastError();
}

// Tile configurations: workgroup tile BM x BN, per-wave WM x WN (four or eight waves),
// BKT 64-input tiles per LDS stage, NSTAGE stages.  One table feeds both the
// dispatch below and the planner's queries.
struct MfmaCfg {
  int BM, BN, WM, WN, BKT, NSTAGE;
  bool w8a16;   // instantiated for the weight-only scheme too (else W8A8 only)
};
constexpr MfmaCfg kMfmaCfgs[] = {
    {128, 256, 128, 64, 1, 4, true},     // 0
    {128, 128, 64, 64, 1, 4, true},      // 1
    {128, 256, 128, 64, 2, 2, true},     // 2
    {128, 128, 64, 64, 2, 3, true},      // 3
    {256, 256, 128, 64, 1, 3, true},     // 4: eight waves, two per SIMD
    {256, 256, 128, 64, 2, 2, false},    // 5: eight waves (bf16 x would need 192 KiB of LDS)
    {256, 192, 64, 96, 2, 2, false},     // 6: eight waves 64x96; 192 columns: 58 column tiles at N = 11008
    {128, 128, 128, 32, 1, 4, true},     // 7: four waves 128x32: each weight column dequantized once
    {128, 128, 64, 32, 2, 3, false},     // 8: eight waves 64x32: twice the waves issuing operand DMAs
};
constexpr int kNumMfmaCfgs = sizeof(kMfmaCfgs) / sizeof(kMfmaCfgs[0]);

template <int QT, int SCH, int C>
hipError_t launch_cfg(const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  constexpr MfmaCfg c = kMfmaCfgs[C];
  if constexpr (SCH == kW8A16 && !c.w8a16) {
    return hipErrorInvalidValue;
  } else {
    return launch_t<QT, SCH, c.BM, c.BN, c.WM, c.WN, c.BKT, c.NSTAGE>(p, a, st);
  }
}

template <int QT, int SCH, int... C>
hipError_t dispatch_cfg(int cfg, const GemmPlan& p, const GemmArgs& a, hipStream_t st,
                        std::integer_sequence<int, C...>) {
  hipError_t r = hipErrorInvalidValue;
  ((cfg == C ? (r = launch_cfg<QT, SCH, C>(p, a, st), 0) : 0), ...);
  return r;
}

}  // namespace

hipError_t launch_gemm_mfma(int scheme, int qtype, const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  const auto all = std::make_integer_sequence<int, kNumMfmaCfgs>{};
  if (scheme == kW8A16)
    return qtype == kFp8 ? dispatch_cfg<kFp8, kW8A16>(p.cfg, p, a, st, all)
                         : dispatch_cfg<kInt8, kW8A16>(p.cfg, p, a, st, all);
  return qtype == kFp8 ? dispatch_cfg<kFp8, kW8A8>(p.cfg, p, a, st, all)
                       : dispatch_cfg<kInt8, kW8A8>(p.cfg, p, a, st, all);
}

int mfma_cfg_tile_m(int cfg) { return cfg >= 0 && cfg < kNumMfmaCfgs ? kMfmaCfgs[cfg].BM : 0; }
int mfma_cfg_tile_n(int cfg) { return cfg >= 0 && cfg < kNumMfmaCfgs ? kMfmaCfgs[cfg].BN : 0; }
int mfma_cfg_bkt(int cfg) { return cfg >= 0 && cfg < kNumMfmaCfgs ? kMfmaCfgs[cfg].BKT : 1; }
int mfma_num_cfgs() { return kNumMfmaCfgs; }
bool mfma_cfg_valid(int scheme, int cfg) {
  return cfg >= 0 && cfg < kNumMfmaCfgs && (scheme != kW8A16 || kMfmaCfgs[cfg].w8a16);
}

}  // namespace qlq
