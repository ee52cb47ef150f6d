// C ABI of libqlq.so: argument validation, kernel-family choice and launch.
// Declarations and their contracts: include/qlq.h.
#include "qlq.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "qlq_launch.h"

namespace {

thread_local std::string g_last_error;

qlq_status fail(qlq_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
qlq_status fail(qlq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

qlq_status ok() {
  g_last_error.clear();
  return QLQ_OK;
}

qlq_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QLQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int64_t kMaxDim = int64_t(1) << 24;        // keeps every in-kernel index in range
constexpr int64_t kMaxOutputs = int64_t(1) << 40;   // keeps every launch grid below 2^31
constexpr int64_t kMaxInt8K = 133144;                // 127 * 127 * K < 2^31
// Split-K workspaces start with one fixed-size counter region shared by every
// plan, so partial sums of one call never land on counters of another.
constexpr int64_t kMaxSplitTiles = 1024;
constexpr size_t kCounterBytes = kMaxSplitTiles * 4;
constexpr int64_t kSmallUnitsPerWave = 8;   // matches kUnroll of the small-M kernel
// Batched decode: the small-M kernel takes up to this many rows (16-row groups, aligned
// path; above 64 rows narrow or small weights only) before the direct-to-LDS kernel's
// 128-row tiles (see plan_gemm).  Eight groups of at most 127 column tiles keep one split-K
// arrival counter per (group, column tile) inside the counter region.
constexpr int64_t kSmallMaxRows = 128;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// True when s = fp32(a / qmax) for a positive finite bf16 a and qmax 127 or 448 (how
// calibration and the per-token quantizer form scales) and s >= 2^-100: the scales for
// which the kernels' refined-reciprocal division (RcpDivAny) was checked to give the
// IEEE division's codes for every bf16 x.  Other scales keep the IEEE division.
bool calibrated_scale(float s) {
  if (!std::isfinite(s) || !(s >= 0x1p-100f)) return false;
  for (const float qmax : {127.0f, 448.0f}) {
    const float guess = s * qmax;
    uint32_t bits;
    std::memcpy(&bits, &guess, sizeof bits);
    const int64_t hi = bits >> 16;
    for (int d = -2; d <= 2; ++d) {
      const uint32_t cb = (uint32_t)(hi + d) << 16;
      float c;
      std::memcpy(&c, &cb, sizeof c);
      if (std::isfinite(c) && c > 0.0f && c / qmax == s) return true;
    }
  }
  return false;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

qlq_status check_dims(int64_t M, int64_t K, int64_t N) {
  if (M < 1 || K < 1 || N < 1) return fail(QLQ_ERR_INVALID_ARG, "sizes must be >= 1 (M=%lld K=%lld N=%lld)",
                                           (long long)M, (long long)K, (long long)N);
  if (M > kMaxDim || K > kMaxDim || N > kMaxDim)
    return fail(QLQ_ERR_INVALID_ARG, "sizes above 2^24 are not supported");
  return QLQ_OK;
}

qlq_status check_qtype(qlq_qtype q) {
  if (q != QLQ_INT8 && q != QLQ_FP8_E4M3FN) return fail(QLQ_ERR_UNSUPPORTED, "unknown qtype %d", (int)q);
  return QLQ_OK;
}

qlq_status check_scale(float s, const char* name) {
  if (!std::isfinite(s) || !(s > 0.0f)) return fail(QLQ_ERR_INVALID_ARG, "%s must be finite and > 0", name);
  return QLQ_OK;
}

}  // namespace

namespace qlq {

namespace {

// Direct-to-LDS MFMA kernel: choose the tile configuration and split-K factor
// that minimise the estimated time on 256 CUs:
//   rounds x (K stages per slice x t x load + e) + split-K (partial bytes x a + S x b),
// where a round is one wave of resident workgroups and load = (1 - w) + w x the
// fraction of CUs the grid keeps busy (a share w of the per-stage time is shared
// bandwidth that a partly filled chip gives to fewer CUs; w = 0.2 for W8A16, 0
// for W8A8).  t (per 64-input tile of K), e (per round: prologue, epilogue,
// launch), a, b and w were fitted to MI355X timings of every (configuration,
// split) at the 3B-scale stack's shapes, M = 256 and 1024, with cold weights; in
// total, the fit's picks are within 1 % (W8A16) and 2 % (W8A8) of the fastest
// measured plans.
GemmPlan plan_mfma(int scheme, int64_t M, int64_t K, int64_t N) {
  constexpr int64_t kCUs = 256;
  const int64_t KT = cdiv(K, 64);
  constexpr int kCfgs = 9;
  // {W8A16, W8A8} x cfg 0..8 (cfgs 5, 6 and 8 are W8A8 only; a zero t leaves a cfg out)
  const double t_us[2][kCfgs] = {{1.044, 0.7, 0.951, 0.716, 1.445, 0.0, 0.0, 0.617, 0.0},
                                 {0.639, 0.472, 0.571, 0.326, 0.919, 0.68, 0.601, 0.468, 0.324}};
  const double e_us[2][kCfgs] = {{6.105, 3.393, 6.54, 4.038, 13.98, 0.0, 0.0, 3.455, 0.0},
                                 {2.215, 2.381, 2.018, 1.341, 6.621, 7.423, 4.637, 2.392, 0.59}};
  const double a_us_per_mb[2] = {0.067, 0.143}, b_us[2] = {1.433, 1.459};
  // share of t that scales with the fraction of CUs the grid keeps busy
  const double load_weight[2] = {0.2, 0.0};
  const int per_cu[2][kCfgs] = {{1, 1, 1, 1, 1, 1, 1, 1, 1}, {1, 2, 1, 1, 1, 1, 1, 2, 1}};
  const int sch = scheme == kW8A16 ? 0 : 1;
  GemmPlan best;
  double best_cost = 1e300;
  for (int cfg = 0; cfg < kCfgs && cfg < mfma_num_cfgs(); ++cfg) {
    if (!mfma_cfg_valid(scheme, cfg) || !(t_us[sch][cfg] > 0.0)) continue;
    const int64_t BKT = mfma_cfg_bkt(cfg);
    if (KT % BKT != 0) continue;
    const int64_t KS = KT / BKT;                                // LDS stages over K
    const int64_t BM = mfma_cfg_tile_m(cfg), BN = mfma_cfg_tile_n(cfg);
    const int64_t tiles = cdiv(M, BM) * cdiv(N, BN);
    for (int64_t S = 1; S <= 8; ++S) {
      if (S > 1 && (tiles > kMaxSplitTiles || KS / S < 2)) break;
      const int64_t ups = cdiv(KS, S);
      if (cdiv(KS, ups) != S) continue;
      const int64_t slots = kCUs * per_cu[sch][cfg];
      const int64_t rounds = cdiv(tiles * S, slots);
      const double busy = std::min(1.0, (double)(tiles * S) / (double)slots);
      const double load = (1.0 - load_weight[sch]) + load_weight[sch] * busy;
      double cost = (double)rounds * ((double)(ups * BKT) * t_us[sch][cfg] * load + e_us[sch][cfg]);
      if (S > 1) cost += (double)(S * tiles * BM * BN * 8) * 1e-6 * a_us_per_mb[sch] + b_us[sch] * (double)S;
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best = GemmPlan();
        best.kind = 2;
        best.cfg = cfg;
        best.BM = (int)BM;
        best.BN = (int)BN;
        best.S = (int)S;
        best.units_per_split = (int)ups;
        best.tiles = (int)tiles;
        best.grid = (int)(tiles * S);
        if (S > 1) {   // one fp32/int32 partial per output element and slice
          best.ws_counter_bytes = kCounterBytes;
          best.ws_bytes = kCounterBytes + (size_t)S * tiles * BM * BN * 4;
        }
      }
    }
  }
  return best;
}

}  // namespace

GemmPlan plan_gemm(int scheme, int qtype, int64_t M, int64_t K, int64_t N, bool fast) {
  const bool aligned_path = fast && K % 64 == 0;
  // Batched decode (16 < M <= 64, aligned path): the small-M kernel with one workgroup
  // per 16-row group (each group re-reads the weights, from L2 when its siblings run
  // beside it) against the direct-to-LDS kernel, whose 128-row tiles stream 128 rows
  // of x whatever M is.  Same-box timings (INT8 W8A16 and FP8 W8A8 over 17 shapes from
  // 1024 to 28672 inputs and outputs; INT8 W8A8 on the stack's): narrow outputs (fewer
  // than 128 column tiles) ran faster with the groups at every M (14336 -> 1024 at M =
  // 24: 25.0 -> 12.4 us); with two groups wider outputs did too (0.36-0.85 of the time)
  // except over K >= 12288 (14336 -> 4096: 1.11, 13824 -> 5120: 1.23-1.28); with three
  // groups weights up to about 17M codes gained (0.78-0.95; 22.5M mixed, 0.85-1.17;
  // larger slower; up to 26M over K <= 8192: W8A16 0.78-0.89, W8A8 on at most 512 column
  // tiles 0.86-0.88 (3072 -> 8192 and 5120 x 5120), on 688 1.0-1.14) and with four only up to
  // about 12M (2048 -> 5632: 0.79-0.82; 16.8M 0.91-1.10; larger up to 1.8; W8A16 over
  // K = 2048 up to 22.5M: 0.79-0.91).  From 65 to 128 rows narrow outputs over K <= 4096
  // gained (0.44-0.72; K = 8192 0.93-1.02, deeper up to 1.9), and of wider ones only
  // weights of at most 4M codes on at most 128 column tiles (2048 x 2048: 0.69-0.83;
  // 1024 -> 4096 0.74-1.30, 2048 -> 4096 0.96-1.35, larger up to 1.9).
  bool small = M <= 16;
  if (!small && aligned_path && M <= kSmallMaxRows) {
    const int64_t groups = cdiv(M, 16), NT = cdiv(N, 16);
    if (groups > 4) small = (NT < 128 && K <= 4096) || (NT <= 128 && N * K <= (int64_t(4) << 20));
    else if (NT < 128) small = true;
    else if (groups <= 2) small = K < 12288;
    else if (groups == 3)
      small = N * K <= (int64_t(20) << 20) ||
              (K <= 8192 && N * K <= (int64_t(28) << 20) && (scheme == kW8A16 || NT <= 512)) ||
              (K >= 8192 && NT == 128);   // four groups per workgroup, see below
    else small = N * K <= (int64_t(12) << 20) || (scheme == kW8A16 && K <= 2048 && N * K <= (int64_t(24) << 20));
  }
  if (!small && aligned_path) return plan_mfma(scheme, M, K, N);
  GemmPlan p;
  const int64_t KT = cdiv(K, 64), NT = cdiv(N, 16);
  if (small) {
    // Small-M: one workgroup per 16 output columns, with 4, 8 or 16 waves
    // splitting K inside it (summed through LDS).  Measured on MI355X over
    // decode shapes with N from 2048 to 14336 and K from 2048 to 14336: K splits
    // across workgroups cost more than they gain (the partial-sum handoff is a
    // few memory round trips) except for narrow, deep weights, and each wave
    // should issue all its loads at once (at most kSmallUnitsPerWave units),
    // with more waves only while the grid is small (about 512 waves; 256 for
    // FP8 W8A8, whose units are twice as long).  FP8 W8A8 with one column tile
    // stops at 8 waves (that 16-wave build would spill registers).
    //
    // A second sweep (N 2048 to 28672, K 2048 to 8192, M 1 / 8 / 16 and, for FP8
    // W8A8, M 6 to 16; every choice of CT column tiles per workgroup and waves)
    // refined this for wide weights:
    //  * without K slices, more than about 12 waves per CU (W8A16; 24 for W8A8)
    //    only add scheduling pressure, so W is halved down to that;
    //  * a unit's x loads serve CT column tiles, which pays once x is a sizeable
    //    share of the unit's loads: two tiles from 320 column tiles on (W8A16 from
    //    M = 6, W8A8 from M = 12), four from 640 (W8A16 from M = 8, FP8 W8A8 from
    //    M = 12; INT8 W8A8 never gained from four).  Their waves are chosen for
    //    about 14 per CU (W8A8 with two tiles: at most 8 waves).
    // Over that sweep the rule is within 3.3 % of the best plan per shape (in
    // total; single measurements vary by about 2 %) and 20 % (W8A16) / 6 % (INT8
    // W8A8) / 4 % (FP8 W8A8) faster than the first rule alone.
    p.kind = 0;
    // Above 16 rows every 16-row group is a workgroup of its own: the rules below see
    // a group's rows (Mg) and count workgroups and waves over all NRG groups (NRW
    // workgroups per column tile and slice).  Three groups over K >= 8192 on exactly
    // 128 column tiles take one workgroup of four groups instead (each unit's weights
    // loaded once for all of them; the fourth group lies past M): two K slices then make
    // one workgroup per CU.  Same-box timings against the plans before (three single
    // groups up to 20M weight codes, the direct-to-LDS kernel above) at M = 33 / 40 / 48
    // over K = 8192 to 16384 to 2048 outputs: INT8 W8A16 0.73-1.05 of the time (11008 ->
    // 2048 at M = 33: 24.4 -> 18.7 us), FP8 W8A8 0.74-0.92, INT8 W8A8 0.79-0.98.  With
    // 138 to 188 column tiles the 276 to 376 workgroups take a second round on part of
    // the CUs (1.01-1.79x), and wider outputs, shallower weights and M = 64 lost too.
    // Narrow outputs of 64 column tiles (1024 outputs) over K >= 14336 take the same
    // workgroup of four groups (K slices up to 256 workgroups) in place of a pair and a
    // single: 14336 / 16384 -> 1024 INT8 W8A16 0.82-0.94, INT8 W8A8 0.82-0.94, FP8 W8A8
    // 0.94-1.07 (so FP8 W8A8 only from K = 28672), 28672 -> 1024 0.75-0.89 in all three.
    // 32 and 96 column tiles, and 64 over K = 8192, lost (up to 1.3x), except in W8A8:
    // on 80 to 127 column tiles FP8 W8A8 took 0.62-0.99 of the time over K = 8192 to 14336
    // up to 24M weight codes (14336 -> 1920: 0.95-1.13), INT8 W8A8 0.83-0.98 over K = 8192
    // (deeper, at M = 40 / 48: up to 1.19x).
    const int64_t Mg = std::min<int64_t>(M, 16), NRG = cdiv(M, 16);
    const int64_t TPU = (scheme == kW8A8 && qtype == 1) ? 2 : 1;
    const bool quad = NRG == 3 && fast &&
                      ((K >= 8192 && NT == 128) || (NT == 64 && K >= 14336 && (TPU == 1 || K >= 28672)) ||
                       (scheme == kW8A8 && NT >= 80 && NT < 128 && K >= 8192 &&
                        (TPU == 2 ? N * K <= (int64_t(24) << 20) : K < 10240)));
    const int64_t NRW = quad ? 1 : NRG;
    const int64_t KU = cdiv(KT, TPU);
    const int64_t max_waves = TPU == 2 ? 8 : 16;
    // A third sweep (N 1024 to 8192 with K 4096 to 28672, M 1 / 4 / 8 / 16, every
    // forced choice of K slices and waves) set the slices of narrow outputs (fewer
    // than 128 column tiles): about 64 one-tile units per slice (48 of FP8 W8A8's
    // two-tile units; 32 for W8A16 above M = 8, whose bf16 x then outweighs the
    // codes), at most 256 workgroups, with the waves that one load batch needs and
    // no more (N = 1024: K = 4096 unsplit at M <= 8, 6-18 % faster than two slices;
    // K = 14336 and 28672 in three or four slices, 9-34 % faster).  That sweep ran
    // on the aligned path; on the generic one (K % 64 != 0 or x not 16-byte aligned:
    // per-element bounds checks) the longer slices were 35-50 % slower (5000 -> 300
    // at M = 8 / 16), so it keeps the first rule's slices.
    int64_t S = 1;
    const bool narrow = NT < 128 && fast;
    const int64_t narrow_units = TPU == 2 ? 48 : (scheme == kW8A16 && Mg > 8 ? 32 : 64);
    if (narrow) S = std::max<int64_t>(1, std::min(cdiv(256, NT * NRW), cdiv(KU, narrow_units)));
    else if (NT < 128) S = std::min(cdiv(128, NT), std::max<int64_t>(1, KU / kSmallUnitsPerWave));
    else if (NT < 192 && KU >= 64) S = 2;
    int64_t ups = cdiv(KU, S);
    S = cdiv(KU, ups);
    int64_t W = 4;
    while (W < max_waves && cdiv(ups, W) > kSmallUnitsPerWave) W *= 2;
    if (!narrow)
      while (W < max_waves && NT * NRW * S * W <= (TPU == 2 ? 256 : 512)) W *= 2;
    int64_t ct = 1;
    if (S == 1) {
      const int64_t cap = scheme == kW8A16 ? 12 : 24;           // waves per CU
      while (W > 4 && NT * NRW * W > cap * 256) W /= 2;
      const int64_t m2 = scheme == kW8A16 ? 6 : 12;                      // rows for two tiles
      const int64_t m4 = scheme == kW8A16 ? 8 : (TPU == 2 ? 12 : Mg + 1);  // rows for four
      // With 4096 <= K < 8192, two tiles at any M (each unit's x loads then serve
      // both) unless that spreads the workgroups worse over the 256 CUs: every
      // workgroup has the same work, so the busiest CU (ceil(g / 256) of g
      // workgroups) against the mean (g / 256) sets the time.  Measured below the M
      // thresholds above: 2-12 % faster on 5504, 6144, 8192, 14336 and 16384 outputs
      // (equal spread), slower on 11008 and 28672 (one tile spreads better); at K =
      // 2048 (mixed, up to 6 % either way) and 8192 (slower) one tile stays.
      auto spread = [](int64_t g) {
        const double r = (double)g / 256.0;
        return std::ceil(r) / r;
      };
      const bool k_mid = K >= 4096 && K < 8192 && spread(cdiv(NT, 2) * NRW) <= spread(NT * NRW) + 1e-9;
      if (!quad && fast && Mg >= m4 && NT >= 640) ct = 4;
      else if (!quad && fast && (Mg >= m2 || k_mid) && NT >= 320) ct = 2;
      if (ct > 1) {
        const int64_t groups = cdiv(NT, ct);
        const int64_t w_max = (ct == 2 && scheme == kW8A8) ? 8 : 16;
        double best = 1e300;
        for (int64_t w = 4; w <= w_max; w *= 2) {
          if (w > 4 && w > KU) break;
          const double d = std::fabs((double)(groups * NRW * w) / 256.0 - 14.0);
          if (d < best - 1e-9) {
            best = d;
            W = w;
          }
        }
      }
      // One column tile per workgroup over deep weights (at least 128 one-tile or
      // 96 two-tile units), when 257 to 1024 tiles leave the busiest CU more than 1.2
      // times the mean: K slices (2 to 4, the best spread, fewest on ties) with four waves.
      // The third sweep: 320 and 384 column tiles over K = 8192 to 14336 at M <= 8,
      // 5-15 % faster (13824 -> 5120, 14336 -> 6144); shallower weights on the same
      // tile counts gained nothing.
      if (ct == 1 && NRW == 1 && NT > 256 && NT <= kMaxSplitTiles && KU >= (TPU == 2 ? 96 : 128) && spread(NT) > 1.2 + 1e-9) {
        int64_t s_best = 2;
        for (int64_t s = 3; s <= 4; ++s)
          if (spread(NT * s) < spread(NT * s_best) - 1e-9) s_best = s;
        ups = cdiv(KU, s_best);
        S = cdiv(KU, ups);
        W = 4;
      }
      // FP8 W8A8 without slices over K >= 8192 (64 two-tile units) on 256 or more
      // column tiles: four waves, each looping over several load batches, were 1-7 %
      // faster than eight in the third sweep.
      if (ct == 1 && S == 1 && TPU == 2 && NT >= 256 && KU >= 64) W = 4;
    }
    // Two row groups per workgroup (each unit's weights loaded once for both) with one
    // column tile, where the halved grid still fills the chip.  Same-box timings against
    // one group per workgroup, all three schemes: two groups over K >= 8192 on at least
    // 128 column tiles (8192 and 11008 inputs to 2048 and 4096 outputs) 0.61-0.83 /
    // 0.69-0.92 / 0.78-0.99 of the time at M = 17 / 24 / 32 (11008 -> 4096 INT8 W8A16 at
    // M = 17: 26.7 -> 16.7 us), on 192 or more column tiles at any depth 0.66-0.98
    // (6144 -> 4096 INT8 W8A16 at M = 17: 0.66); three groups on narrow outputs over
    // K >= 8192 0.78-1.00 at M = 40 / 48 (M = 33, one row in the third group: 0.81-1.05).
    // Elsewhere the halved grid lost (2048 x 2048 at M = 24: 1.12-1.19x; 14336 -> 1024
    // with two groups: 1.06-1.43x; wide outputs with three groups: 1.03-1.21x).
    int64_t rw = 1;
    if (quad && TPU == 2 && W == 16) W = 8;            // no 16-wave FP8 W8A8 build of several groups
    if (ct == 1 && fast && !(TPU == 2 && W == 16)) {   // no 16-wave FP8 W8A8 pair build
      if (quad) rw = 4;
      else if (NRG == 2 && (NT >= 192 || (K >= 8192 && NT >= 128))) rw = 2;
      else if (NRG == 3 && NT < 128 && K >= 8192) rw = 2;
    }
    // One arrival counter per (row group, column tile): NRG <= 4 keeps every split plan
    // above (fewer than 192 column tiles, or one row group) within the counter region.
    if (S > 1 && NT * NRG > kMaxSplitTiles) {
      S = 1;
      ups = KU;
    }
    p.S = (int)S;
    p.ct = (int)ct;
    p.rw = (int)rw;
    p.units_per_split = (int)ups;
    p.units_per_wave = (int)cdiv(ups, W);
    p.waves = (int)W;
    p.tiles = (int)NT;
    p.grid = (int)(cdiv(NT, ct) * S * cdiv(NRG, rw));
    if (S > 1) {   // S > 1 only when NT < 192 or 256 < NT <= kMaxSplitTiles
      p.ws_counter_bytes = kCounterBytes;
      p.ws_bytes = p.ws_counter_bytes + (size_t)S * NRG * NT * 64 * 16;
    }
  } else {
    p.kind = 1;
    p.BM = 128;
    p.BN = 128;
    const int64_t tiles = cdiv(M, p.BM) * cdiv(N, p.BN);
    const int64_t BKT = scheme == kW8A16 ? 1 : 2;
    const int64_t KU = cdiv(KT, BKT);
    int64_t S = 1;
    if (tiles < 240) {   // 240 <= kMaxSplitTiles
      S = cdiv(256, tiles);
      int64_t cap = KU / 4 > 1 ? KU / 4 : 1;
      if (S > cap) S = cap;
    }
    const int64_t ups = cdiv(KU, S);
    S = cdiv(KU, ups);
    p.S = (int)S;
    p.units_per_split = (int)ups;
    p.tiles = (int)tiles;
    p.grid = (int)(tiles * S);
    if (S > 1) {
      const int64_t nv = (p.BM / 32) * (p.BN / 32);   // f32x4 values per thread
      p.ws_counter_bytes = kCounterBytes;
      p.ws_bytes = p.ws_counter_bytes + (size_t)S * tiles * nv * 256 * 16;
    }
  }
  return p;
}

}  // namespace qlq

extern "C" {

const char* qlq_status_string(qlq_status s) {
  switch (s) {
    case QLQ_OK: return "QLQ_OK";
    case QLQ_ERR_INVALID_ARG: return "QLQ_ERR_INVALID_ARG";
    case QLQ_ERR_UNSUPPORTED: return "QLQ_ERR_UNSUPPORTED";
    case QLQ_ERR_HIP: return "QLQ_ERR_HIP";
  }
  return "QLQ_UNKNOWN_STATUS";
}

const char* qlq_last_error(void) { return g_last_error.c_str(); }

const char* qlq_version(void) { return "qlq 0.1.0 gfx950"; }

size_t qlq_packed_weight_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1) return 0;
  return (size_t)cdiv(N, 16) * 16 * (size_t)cdiv(K, 64) * 64;
}

// Workspace of the GEMM proper (split-K counters and partials).  The call picks
// the direct-to-LDS kernel only for aligned x, so this covers both plans.
static size_t gemm_ws_bytes(int scheme, int64_t M, int64_t K, int64_t N, int qtype) {
  const size_t a = qlq::plan_gemm(scheme, qtype, M, K, N, true).ws_bytes;
  const size_t b = qlq::plan_gemm(scheme, qtype, M, K, N, false).ws_bytes;
  return a > b ? a : b;
}

// Fused static W8A8: offset of the activation codes inside the workspace.  They go after the GEMM's region and never below the counter
// region, so the counters (which every call leaves at zero) are never
// overwritten by codes, whatever M earlier calls on the same buffer used.
static size_t fused_xq_offset(int64_t M, int64_t K, int64_t N, int qtype) {
  const size_t g = (gemm_ws_bytes(qlq::kW8A8, M, K, N, qtype) + 255) / 256 * 256;
  return g > kCounterBytes ? g : kCounterBytes;
}

size_t qlq_workspace_bytes(qlq_scheme scheme, int64_t M, int64_t K, int64_t N, qlq_qtype qtype) {
  if (M < 1 || K < 1 || N < 1 || M > kMaxDim || K > kMaxDim || N > kMaxDim) return 0;
  switch (scheme) {
    case QLQ_SCHEME_W8A16: return gemm_ws_bytes(qlq::kW8A16, M, K, N, (int)qtype);
    case QLQ_SCHEME_W8A8_STATIC:
    case QLQ_SCHEME_W8A8_DYNAMIC: return gemm_ws_bytes(qlq::kW8A8, M, K, N, (int)qtype);
    case QLQ_SCHEME_W8A8_STATIC_FUSED: return fused_xq_offset(M, K, N, (int)qtype) + (size_t)M * (size_t)K;
  }
  return 0;
}

qlq_status qlq_quantize_weight(const void* w, int w_is_bf16, int64_t N, int64_t K, qlq_qtype qtype,
                               qlq_granularity granularity, void* wq_packed, float* w_scale,
                               hipStream_t stream) {
  if (!w || !wq_packed || !w_scale) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_dims(1, K, N)) return st;
  if (qlq_status st = check_qtype(qtype)) return st;
  if (granularity != QLQ_PER_CHANNEL && granularity != QLQ_PER_TENSOR)
    return fail(QLQ_ERR_UNSUPPORTED, "unknown granularity %d", (int)granularity);
  if (!aligned(wq_packed, 16)) return fail(QLQ_ERR_INVALID_ARG, "wq_packed must be 16-byte aligned");
  if (!aligned(w, w_is_bf16 ? 2 : 4) || !aligned(w_scale, 4)) return fail(QLQ_ERR_INVALID_ARG, "misaligned pointer");
  return hip_status(qlq::launch_pack_weight(w, w_is_bf16 ? 1 : 0, (int)N, (int)K, (int)qtype,
                                            granularity == QLQ_PER_TENSOR, static_cast<uint8_t*>(wq_packed),
                                            w_scale, stream),
                    "quantize_weight");
}

qlq_status qlq_unpack_weight(const void* wq_packed, int64_t N, int64_t K, void* wq_rowmajor, hipStream_t stream) {
  if (!wq_packed || !wq_rowmajor) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_dims(1, K, N)) return st;
  return hip_status(qlq::launch_unpack_weight(static_cast<const uint8_t*>(wq_packed), (int)N, (int)K,
                                              static_cast<uint8_t*>(wq_rowmajor), stream),
                    "unpack_weight");
}

qlq_status qlq_calibrate_input_scale(const void* x_calib_bf16, int64_t numel, qlq_qtype qtype,
                                     float* input_scale_out, hipStream_t stream) {
  if (!x_calib_bf16 || !input_scale_out) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (numel < 1) return fail(QLQ_ERR_INVALID_ARG, "numel must be >= 1");
  if (qlq_status st = check_qtype(qtype)) return st;
  if (!aligned(x_calib_bf16, 2) || !aligned(input_scale_out, 4)) return fail(QLQ_ERR_INVALID_ARG, "misaligned pointer");
  return hip_status(qlq::launch_absmax_scale(x_calib_bf16, 1, numel, qtype == QLQ_FP8_E4M3FN ? 448.0f : 127.0f,
                                             input_scale_out, stream),
                    "calibrate_input_scale");
}

qlq_status qlq_quantize_act_static(const void* x_bf16, int64_t M, int64_t K, float input_scale, qlq_qtype qtype,
                                   void* xq, hipStream_t stream) {
  if (!x_bf16 || !xq) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_dims(M, K, 1)) return st;
  if (qlq_status st = check_qtype(qtype)) return st;
  if (qlq_status st = check_scale(input_scale, "input_scale")) return st;
  if (!aligned(x_bf16, 2)) return fail(QLQ_ERR_INVALID_ARG, "misaligned pointer");
  return hip_status(qlq::launch_quant_act(x_bf16, M * K, input_scale, (int)qtype, xq, stream,
                                          calibrated_scale(input_scale)),
                    "quantize_act_static");
}

qlq_status qlq_quantize_act_dynamic(const void* x_bf16, int64_t M, int64_t K, qlq_qtype qtype, void* xq,
                                    float* x_scale, hipStream_t stream) {
  if (!x_bf16 || !xq || !x_scale) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_dims(M, K, 1)) return st;
  if (qlq_status st = check_qtype(qtype)) return st;
  if (!aligned(x_bf16, 2) || !aligned(x_scale, 4)) return fail(QLQ_ERR_INVALID_ARG, "misaligned pointer");
  return hip_status(qlq::launch_quant_act_dynamic(x_bf16, (int)M, (int)K, (int)qtype, xq, x_scale, stream),
                    "quantize_act_dynamic");
}

// A GEMM call after validation: its plan and kernel arguments.  Preparing runs
// every check and has no side effect; launching enqueues the kernels.  Calls that
// enqueue more than one kernel prepare everything before the first launch, so a
// rejected call leaves the stream (or a graph being captured) untouched.
struct PreparedGemm {
  int scheme = 0;
  int qtype = 0;
  qlq::GemmPlan plan;
  qlq::GemmArgs args{};
  const char* what = "";
};

// Points a prepared call's split-K counters and partials into `workspace` (checks
// its size and alignment; nothing when the plan needs no workspace).
static qlq_status bind_workspace(PreparedGemm& g, void* workspace, size_t workspace_bytes) {
  const qlq::GemmPlan& plan = g.plan;
  qlq::GemmArgs& a = g.args;
  a.counters = nullptr;
  a.partials = nullptr;
  a.partials_bytes = 0u;
  if (plan.ws_bytes == 0) return QLQ_OK;
  if (!workspace || workspace_bytes < plan.ws_bytes)
    return fail(QLQ_ERR_INVALID_ARG, "workspace too small: need %zu bytes, got %zu", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(QLQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  a.counters = static_cast<uint32_t*>(workspace);
  a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + plan.ws_counter_bytes);
  a.partials_bytes = (uint32_t)(plan.ws_bytes - plan.ws_counter_bytes);
  return QLQ_OK;
}

// Passed as prepare_gemm's workspace to leave the binding to a later bind_workspace.
static void* const kWorkspaceLater = reinterpret_cast<void*>(~uintptr_t{0});

// x: bf16 for W8A16, codes for W8A8.
static qlq_status prepare_gemm(PreparedGemm& g, int scheme, const void* x, int64_t M, int64_t K, int64_t N,
                               const void* wq_packed, const float* w_scale, int64_t w_scale_numel, qlq_qtype qtype,
                               float input_scale, const float* row_scale, int out_acc, void* y, void* workspace,
                               size_t workspace_bytes, const char* what, const void* bias = nullptr,
                               void* y_codes = nullptr, float next_scale = 1.0f) {
  if (!x || !wq_packed || !w_scale || !y) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_dims(M, K, N)) return st;
  if (M * N > kMaxOutputs) return fail(QLQ_ERR_UNSUPPORTED, "M * N above 2^40 outputs is not supported");
  if (qlq_status st = check_qtype(qtype)) return st;
  if (w_scale_numel != 1 && w_scale_numel != N)
    return fail(QLQ_ERR_INVALID_ARG, "w_scale_numel must be 1 or N (got %lld, N=%lld)", (long long)w_scale_numel,
                (long long)N);
  if (!aligned(wq_packed, 16)) return fail(QLQ_ERR_INVALID_ARG, "wq_packed must be 16-byte aligned");
  if (!aligned(w_scale, 4) || !aligned(y, 4) || !aligned(x, scheme == qlq::kW8A16 ? 2 : 1) ||
      !aligned(row_scale, 4) || !aligned(bias, 2))
    return fail(QLQ_ERR_INVALID_ARG, "misaligned pointer");
  const bool fast = (K % 64 == 0) && aligned(x, 16);
  qlq::GemmPlan plan = qlq::plan_gemm(scheme, (int)qtype, M, K, N, fast);
  if (plan.ws_bytes > 0 && plan.ws_bytes - plan.ws_counter_bytes >= ((size_t)1 << 31))
    return fail(QLQ_ERR_UNSUPPORTED, "split-K partials above 2 GiB");
  qlq::GemmArgs& a = g.args;
  a = qlq::GemmArgs{};
  a.x = x;
  a.w = static_cast<const uint8_t*>(wq_packed);
  a.w_scale = w_scale;
  a.scale_per_tensor = w_scale_numel == 1 ? 1 : 0;
  a.y = y;
  a.M = (int)M;
  a.K = (int)K;
  a.N = (int)N;
  a.KT = (int)cdiv(K, 64);
  a.NT = (int)cdiv(N, 16);
  a.input_scale = input_scale;
  a.row_scale = row_scale;
  a.bias = static_cast<const uint16_t*>(bias);
  a.y_codes = static_cast<uint8_t*>(y_codes);
  a.next_scale = next_scale;
  a.next_scale_rcp = (y_codes && calibrated_scale(next_scale)) ? 1 : 0;
  a.out_acc = out_acc;
  a.fast = fast;
  g.scheme = scheme;
  g.qtype = (int)qtype;
  g.plan = plan;
  g.what = what;
  if (workspace == kWorkspaceLater) return QLQ_OK;
  return bind_workspace(g, workspace, workspace_bytes);
}

static qlq_status launch_gemm(const PreparedGemm& g, hipStream_t stream) {
  hipError_t e = g.plan.kind == 0   ? qlq::launch_gemm_small(g.scheme, g.qtype, g.plan, g.args, stream)
                 : g.plan.kind == 1 ? qlq::launch_gemm_large(g.scheme, g.qtype, g.plan, g.args, stream)
                                    : qlq::launch_gemm_mfma(g.scheme, g.qtype, g.plan, g.args, stream);
  return hip_status(e, g.what);
}

static qlq_status run_gemm(int scheme, const void* x, int64_t M, int64_t K, int64_t N, const void* wq_packed,
                           const float* w_scale, int64_t w_scale_numel, qlq_qtype qtype, float input_scale,
                           const float* row_scale, int out_acc, void* y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream, const char* what,
                           const void* bias = nullptr, void* y_codes = nullptr, float next_scale = 1.0f) {
  PreparedGemm g;
  if (qlq_status st = prepare_gemm(g, scheme, x, M, K, N, wq_packed, w_scale, w_scale_numel, qtype, input_scale,
                                   row_scale, out_acc, y, workspace, workspace_bytes, what, bias, y_codes,
                                   next_scale))
    return st;
  return launch_gemm(g, stream);
}

qlq_status qlq_qlinear_w8a16(const void* x_bf16, int64_t M, int64_t K, int64_t N, const void* wq_packed,
                             const float* w_scale, int64_t w_scale_numel, qlq_qtype qtype, void* y_bf16,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_gemm(qlq::kW8A16, x_bf16, M, K, N, wq_packed, w_scale, w_scale_numel, qtype, 1.0f, nullptr, 0,
                  y_bf16, workspace, workspace_bytes, stream, "qlinear_w8a16");
}

qlq_status qlq_qlinear_w8a8_static(const void* xq, float input_scale, int64_t M, int64_t K, int64_t N,
                                   const void* wq_packed, const float* w_scale, int64_t w_scale_numel,
                                   qlq_qtype qtype, qlq_out out, void* y, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  if (qlq_status st = check_scale(input_scale, "input_scale")) return st;
  if (out != QLQ_OUT_BF16 && out != QLQ_OUT_ACC) return fail(QLQ_ERR_UNSUPPORTED, "unknown out mode %d", (int)out);
  if (qtype == QLQ_INT8 && K > kMaxInt8K)
    return fail(QLQ_ERR_INVALID_ARG, "INT8 W8A8 needs K <= %lld for an exact int32 accumulator",
                (long long)kMaxInt8K);
  return run_gemm(qlq::kW8A8, xq, M, K, N, wq_packed, w_scale, w_scale_numel, qtype, input_scale, nullptr,
                  out == QLQ_OUT_ACC ? 1 : 0, y, workspace, workspace_bytes, stream, "qlinear_w8a8_static");
}

qlq_status qlq_qlinear_w8a8_static_requant(const void* xq, float input_scale, int64_t M, int64_t K, int64_t N,
                                           const void* wq_packed, const float* w_scale, int64_t w_scale_numel,
                                           qlq_qtype qtype, float next_scale, void* y, void* y_codes,
                                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (qlq_status st = check_scale(input_scale, "input_scale")) return st;
  if (qlq_status st = check_scale(next_scale, "next_scale")) return st;
  if (!y_codes) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(y_codes, 16)) return fail(QLQ_ERR_INVALID_ARG, "y_codes must be 16-byte aligned");
  if (qtype == QLQ_INT8 && K > kMaxInt8K)
    return fail(QLQ_ERR_INVALID_ARG, "INT8 W8A8 needs K <= %lld for an exact int32 accumulator",
                (long long)kMaxInt8K);
  return run_gemm(qlq::kW8A8, xq, M, K, N, wq_packed, w_scale, w_scale_numel, qtype, input_scale, nullptr, 0, y,
                  workspace, workspace_bytes, stream, "qlinear_w8a8_static_requant", nullptr, y_codes, next_scale);
}

static qlq_status check_w8a8(qlq_qtype qtype, qlq_out out, int64_t K) {
  if (out != QLQ_OUT_BF16 && out != QLQ_OUT_ACC) return fail(QLQ_ERR_UNSUPPORTED, "unknown out mode %d", (int)out);
  if (qtype == QLQ_INT8 && K > kMaxInt8K)
    return fail(QLQ_ERR_INVALID_ARG, "INT8 W8A8 needs K <= %lld for an exact int32 accumulator",
                (long long)kMaxInt8K);
  return QLQ_OK;
}

qlq_status qlq_qlinear_w8a8_static_fused(const void* x_bf16, float input_scale, int64_t M, int64_t K, int64_t N,
                                         const void* wq_packed, const float* w_scale, int64_t w_scale_numel,
                                         qlq_qtype qtype, qlq_out out, void* y, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  if (qlq_status st = check_scale(input_scale, "input_scale")) return st;
  if (qlq_status st = check_qtype(qtype)) return st;
  if (qlq_status st = check_w8a8(qtype, out, K)) return st;
  // one quantization pass into the workspace, then the GEMM on the codes
  if (!x_bf16 || !wq_packed || !w_scale || !y) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_dims(M, K, N)) return st;
  if (!aligned(x_bf16, 2)) return fail(QLQ_ERR_INVALID_ARG, "misaligned pointer");
  const size_t off = fused_xq_offset(M, K, N, (int)qtype);
  const size_t need = off + (size_t)M * (size_t)K;
  if (!workspace || workspace_bytes < need)
    return fail(QLQ_ERR_INVALID_ARG, "workspace too small: need %zu bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(QLQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  void* xq = static_cast<uint8_t*>(workspace) + off;
  PreparedGemm g;
  if (qlq_status st = prepare_gemm(g, qlq::kW8A8, xq, M, K, N, wq_packed, w_scale, w_scale_numel, qtype,
                                   input_scale, nullptr, out == QLQ_OUT_ACC ? 1 : 0, y, workspace, off,
                                   "qlinear_w8a8_static_fused"))
    return st;
  if (qlq_status st = hip_status(qlq::launch_quant_act(x_bf16, M * K, input_scale, (int)qtype, xq, stream,
                                                       calibrated_scale(input_scale)),
                                 "qlinear_w8a8_static_fused"))
    return st;
  return launch_gemm(g, stream);
}

qlq_status qlq_qlinear_w8a8_dynamic(const void* xq, const float* x_scale, int64_t M, int64_t K, int64_t N,
                                    const void* wq_packed, const float* w_scale, int64_t w_scale_numel,
                                    qlq_qtype qtype, qlq_out out, void* y, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  if (!x_scale) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_qtype(qtype)) return st;
  if (qlq_status st = check_w8a8(qtype, out, K)) return st;
  return run_gemm(qlq::kW8A8, xq, M, K, N, wq_packed, w_scale, w_scale_numel, qtype, 1.0f, x_scale,
                  out == QLQ_OUT_ACC ? 1 : 0, y, workspace, workspace_bytes, stream, "qlinear_w8a8_dynamic");
}

static qlq_status check_kv_dims(int64_t T, int64_t H, int64_t D) {
  if (T < 1 || H < 1 || D < 1) return fail(QLQ_ERR_INVALID_ARG, "T, H and D must be >= 1");
  if (D % 32 != 0 || D > 1024) return fail(QLQ_ERR_INVALID_ARG, "head_dim D must be a multiple of 32, at most 1024");
  if (T > kMaxDim || H > kMaxDim || T * H > kMaxDim) return fail(QLQ_ERR_INVALID_ARG, "T * H too large");
  return QLQ_OK;
}

qlq_status qlq_kv_quantize(const void* k_bf16, const void* v_bf16, int64_t T, int64_t H, int64_t D, void* k_codes,
                           void* k_scales, void* v_codes, void* v_scales, hipStream_t stream) {
  if (!k_bf16 || !v_bf16 || !k_codes || !k_scales || !v_codes || !v_scales)
    return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_kv_dims(T, H, D)) return st;
  if (!aligned(k_bf16, 2) || !aligned(v_bf16, 2) || !aligned(k_scales, 2) || !aligned(v_scales, 2))
    return fail(QLQ_ERR_INVALID_ARG, "misaligned pointer");
  return hip_status(qlq::launch_kv_quantize(k_bf16, v_bf16, T * H, (int)D, k_codes, k_scales, v_codes, v_scales,
                                            stream),
                    "kv_quantize");
}

qlq_status qlq_kv_dequantize(const void* k_codes, const void* k_scales, const void* v_codes, const void* v_scales,
                             int64_t T, int64_t H, int64_t D, void* k_bf16, void* v_bf16, hipStream_t stream) {
  if (!k_bf16 || !v_bf16 || !k_codes || !k_scales || !v_codes || !v_scales)
    return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_kv_dims(T, H, D)) return st;
  if (!aligned(k_codes, 8) || !aligned(v_codes, 8) || !aligned(k_bf16, 16) || !aligned(v_bf16, 16) ||
      !aligned(k_scales, 2) || !aligned(v_scales, 2))
    return fail(QLQ_ERR_INVALID_ARG, "misaligned pointer (codes 8-byte, outputs 16-byte aligned)");
  return hip_status(qlq::launch_kv_dequantize(k_codes, k_scales, v_codes, v_scales, T * H * D, (int)D, k_bf16,
                                              v_bf16, stream),
                    "kv_dequantize");
}

// Routed Linear: workspace layout [GEMM region][codes M*K][row scales 4M], the
// codes at the same offset as the fused static call (never below the counters).
static size_t linear_codes_offset(int64_t M, int64_t K, int64_t N, int qtype) {
  return fused_xq_offset(M, K, N, qtype);
}

size_t qlq_linear_workspace_bytes(qlq_scheme scheme, int64_t M, int64_t K, int64_t N, qlq_qtype qtype) {
  if (M < 1 || K < 1 || N < 1 || M > kMaxDim || K > kMaxDim || N > kMaxDim) return 0;
  const size_t w16 = gemm_ws_bytes(qlq::kW8A16, M, K, N, (int)qtype);
  if (scheme == QLQ_SCHEME_W8A16) return w16;
  if (scheme != QLQ_SCHEME_W8A8_STATIC && scheme != QLQ_SCHEME_W8A8_DYNAMIC) return 0;
  size_t need = linear_codes_offset(M, K, N, (int)qtype) + ((size_t)M * (size_t)K + 255) / 256 * 256 +
                (scheme == QLQ_SCHEME_W8A8_DYNAMIC ? (size_t)M * 4 : 0);
  return need > w16 ? need : w16;           // the BF16 fallback runs the W8A16 GEMM in the same buffer
}

qlq_status qlq_linear(qlq_scheme scheme, const void* x_bf16, int64_t M, int64_t K, int64_t N, const void* wq_packed,
                      const float* w_scale, int64_t w_scale_numel, qlq_qtype qtype, float input_scale,
                      const void* bias_bf16, int64_t bf16_fallback_max_m, void* y_bf16, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  if (qlq_status st = check_qtype(qtype)) return st;
  if (scheme != QLQ_SCHEME_W8A16 && scheme != QLQ_SCHEME_W8A8_STATIC && scheme != QLQ_SCHEME_W8A8_DYNAMIC)
    return fail(QLQ_ERR_UNSUPPORTED, "qlq_linear: unknown scheme %d", (int)scheme);
  if (bf16_fallback_max_m < 0) return fail(QLQ_ERR_INVALID_ARG, "bf16_fallback_max_m must be >= 0");
  if (scheme == QLQ_SCHEME_W8A8_STATIC)
    if (qlq_status st = check_scale(input_scale, "input_scale")) return st;
  if (scheme == QLQ_SCHEME_W8A16 || M <= bf16_fallback_max_m)
    return run_gemm(qlq::kW8A16, x_bf16, M, K, N, wq_packed, w_scale, w_scale_numel, qtype, 1.0f, nullptr, 0,
                    y_bf16, workspace, workspace_bytes, stream, "linear", bias_bf16);
  if (qlq_status st = check_w8a8(qtype, QLQ_OUT_BF16, K)) return st;
  if (!x_bf16 || !wq_packed || !w_scale || !y_bf16) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_dims(M, K, N)) return st;
  if (!aligned(x_bf16, 2)) return fail(QLQ_ERR_INVALID_ARG, "misaligned pointer");
  const size_t need = qlq_linear_workspace_bytes(scheme, M, K, N, qtype);
  if (!workspace || workspace_bytes < need)
    return fail(QLQ_ERR_INVALID_ARG, "workspace too small: need %zu bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(QLQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t off = linear_codes_offset(M, K, N, (int)qtype);
  void* xq = static_cast<uint8_t*>(workspace) + off;
  float* xs = scheme == QLQ_SCHEME_W8A8_DYNAMIC
                  ? reinterpret_cast<float*>(static_cast<uint8_t*>(xq) + ((size_t)M * (size_t)K + 255) / 256 * 256)
                  : nullptr;
  PreparedGemm g;
  if (qlq_status st = prepare_gemm(g, qlq::kW8A8, xq, M, K, N, wq_packed, w_scale, w_scale_numel, qtype,
                                   scheme == QLQ_SCHEME_W8A8_STATIC ? input_scale : 1.0f, xs, 0, y_bf16, workspace,
                                   off, "linear", bias_bf16))
    return st;
  hipError_t e = scheme == QLQ_SCHEME_W8A8_STATIC
                     ? qlq::launch_quant_act(x_bf16, M * K, input_scale, (int)qtype, xq, stream,
                                             calibrated_scale(input_scale))
                     : qlq::launch_quant_act_dynamic(x_bf16, (int)M, (int)K, (int)qtype, xq, xs, stream);
  if (qlq_status st = hip_status(e, "linear")) return st;
  return launch_gemm(g, stream);
}

// ------------------------------------------------------------------ test hooks

int qlq_scale_is_calibrated(float s) { return calibrated_scale(s) ? 1 : 0; }

qlq_status qlq_gemm_plan(qlq_scheme scheme, int64_t M, int64_t K, int64_t N, qlq_qtype qtype,
                         qlq_plan_info* info) {
  if (!info) return fail(QLQ_ERR_INVALID_ARG, "null pointer");
  if (qlq_status st = check_dims(M, K, N)) return st;
  if (qlq_status st = check_qtype(qtype)) return st;
  if (scheme != QLQ_SCHEME_W8A16 && scheme != QLQ_SCHEME_W8A8_STATIC && scheme != QLQ_SCHEME_W8A8_DYNAMIC &&
      scheme != QLQ_SCHEME_W8A8_STATIC_FUSED)
    return fail(QLQ_ERR_UNSUPPORTED, "unknown scheme %d", (int)scheme);
  const int sch = scheme == QLQ_SCHEME_W8A16 ? qlq::kW8A16 : qlq::kW8A8;
  const qlq::GemmPlan p = qlq::plan_gemm(sch, (int)qtype, M, K, N, K % 64 == 0);
  info->kind = p.kind;
  info->cfg = p.kind == 2 ? p.cfg : -1;
  info->split_k = p.S;
  info->tile_m = p.kind == 0 ? 16 * p.rw : p.BM;
  info->tile_n = p.kind == 0 ? 16 * p.ct : p.BN;
  info->waves = p.kind == 0 ? p.waves : 0;
  info->grid = p.grid;
  info->workspace_bytes = (int64_t)p.ws_bytes;
  return ok();
}

}  // extern "C"

// ------------------------------------------------------- allocation-free W8A16
// For callers that cannot allocate (HIP graph capture, tight serving loops): the
// split-K counters and partials live in this file-scope device array, one copy per
// GPU, instead of a caller's workspace.  Host code uses the array only through the
// device address hipGetSymbolAddress returns for the current device.

static __device__ __align__(256) uint8_t scratch[QLQ_NOALLOC_MAX_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = QLQ_NOALLOC_MAX_SCRATCH_BYTES;
static_assert(kScratchBytes > kCounterBytes, "scratch holds the counter region and partials");

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
qlq_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (qlq_status st = hip_status(hipGetDevice(&dev), "qlinear_w8a16_noalloc")) return st;
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(QLQ_ERR_UNSUPPORTED, "qlinear_w8a16_noalloc: device index %d above %d", dev, kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (qlq_status st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "qlinear_w8a16_noalloc: scratch"))
      return st;
    if (!p || !aligned(p, 256)) return fail(QLQ_ERR_HIP, "qlinear_w8a16_noalloc: scratch address unusable");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLQ_OK;
}

// Zeroes n arrival counters (a kernel, not a memset node, so the call stays capturable).
__global__ void clear_counters_kernel(uint32_t* c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = 0u;
}

}  // namespace

extern "C" qlq_status qlq_qlinear_w8a16_noalloc(const void* x_bf16, int64_t M, int64_t K, int64_t N,
                                                const void* wq_packed, const float* w_scale,
                                                int64_t w_scale_numel, qlq_qtype qtype, void* y_bf16,
                                                hipStream_t stream) {
  PreparedGemm g;
  if (qlq_status st = prepare_gemm(g, qlq::kW8A16, x_bf16, M, K, N, wq_packed, w_scale, w_scale_numel, qtype, 1.0f,
                                   nullptr, 0, y_bf16, kWorkspaceLater, 0, "qlinear_w8a16_noalloc"))
    return st;
  if (g.plan.ws_bytes > kScratchBytes)
    return fail(QLQ_ERR_INVALID_ARG,
                "qlinear_w8a16_noalloc: this plan needs %zu bytes of split-K scratch, above the %zu the "
                "allocation-free call holds (use qlq_qlinear_w8a16 with a workspace)",
                g.plan.ws_bytes, kScratchBytes);
  if (g.plan.ws_bytes > 0) {
    void* p = nullptr;
    if (qlq_status st = scratch_of_current_device(&p)) return st;
    if (qlq_status st = bind_workspace(g, p, kScratchBytes)) return st;
    // The array keeps the last call's contents: the counters this plan uses start at zero.
    const int n = g.plan.tiles;
    clear_counters_kernel<<<(n + 255) / 256, 256, 0, stream>>>(g.args.counters, n);
    if (qlq_status st = hip_status(hipGetLastError(), "qlinear_w8a16_noalloc")) return st;
  }
  return launch_gemm(g, stream);
}
