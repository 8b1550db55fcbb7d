// Host-only planning of the gemm_f32 library (see host_plan.hpp).
#include "host_plan.hpp"

#include <cstdint>

namespace gemm_f32_impl {

// ---- argument checks ---------------------------------------------------

namespace {

bool misaligned(const void *p, int align) {
  return (reinterpret_cast<std::uintptr_t>(p) & static_cast<std::uintptr_t>(align - 1)) != 0;
}

int max1(int v) { return v > 1 ? v : 1; }

}  // namespace

int check_shape(int M, int N, int K) {
  return (M < 0 || N < 0 || K < 0) ? kInvalidDim : kOk;
}

int check_ld(int N, int K, int lda, int ldb, int ldc) {
  return (lda < max1(K) || ldb < max1(N) || ldc < max1(N)) ? kInvalidLd : kOk;
}

int check_pointers(int M, int N, int K, const void *A, const void *B, const void *C,
                   int in_align) {
  if (M == 0 || N == 0) return kOk;
  if (C == nullptr) return kNullPtr;
  if (K > 0 && (A == nullptr || B == nullptr)) return kNullPtr;
  if (misaligned(C, 4) || (K > 0 && (misaligned(A, in_align) || misaligned(B, in_align))))
    return kMisaligned;
  return kOk;
}

int check_operands(int M, int N, int K, const void *A, int lda, const void *B, int ldb,
                   const void *C, int ldc, int in_align) {
  const int rc = check_ld(N, K, lda, ldb, ldc);
  return rc != kOk ? rc : check_pointers(M, N, K, A, B, C, in_align);
}

bool bad_buffer(const void *p) { return p == nullptr || misaligned(p, 4); }

// ---- the production kernel's launch table ------------------------------

namespace {

struct Entry {
  ProdConfig cfg;
  ProdKind kind;
};

// Index = launch-table entry of GEMM_F32_PROD.  The kernels behind each
// entry are in prod.hip and w16_vgpr.hip; the automatic choice uses 16, 19,
// 21, 22, 23, 24, 25, 26 and 27 (and 3 for thin strips), the others stay
// reachable by index for tests and measurements.  Entries 26 and 27 list
// the most rows (columns) a workgroup holds; gemm_f32_tile reports
// strip_rows(M) (strip_cols(N)).
const Entry kEntries[] = {
    {{128, 128, 32, 2, 2, 2, "128x128x32_w2x2"}, kKloop},
    {{128, 128, 16, 2, 2, 3, "128x128x16_w2x2"}, kKloop},
    {{256, 128, 16, 4, 2, 2, "256x128x16_w4x2"}, kKloop},
    {{64, 64, 32, 2, 2, 4, "64x64x32_w2x2"}, kKloop},
    {{128, 64, 32, 2, 2, 2, "128x64x32_w2x2"}, kKloop},
    {{128, 128, 32, 2, 2, 2, "128x128x32_w2x2_nt"}, kKloop},
    {{128, 128, 16, 2, 2, 3, "128x128x16_w2x2_nt"}, kKloop},
    {{256, 128, 32, 4, 2, 1, "256x128x32_w4x2"}, kKloop},
    {{128, 128, 64, 2, 2, 2, "panel128x128_k64"}, kPanel},
    {{256, 128, 64, 4, 2, 1, "panel256x128_k64"}, kPanel},
    {{256, 256, 16, 4, 4, 1, "256x256x16_w4x4"}, kKloop},
    {{256, 256, 16, 4, 2, 1, "256x256x16_w4x2"}, kKloop},
    {{256, 256, 32, 4, 4, 1, "256x256x32_w4x4"}, kKloop},
    {{256, 128, 64, 4, 2, 1, "panel256x128_k64_pipe"}, kPanel},
    {{256, 128, 64, 4, 2, 1, "panel256x128_k64_arow"}, kPanel},
    {{256, 256, 32, 4, 4, 1, "256x256x32_w4x4_ldsdma"}, kKloop},
    {{64, 64, 64, 2, 2, 1, "64x64x64_ksplit4_ldsdma"}, kKsplit},
    {{128, 128, 64, 2, 2, 1, "128x128x64_w16_ldsdma"}, kKsplit},
    {{256, 256, 32, 4, 4, 1, "256x256x32_w4x4_ldsdma_mfma16"}, kKsplit},
    {{256, 256, 32, 2, 2, 1, "256x256x32_w2x2_ldsdma_mfma16"}, kKsplit},
    {{256, 256, 32, 2, 2, 1, "256x256x32_w2x2_regs_mfma16"}, kKsplit},
    {{256, 128, 64, 2, 2, 1, "panel256x128_k64_arow_mfma16"}, kPanel},
    {{192, 192, 32, 2, 2, 1, "192x192x32_w2x2_ldsdma_mfma16"}, kKsplit},
    {{128, 128, 32, 2, 2, 2, "128x128x32_w2x2_ldsdma_mfma16"}, kKsplit},
    {{192, 256, 32, 2, 2, 1, "192x256x32_w2x2_ldsdma_mfma16"}, kKsplit},
    {{256, 256, 32, 2, 2, 1, "rows256_rounds+rest"}, kKsplit},
    {{16, 16, 1, 4, 2, 1, "strip_rows16_cols16"}, kStrip},
    {{16, 16, 1, 4, 2, 1, "strip_cols16_rows16"}, kStripN},
};
constexpr int kNumConfigs = sizeof(kEntries) / sizeof(kEntries[0]);

// ---- measured constants of the automatic choice -------------------------
//
// The choice is a model fitted to one MI355X (256 CUs): each candidate's
// sustained rate when every CU is busy, scaled by how busy the persistent
// grid keeps the CUs and by the useful fraction of its tiles' work.  The
// rates were measured with the ladder tool (10-20 calls after warm-up) on
// products that fill the chip; a change of clock policy or driver that moves
// them is caught by the host test that pins the choice on the shapes where
// every entry was timed, after which these numbers are re-measured.
//
//   entry  tile      K % 32 == 0   otherwise   slots  kernel
//   19     256x256   148           140         256    direct loads, 128x128 waves
//   24     192x256   140           -           256    direct loads, 96x128 waves
//   22     192x192   138           -           256    direct loads, 96x96 waves
//   23     128x128   141           -           512    direct loads, 64x64 waves
//   17     128x128   124           124         256    64x64 waves, register K tail
//   16     64x64     108           108         256    K split over the waves
//
// The entry 19 rate for partial K steps is its direct-load tail form on
// ragged 4097 x 4095 x 2049 (0.49 ms for the 4096-row main part).
const KloopRate kRates[] = {{19, 256, 256, 148.0, 140.0, 256}, {24, 192, 256, 140.0, 0.0, 256},
                            {22, 192, 192, 138.0, 0.0, 256},   {23, 128, 128, 141.0, 0.0, 512},
                            {17, 128, 128, 124.0, 124.0, 256}, {16, 64, 64, 108.0, 108.0, 256}};
constexpr int kNumRates = sizeof(kRates) / sizeof(kRates[0]);

constexpr long long kCus = 256;  // compute units of an MI355X

// The row cut pays only if it beats the single entry by more than the cost
// of its second launch.
constexpr double kLaunchUs = 4.0;

// Split-K plan: one 128 x 128 x 32 k step (1 MFLOP) takes about
// kStepUsPerMflop microseconds on one CU, and HBM moves about
// kStepHbmBytes in that time.
constexpr double kStepUsPerMflop = 2.0;
constexpr double kStepHbmBytes = 9.0e6;

}  // namespace

int prod_num_configs() { return kNumConfigs; }

const ProdConfig &prod_config(int index) { return kEntries[index].cfg; }

ProdKind prod_kind(int index) { return kEntries[index].kind; }

bool prod_supports(int index, int M, int N, int K) {
  if (index < 0 || index >= kNumConfigs) return false;
  if (kEntries[index].kind == kStrip) return M <= kStripMaxRows;
  if (kEntries[index].kind == kStripN) return N <= kStripMaxCols;
  return kEntries[index].kind != kPanel || K <= kEntries[index].cfg.BK;
}

int kloop_rate_count() { return kNumRates; }

const KloopRate &kloop_rate(int i) { return kRates[i]; }

int thin_remainder(int extent, int tile) {
  const int rem = extent % tile;
  return (extent > tile && rem > 0 && rem * 8 <= tile) ? rem : 0;
}

// Each candidate's score: its rate when every CU is busy, times the
// fraction of the time the CUs are busy on the persistent grid -- G =
// min(resident workgroups, tiles) workgroups, ceil(G / 256) of them per CU,
// ceil(tiles / G) tiles each, against tiles / 256 if the work spread evenly
// -- and times the useful fraction of the tiles' work (edge tiles moved back
// inside C repeat part of a neighbour's), counting tiles after the thin
// remainder strips are split off.
KloopModel model_kloop(int M, int N, int K) {
  const bool whole_steps = K % 32 == 0;
  KloopModel best{16, -1.0, 0.0};
  for (const KloopRate &c : kRates) {
    const double rate = whole_steps ? c.tflops_whole_steps : c.tflops_partial_steps;
    const long long tm = ceil_div(M - thin_remainder(M, c.bm), c.bm);
    const long long tn = ceil_div(N - thin_remainder(N, c.bn), c.bn);
    const long long tiles = tm * tn;
    if (tiles <= 0) continue;
    const long long grid = tiles < c.slots ? tiles : c.slots;
    const long long busy = ceil_div(grid, kCus) * ceil_div(tiles, grid);  // tile times per CU
    const double useful = (double)(M - thin_remainder(M, c.bm)) * (N - thin_remainder(N, c.bn)) /
                          ((double)tm * c.bm * (double)tn * c.bn);
    const double score = rate * useful * (double)tiles / (double)(busy * kCus);
    if (score > best.score) best = {c.entry, score, tiles >= c.slots ? score : 0.0};
  }
  return best;
}

// Entry 25 cuts C by rows: rows [0, 256 r) run entry 19 on whole rounds of
// 256x256 tiles (r * tiles-per-row <= 256 q for some q), the rest runs its
// own best k-loop entry in a second launch.  Returns the r whose modelled
// time beats the best single entry by more than a launch, else 0.
int region_rows(int M, int N, int K) {
  if (K % 32 != 0 || M < 512 || N < 256) return 0;
  const long long tn = ceil_div(N - thin_remainder(N, 256), 256);
  const long long tm = M / 256;
  const double flops_per_row = 2.0 * N * (double)K;
  const KloopModel whole = model_kloop(M, N, K);
  double best_us = flops_per_row * M / (whole.score * 1e6);
  int best_r = 0;
  const double rate19 = kRates[0].tflops_whole_steps;
  for (long long q = 1; q <= 8; ++q) {
    const long long r = 256 * q / tn;
    if (r < 1) continue;
    if (r >= tm) break;
    const int m1 = (int)(256 * r);
    if (M - m1 < 128) break;
    const double top = rate19 * (double)(r * tn) / (double)(ceil_div(r * tn, 256) * 256);
    const KloopModel rest = model_kloop(M - m1, N, K);
    const double us = flops_per_row * m1 / (top * 1e6) +
                      flops_per_row * (M - m1) / (rest.score * 1e6) + kLaunchUs;
    if (us < best_us) {
      best_us = us;
      best_r = (int)r;
    }
  }
  return best_r;
}

// Shape-based choice.  At most kStripMaxRows rows: the thin-M strip kernel
// (entry 26), which streams B once, where a tile kernel would fill its 64-
// to 256-row tiles with 1 to 32 useful rows (1 x 4095 x 2049: 91 us on the
// 64 x 64 K-split entry, 13 us as a strip; 32 x 4095 x 2049: 101 against
// 34 us).  At most kStripMaxCols columns: the thin-N kernel
// (entry 27), which streams A once.  K <= 64 with many tiles: the
// A-resident small-K kernel (only B moves per tile; C stores of one
// tile drained during the next tile's MFMAs), on 16x16 MFMAs with one wave
// per SIMD when K == 64 and the rows are aligned (entry 21's launcher falls
// back to the 32x32 form otherwise).  Otherwise entry 25 when its row cut
// models faster, else the k-loop entry with the best modelled rate
// (model_kloop).
int prod_choose(int M, int N, int K, double *full_rate) {
  if (full_rate) *full_rate = 0.0;
  if (M <= kStripMaxRows) return kStripConfig;
  if (N <= kStripMaxCols) return kColStripConfig;
  const long long t256x128 = ceil_div(M, 256) * ceil_div(N, 128);
  if (K <= 64 && t256x128 >= 1024) return 21;
  if (region_rows(M, N, K) > 0) return 25;
  const KloopModel m = model_kloop(M, N, K);
  if (full_rate) *full_rate = m.full_rate;
  return m.entry;
}

namespace {

// Entries the split-K path can run: the k-loop kernels without
// non-temporal stores (the slabs are read back at once).
bool split_supports(int index) {
  switch (index) {
    case 0: case 1: case 2: case 3: case 4: case 7: case 12: case 23: return true;
    default: return false;
  }
}

}  // namespace

// Split-K plan.  Automatic entry: 128 x 128 x 32 tiles (64 x 64 below a
// 128 x 128 output), two workgroups per CU -- entry 23, whose split form
// runs the direct-load 16x16-MFMA kernel where the product fits it and
// entry 0's otherwise.  Automatic split count: the one with the least
// estimated time, counted in k steps of one tile,
//   rounds(s) * ceil(ksteps / s) + (partial-slab bytes written and read back) / B,
// where rounds(s) = ceil(tiles * s / 256): a CU given two (tile, chunk) pairs
// takes about twice as long as one given one, so the launch's time is its
// busiest CU's; B is the HBM bytes moved in the time of one k step.  One
// split is the plain product: ceil(tiles / 256) * ksteps, or, when the plain
// product's own entry fills every workgroup slot (so its full-occupancy rate
// applies), that rate's time in steps.  Each split is at least four k steps
// deep; products with a tile for every CU, or fewer than 32 k steps, are
// not split.  An explicit count is honoured up to one k step per split.
// The chunk kc is a multiple of BK, and splits = ceil(K / kc).
bool splitk_plan(int M, int N, int K, int config, int splits, SplitPlan *out) {
  if (M < 0 || N < 0 || K < 0 || splits < 0 || out == nullptr) return false;
  const bool auto_config = config == -1;
  if (auto_config) config = (M < 128 && N < 128) ? 3 : 23;
  if (config < 0 || config >= kNumConfigs || !split_supports(config)) return false;
  const ProdConfig &c = kEntries[config].cfg;
  const long long tiles = ceil_div(M, c.BM) * ceil_div(N, c.BN);
  const long long ksteps = ceil_div(K, c.BK);
  long long want = splits;
  if (want == 0) {
    want = 1;
    if (tiles > 0 && tiles < kCus && ksteps >= 32) {
      const double step_bytes = kStepHbmBytes * ((double)c.BM * c.BN * c.BK / (128.0 * 128.0 * 32.0));
      const double slab_bytes = 8.0 * M * N;  // one chunk's partial written and read back
      long long most = ksteps / 4;
      if (most > 4 * kCus) most = 4 * kCus;
      double best = (double)ksteps;  // one split: one round, no slabs
      double plain_rate;
      prod_choose(M, N, K, &plain_rate);
      if (plain_rate > 0.0) {  // TFLOP/s -> k steps of 1 MFLOP
        const double plain_steps =
            2.0 * M * N * (double)K / (plain_rate * 1e6) / kStepUsPerMflop;
        if (plain_steps < best) best = plain_steps;
      }
      for (long long sp = 2; sp <= most; ++sp) {
        const double est = (double)ceil_div(tiles * sp, kCus) * ceil_div(ksteps, sp) +
                           sp * slab_bytes / step_bytes;
        if (est < best) {
          best = est;
          want = sp;
        }
      }
    }
  }
  if (want > ksteps) want = ksteps;
  if (want > kMaxGridY) want = kMaxGridY;
  if (want < 1) want = 1;
  const long long kc = ceil_div(ksteps, want) * c.BK;
  const long long used = K > 0 ? ceil_div(K, kc) : 1;
  // Unsplit with an automatic entry: the plain product's own choice.
  out->config = used == 1 && auto_config ? prod_choose(M, N, K) : config;
  out->splits = (int)used;
  out->kc = (int)kc;
  out->workspace_bytes = used > 1 ? used * (long long)M * N * 4 : 0;
  return true;
}

}  // namespace gemm_f32_impl
