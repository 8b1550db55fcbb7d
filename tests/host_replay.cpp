// Host replay of the production kernels' memory addresses and of the
// host-side plan, built with the address and undefined-behaviour sanitizers
// by tests/test_host_sanitized.py (no GPU).
//
// For the benchmark's workloads and a sweep of edge shapes it follows
// launch_prod's split of each product into a main part and thin strips,
// takes the entry the automatic choice runs, and replays every tile of the
// kernels those workloads use -- the direct-load 128x128-wave kernel (whole
// and partial last k steps), the K-split 64x64 kernel (per-wave direct loads and
// its per-wave register tail), the A-resident small-K kernel and the thin-M
// strip kernel -- with the same constexpr index functions the kernels call
// (addr_math.hpp): every 16-byte load must lie inside its matrix's rows and
// columns (not merely inside the allocation), every store inside C's M x N
// window, and every direct-load lane offset below 2^32.  It also checks the
// 32-bit offset guard at its boundary for each direct-load tile family, the
// guarded and partial windows exhaustively on small sizes, the 16-bit
// kernels' LDS layouts, and invariants of the automatic choice and the
// split-K plan.
//
// Loads at k steps between the first and the last whole step are not all
// replayed: for a fixed lane and instruction the column (A) or row (B) grows
// with the step, so the first and last whole steps bound the rest.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "addr_math.hpp"
#include "addr_math16.hpp"
#include "host_plan.hpp"

using namespace gemm_f32_impl;

namespace {

struct Shape {
  int M, N, K;
  long long lda, ldb, ldc;
  const char *name;
};

long long g_checks = 0;
int g_failures = 0;
// --plant-unclamped: replay with the edge tiles left overhanging C (the
// clamp of edge_tile_origin skipped), a mistake the replay must report.
bool g_plant_unclamped = false;

void origin(int t, int tiles_m, int tiles_n, int BM, int BN, const struct Shape &s, int &m0,
            int &n0);

void fail(const Shape &s, const char *what, long long a, long long b) {
  if (g_failures < 25)
    std::printf("FAIL %s %dx%dx%d (lda %lld ldb %lld): %s [%lld, %lld]\n", s.name, s.M, s.N, s.K,
                s.lda, s.ldb, what, a, b);
  ++g_failures;
}

void origin(int t, int tiles_m, int tiles_n, int BM, int BN, const Shape &s, int &m0, int &n0) {
  if (g_plant_unclamped) {
    int tm = 0, tn = 0;
    tile_coords(t, tiles_m, tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
    return;
  }
  edge_tile_origin(t, tiles_m, tiles_n, BM, BN, s.M, s.N, m0, n0);
}

// A 16-byte load of A at element offset e from A: inside rows [0, M) and
// columns [0, K).
void check_a(const Shape &s, long long e, const char *what) {
  ++g_checks;
  if (e < 0) return fail(s, what, e, -1);
  const long long row = e / s.lda, col = e % s.lda;
  if (row >= s.M || col + 4 > s.K) fail(s, what, row, col);
}

// A one-element load of A[row][col].
void check_a1(const Shape &s, long long row, long long col, const char *what) {
  ++g_checks;
  if (row < 0 || col < 0 || row >= s.M || col >= s.K) fail(s, what, row, col);
}

void check_b(const Shape &s, long long e, const char *what) {
  ++g_checks;
  if (e < 0) return fail(s, what, e, -1);
  const long long row = e / s.ldb, col = e % s.ldb;
  if (row >= s.K || col + 4 > s.N) fail(s, what, row, col);
}

// A store of n floats at C[i][j..j+n).
void check_c(const Shape &s, long long i, long long j, int n, const char *what) {
  ++g_checks;
  if (i < 0 || j < 0 || i >= s.M || j + n > s.N) fail(s, what, i, j);
}

// A direct load's per-lane byte offset must fit the 32-bit operand.
void check_voff(const Shape &s, long long elem, const char *what) {
  ++g_checks;
  if (elem < 0 || elem * 4 >= (1LL << 32)) fail(s, what, elem, 0);
}

// ---- direct-load one-wave-per-SIMD kernels (entries 19, 22, 23, 24) -------
// BM x BN tiles (BM = 2 WTM, BN = 2 WTN), 32-deep steps; per step the
// workgroup issues BM / 8 A and BN / 8 B direct loads of 1 KB (A chunk
// layout ACH = 8, B layout BCH = BN / 4).  Entry 19 (256 x 256) takes
// dword-aligned rows and a partial last step; the others need 16-byte
// aligned rows and K a multiple of 32.
template <int WTM, int WTN>
bool big16_takes(const Shape &s, bool any_k) {
  constexpr int BM = 2 * WTM, BN = 2 * WTN, BK = 32;
  const bool k_ok = any_k ? s.K >= BK : (s.K > 0 && s.K % BK == 0);
  const bool rows_ok = any_k || (s.lda % 4 == 0 && s.ldb % 4 == 0 && s.N % 4 == 0);
  return s.M >= BM && s.N >= BN && k_ok && rows_ok && lane_offsets_fit(BM, s.lda, 4) &&
         lane_offsets_fit(BK, s.ldb, 4);
}

template <int WTM, int WTN>
void replay_big16(const Shape &s) {
  constexpr int BM = 2 * WTM, BN = 2 * WTN, BK = 32;
  const bool tail = s.K % BK != 0;
  const int tiles_m = (int)ceil_div(s.M, BM), tiles_n = (int)ceil_div(s.N, BN);
  const int nk = (int)ceil_div(s.K, BK), nfull = s.K / BK;
  std::vector<int> k0s = {0, (nfull - 1) * BK};
  if (tail) k0s.push_back(s.K - BK);  // the pre-tail step's clamped loads
  for (int t = 0; t < tiles_m * tiles_n; ++t) {
    int m0 = 0, n0 = 0;
    origin(t, tiles_m, tiles_n, BM, BN, s, m0, n0);
    for (int k0 : k0s) {
      for (int blk = 0; blk < BM / 8; ++blk)
        for (int lane = 0; lane < 64; ++lane) {
          const long long ea = dma_a_elem<BK / 4>(blk, lane, s.lda);
          check_voff(s, ea, "w16 A lane offset");
          check_a(s, (long long)m0 * s.lda + k0 + ea, "w16 A direct load");
        }
      for (int blk = 0; blk < BN / 8; ++blk)
        for (int lane = 0; lane < 64; ++lane) {
          const long long eb = dma_b_elem<BN / 4>(64 * blk + lane, s.ldb);
          check_voff(s, eb, "w16 B lane offset");
          check_b(s, (long long)k0 * s.ldb + n0 + eb, "w16 B direct load");
        }
    }
    if (tail) {  // w16_fill_partial over 256 threads
      const int k0 = (nk - 1) * BK;
      for (int tid = 0; tid < 256; ++tid) {
        const int arow = tid / (BK / 4), ac = tid % (BK / 4);
        const int bkr = tid / (BN / 4), bc = tid % (BN / 4);
        int valid = 0, shift = 0;
        const int col = tail_window(k0 + 4 * ac, s.K, valid, shift);
        if (valid > 0 && col + shift != k0 + 4 * ac) fail(s, "tail window shift", col, shift);
        for (int i = 0; i < BM / (256 / (BK / 4)); ++i)
          check_a(s, (long long)(m0 + arow + (256 / (BK / 4)) * i) * s.lda + col, "w16 tail A");
        for (int i = 0; i < BK / (256 / (BN / 4)); ++i) {
          const int k = k0 + bkr + (256 / (BN / 4)) * i;
          check_b(s, (long long)(k < s.K ? k : s.K - 1) * s.ldb + n0 + 4 * bc, "w16 tail B");
        }
      }
    }
    for (int wave = 0; wave < 4; ++wave)
      for (int bm = 0; bm < WTM / 16; ++bm)
        for (int bn = 0; bn < WTN / 16; ++bn)
          for (int lane = 0; lane < 64; ++lane)
            check_c(s, m0 + (wave >> 1) * WTM + 16 * bm + (lane & 15),
                    n0 + (wave & 1) * WTN + 16 * bn + 4 * (lane >> 4), 4, "w16 C store");
  }
}

// ---- K-split 64x64 kernel (entry 16) ----------------------------------------
bool ksplit_takes(const Shape &s) {  // launch_ksplit's condition (pointers aligned)
  return s.lda % 4 == 0 && s.ldb % 4 == 0 && s.N % 4 == 0 && s.M >= 64 && s.N >= 64 &&
         lane_offsets_fit(64, s.lda, 4) && lane_offsets_fit(64, s.ldb, 4);
}

void replay_ksplit(const Shape &s) {
  const bool tail = s.K % 64 != 0;
  const int tiles_m = (int)ceil_div(s.M, 64), tiles_n = (int)ceil_div(s.N, 64);
  const int nk = (int)ceil_div(s.K, 64), nfull = s.K / 64;
  std::vector<int> k0s;
  if (nfull > 0) k0s = {0, (nfull - 1) * 64};
  for (int t = 0; t < tiles_m * tiles_n; ++t) {
    int m0 = 0, n0 = 0;
    origin(t, tiles_m, tiles_n, 64, 64, s, m0, n0);
    for (int k0 : k0s)
      for (int wave = 0; wave < 4; ++wave)
        for (int q = 0; q < 4; ++q)
          for (int lane = 0; lane < 64; ++lane) {
            const long long ea = ks_dma_a_elem(q, lane, wave, s.lda);
            const long long eb = dma_b_elem<16>(64 * (4 * wave + q) + lane, s.ldb);
            check_voff(s, ea, "ksplit A lane offset");
            check_voff(s, eb, "ksplit B lane offset");
            check_a(s, (long long)m0 * s.lda + k0 + ea, "ksplit A direct load");
            check_b(s, (long long)k0 * s.ldb + n0 + eb, "ksplit B direct load");
          }
    if (tail) {  // ks_fill_partial: each wave its own quarter, zero past K
      const int k0 = (nk - 1) * 64;
      for (int wave = 0; wave < 4; ++wave)
        for (int lane = 0; lane < 64; ++lane)
          for (int q = 0; q < 4; ++q) {
            const int r = 16 * q + lane / 4, kc = k0 + 16 * wave + 4 * (lane & 3);
            const int valid = chunk_valid(kc, s.K);
            if (valid == 4)
              check_a(s, (long long)(m0 + r) * s.lda + kc, "ksplit tail A");
            else
              for (int e = 0; e < valid; ++e)
                check_a1(s, m0 + r, kc + e, "ksplit tail A element");
            const int k = k0 + 16 * wave + 4 * q + lane / 16;
            if (k < s.K) check_b(s, (long long)k * s.ldb + n0 + 4 * (lane & 15), "ksplit tail B");
          }
    }
    // final reduction: wave w stores rows 16 w .. 16 w + 15, 4 chunks per lane
    for (int wave = 0; wave < 4; ++wave)
      for (int lane = 0; lane < 64; ++lane)
        for (int j = 0; j < 4; ++j)
          check_c(s, m0 + 16 * wave + (lane >> 2), n0 + 4 * (4 * j + (lane & 3)), 4,
                  "ksplit C store");
  }
}

// ---- A-resident small-K kernel (entry 21) -----------------------------------
bool arow16_takes(const Shape &s) {
  return s.K == 64 && s.M % 256 == 0 && s.N % 128 == 0 && s.M > 0 && s.N > 0 && s.lda % 4 == 0 &&
         s.ldb % 4 == 0 && lane_offsets_fit(256, s.lda, 4) && lane_offsets_fit(64, s.ldb, 4);
}

void replay_arow16(const Shape &s, int slots) {
  const int panels = s.M / 256, tiles_n = s.N / 128;
  long long chunks = ceil_div(slots, panels);
  if (chunks > tiles_n) chunks = tiles_n;
  if (chunks < 1) chunks = 1;
  const int G = (int)(panels * chunks);
  std::vector<char> seen(G, 0);
  for (int b = 0; b < G; ++b) {
    const int lid = xcd_remap(b, G);
    if (lid < 0 || lid >= G || seen[lid]) fail(s, "arow16 xcd_remap not a permutation", b, lid);
    else seen[lid] = 1;
    const int panel = lid / (int)chunks, chunk = lid % (int)chunks;
    if (panel >= panels) continue;
    const int t0 = (int)((long long)chunk * tiles_n / chunks);
    const int t1 = (int)((long long)(chunk + 1) * tiles_n / chunks);
    const int n = t1 - t0;
    if (n < 1) {
      fail(s, "arow16 empty chunk", chunk, n);
      continue;
    }
    const int m0 = panel * 256, rot = panel % n;
    auto col = [&](int i) {
      const int k = i < n ? i : n - 1;
      return (t0 + (k + rot) % n) * 128;
    };
    for (int blk = 0; blk < 64; ++blk)
      for (int lane = 0; lane < 64; ++lane) {
        const long long ea = dma_a_elem<16>(blk, lane, s.lda);
        check_voff(s, ea, "arow16 A lane offset");
        check_a(s, (long long)m0 * s.lda + ea, "arow16 A panel load");
      }
    for (int i = 0; i <= n; ++i) {
      const int n0 = col(i);
      for (int blk = 0; blk < 32; ++blk)
        for (int lane = 0; lane < 64; ++lane) {
          const long long eb = dma_b_elem<32>(64 * blk + lane, s.ldb);
          check_voff(s, eb, "arow16 B lane offset");
          check_b(s, n0 + eb, "arow16 B load");
        }
      if (i == n) break;
      for (int wave = 0; wave < 4; ++wave)
        for (int bm = 0; bm < 8; ++bm)
          for (int bn = 0; bn < 4; ++bn)
            for (int lane = 0; lane < 64; ++lane)
              check_c(s, m0 + (wave >> 1) * 128 + 16 * bm + (lane & 15),
                      n0 + (wave & 1) * 64 + 16 * bn + 4 * (lane >> 4), 4, "arow16 C store");
    }
  }
}

// ---- thin-M strip kernel ------------------------------------------------------
// 512 threads: 4 column quads x 128 k slices, 16 columns per workgroup.
void replay_strip(const Shape &s) {
  const int wgs = (int)ceil_div(s.N, 16);
  const int R = strip_rows(s.M), NB = strip_batch_quads(R), KB = 512;
  auto row_of = [&](int r) { return r < s.M ? r : s.M - 1; };  // rows past M read row M - 1
  for (int w = 0; w < wgs; ++w) {
    const long long n0 = 16LL * xcd_remap(w, wgs);
    const bool whole = n0 + 16 <= s.N;
    for (int tid = 0; tid < 512; ++tid) {
      const int c4 = (tid & 3) * 4, k0 = 4 * (tid >> 2);
      const int valid = (int)(s.N - n0) - c4;
      auto b_row = [&](int k, const char *what) {
        if (whole) {
          check_b(s, (long long)k * s.ldb + n0 + c4, what);
        } else {
          for (int j = 0; j < 4 && j < valid; ++j) {
            ++g_checks;
            if (k < 0 || k >= s.K || n0 + c4 + j >= s.N) fail(s, what, k, n0 + c4 + j);
          }
        }
      };
      int k = k0;
      for (; k + (NB - 1) * KB + 3 < s.K; k += NB * KB) {  // whole batches
        if (k != k0 && k + (2 * NB - 1) * KB + 3 < s.K) continue;  // first and last batch
        for (int u = 0; u < NB; ++u) {
          for (int t = 0; t < 4; ++t) b_row(k + u * KB + t, "strip B row");
          for (int r = 0; r < R; ++r)
            check_a(s, (long long)row_of(r) * s.lda + k + u * KB, "strip A chunk");
        }
      }
      if (k < s.K) {  // the guarded batch: k past K clamped to K - 1
        for (int u = 0; u < NB; ++u)
          for (int t = 0; t < 4; ++t) {
            const int kk = k + u * KB + t, kc = kk < s.K ? kk : s.K - 1;
            b_row(kc, "strip guarded B row");
            for (int r = 0; r < R; ++r) check_a1(s, row_of(r), kc, "strip guarded A");
          }
      }
    }
    for (int tid = 0; tid < 16 * R; ++tid) {
      const int r = tid / 16, c = tid % 16;
      if (r < s.M && n0 + c < s.N) check_c(s, r, n0 + c, 1, "strip C store");
    }
  }
}

// Thin-N kernel (colstrip_kernel): per workgroup of 16 rows and lane, the
// B values it stages per chunk of 1024 k, its A quads (whole or per element
// past K), and the C stores.  First and last chunks of each lane.
void check_b1(const Shape &s, long long k, long long n, const char *what) {
  ++g_checks;
  if (k < 0 || n < 0 || k >= s.K || n >= s.N) fail(s, what, k, n);
}

void replay_colstrip(const Shape &s) {
  const int NC = strip_cols(s.N), KC = col_chunk(NC), STEP = 128;
  const long long wgs = ceil_div(s.M, 16);
  for (long long w = 0; w < wgs; ++w) {
    const long long m0 = 16 * w;
    for (int tid = 0; tid < 512; ++tid) {
      const int lane = tid & 63, wave = tid >> 6, split = wave >> 1;
      const int r = 8 * (wave & 1) + (lane >> 3), q = lane & 7;
      const long long m = m0 + r < s.M ? m0 + r : s.M - 1;  // rows past M read row M - 1
      for (int kc0 = 0; kc0 < s.K; kc0 += KC) {
        if (kc0 != 0 && kc0 + 2 * KC < s.K) continue;
        const int kn = s.K - kc0 < KC ? s.K - kc0 : KC;
        for (int v = 0; v < KC * NC / 512; ++v) {
          const int i = tid + 512 * v, k = i / NC, n = i % NC;
          if (k < kn && n < s.N) check_b1(s, kc0 + k, n, "colstrip B staging");
        }
        for (int j = 0; j < KC / STEP; ++j) {
          const int k = kc0 + STEP * j + 32 * split + 4 * q;
          if (kn == KC || k + 4 <= s.K) {
            check_a(s, m * s.lda + k, "colstrip A quad");
          } else {
            for (int t = 0; t < 4; ++t)
              if (k + t < s.K) check_a1(s, m, k + t, "colstrip A tail");
          }
        }
      }
    }
    for (int tid = 0; tid < 16 * NC; ++tid) {
      const int rr = tid / NC, n = tid % NC;
      if (m0 + rr < s.M && n < s.N) check_c(s, m0 + rr, n, 1, "colstrip C store");
    }
  }
}

// ---- one product as launch_prod runs it --------------------------------------
// The entry's main part, its thin strips (bottom strips of up to 8 rows on
// the thin-M kernel are replayed; other strips run entry 3's register path),
// and entry 25's row cut into two launches.  Kernels other than those of
// entries 16, 19, 21, 22, 23 and 24 (and the fallbacks those launchers take
// for unaligned rows) are not replayed.
void replay_entry(int entry, const Shape &s) {
  if (s.M <= 0 || s.N <= 0) return;
  if (!prod_supports(entry, s.M, s.N, s.K)) fail(s, "entry refuses the shape", entry, 0);
  if (entry == 25) {
    const int r = region_rows(s.M, s.N, s.K);
    if (r == 0) return replay_entry(model_kloop(s.M, s.N, s.K).entry, s);
    Shape top = s, rest = s;
    top.M = 256 * r;
    rest.M = s.M - top.M;
    replay_entry(19, top);
    return replay_entry(model_kloop(rest.M, rest.N, rest.K).entry, rest);
  }
  if (prod_kind(entry) == kStrip) return replay_strip(s);
  if (prod_kind(entry) == kStripN) return replay_colstrip(s);
  const ProdConfig &c = prod_config(entry);
  int rm = entry == kRemainderConfig ? 0 : thin_remainder(s.M, c.BM);
  int rn = entry == kRemainderConfig ? 0 : thin_remainder(s.N, c.BN);
  if (prod_kind(entry) == kPanel) {
    rm = s.M % c.BM;
    rn = s.N % c.BN;
  }
  Shape main = s;
  main.M = s.M - rm;
  main.N = s.N - rn;
  if (entry == 19 && big16_takes<128, 128>(main, true)) replay_big16<128, 128>(main);
  if (entry == 22 && big16_takes<96, 96>(main, false)) replay_big16<96, 96>(main);
  if (entry == 23 && big16_takes<64, 64>(main, false)) replay_big16<64, 64>(main);
  if (entry == 24 && big16_takes<96, 128>(main, false)) replay_big16<96, 128>(main);
  if (entry == 16 && ksplit_takes(main)) replay_ksplit(main);
  if (entry == 21 && arow16_takes(main)) replay_arow16(main, 256);
  if (rm > 0 && rm <= kStripMaxRows) {  // bottom strip on the thin-M kernel
    Shape strip = s;
    strip.M = rm;
    replay_strip(strip);
  }
}

void replay_product(const Shape &s) { replay_entry(prod_choose(s.M, s.N, s.K), s); }

// ---- the 32-bit lane-offset guard at its boundary ------------------------------
// Largest leading dimension the guard admits for a tile of `rows` rows; the
// direct-load offsets of that tile at that ld must stay below 2^32, and the
// next ld must be refused.
template <int ACH>
void boundary_a(int rows, const char *family) {
  const Shape s{rows, 64, 4 * ACH, 0, 0, 0, family};
  const long long ld = (1LL << 32) / (rows * 4LL);
  if (!lane_offsets_fit(rows, ld, 4) || lane_offsets_fit(rows, ld + 1, 4))
    fail(s, "guard boundary (A)", ld, rows);
  const int blocks = rows * ACH / 64;
  for (int blk = 0; blk < blocks; ++blk)
    for (int lane = 0; lane < 64; ++lane) check_voff(s, dma_a_elem<ACH>(blk, lane, ld), family);
}

template <int BCH>
void boundary_b(int rows, const char *family) {
  const Shape s{64, 4 * BCH, rows, 0, 0, 0, family};
  const long long ld = (1LL << 32) / (rows * 4LL);
  if (!lane_offsets_fit(rows, ld, 4) || lane_offsets_fit(rows, ld + 1, 4))
    fail(s, "guard boundary (B)", ld, rows);
  const int blocks = rows * BCH / 64;
  for (int blk = 0; blk < blocks; ++blk)
    for (int lane = 0; lane < 64; ++lane)
      check_voff(s, dma_b_elem<BCH>(64 * blk + lane, ld), family);
}

// The K-split kernel's per-wave A quarters: at the guard's boundary every
// lane offset fits, the layout is a bijection of a wave's 256 chunk
// positions, a direct load's lane lands where the layout puts its chunk,
// and a fragment read (one chunk of 16 consecutive rows) touches distinct
// 16-byte bank groups within every 8 and every 16 lanes.
void check_ksplit_quarters() {
  const Shape s{64, 64, 64, 0, 0, 0, "K-split A quarters"};
  const long long ld = (1LL << 32) / (64 * 4LL);
  if (!lane_offsets_fit(64, ld, 4) || lane_offsets_fit(64, ld + 1, 4))
    fail(s, "guard boundary (K-split A)", ld, 64);
  for (int wave = 0; wave < 4; ++wave)
    for (int q = 0; q < 4; ++q)
      for (int lane = 0; lane < 64; ++lane) {
        const long long e = ks_dma_a_elem(q, lane, wave, ld);
        check_voff(s, e, "K-split A lane offset at the boundary");
        const int r = (int)(e / ld), c = (int)((e % ld) - 16 * wave) / 4;
        ++g_checks;
        if (r != 16 * q + lane / 4 || c < 0 || c > 3 || ks_a_pos(r, c) != 64 * q + lane)
          fail(s, "K-split A load position", 64 * q + lane, ks_a_pos(r, c));
      }
  std::vector<char> seen(256, 0);
  for (int r = 0; r < 64; ++r)
    for (int c = 0; c < 4; ++c) {
      const int pos = ks_a_pos(r, c);
      ++g_checks;
      if (pos < 0 || pos >= 256 || seen[pos]++) fail(s, "K-split A layout not a bijection", r, c);
    }
  for (int r0 = 0; r0 < 64; r0 += 16)
    for (int c = 0; c < 4; ++c)
      for (int span : {8, 16})
        for (int l0 = 0; l0 < 16; l0 += span) {
          std::vector<char> bank(span, 0);
          for (int l = l0; l < l0 + span; ++l) {
            const int b = ks_a_pos(r0 + l, c) % span;
            ++g_checks;
            if (bank[b]++) fail(s, "K-split A fragment read bank conflict", r0 + l, c);
          }
        }
}

// ---- the 16-bit direct-load kernels' LDS layouts (entries 3 and 4 of gemm_mixed) --
// Each layout is a bijection of its stage's 16-byte chunks; the lane of a
// direct load that fills position j loads the chunk the layout puts at j;
// at the guard's boundary (2-byte codes) every lane offset fits.  Fragment
// reads: a 16-byte A read of 16 consecutive rows lands on 16 distinct
// 16-byte bank groups of a 256-byte window; a transposing 8-byte B read
// puts each 16-lane group's four 32-byte pieces on distinct positions of a
// 128-byte window and each 32-lane half's eight on distinct positions of a
// 256-byte window.
void check_voff16(const Shape &s, long long elem, const char *what) {
  ++g_checks;
  if (elem < 0 || elem * 2 + 16 > (1LL << 32)) fail(s, what, elem, 0);
}

template <bool M32>
void check_mixed16_b(const Shape &s) {
  const char *name = M32 ? "32x32x16 B" : "16x16x32 B";
  std::vector<char> seen(64 * 16, 0);
  for (int k = 0; k < 64; ++k)
    for (int sl = 0; sl < 16; ++sl) {
      const int pos = M32 ? m32_b_slot(k, sl) : m16_b_slot(k, sl);
      ++g_checks;
      if (pos < 0 || pos >= 16 || seen[16 * k + pos]++) fail(s, name, k, sl);
    }
  const long long ld = 1000;
  for (int j = 0; j < 64 * 32; ++j) {
    const long long e = m16_dma_b_elem<M32>(j, ld);
    const int k = (int)(e / ld), col = (int)(e % ld), sl = col / 16;
    const int pos = M32 ? m32_b_slot(k, sl) : m16_b_slot(k, sl);
    ++g_checks;
    if (k != j / 32 || col % 8 != 0 || sl >= 16 || 32 * k + 2 * pos + (col % 16) / 8 != j)
      fail(s, "16-bit B load position", j, e);
  }
  // Transposing reads: lane (16-lane group q, l16) reads 8 bytes at byte
  // 32 * slot_pos + 8 (l16 % 4) of k row kbase + l16 / 4 (+ 8 for the second
  // half of the 16x16x32 kernel's groups); rows are 512 bytes apart.
  for (int kb = 0; kb < 64; kb += 4)
    for (int sl0 = 0; sl0 < 16; ++sl0) {
      if (M32 && (sl0 & 1)) continue;
      if (!M32 && (kb & 8)) continue;
      if (!M32 && kb + 8 + 3 >= 64) continue;
      std::vector<long long> addr;
      for (int lane = 0; lane < 32; ++lane) {
        const int q = lane / 16, l16 = lane % 16;
        const int k = kb + l16 / 4 + (M32 ? 0 : 8 * q);
        const int sl = M32 ? sl0 + q : sl0;
        const int pos = M32 ? m32_b_slot(k, sl) : m16_b_slot(k, sl);
        addr.push_back(512LL * k + 32 * pos + 8 * (l16 % 4));
      }
      for (int span : {16, 32}) {
        const int window = 8 * span;  // bytes served per cycle in that model
        for (int l0 = 0; l0 < 32; l0 += span) {
          std::vector<char> bank(window / 8, 0);
          for (int l = l0; l < l0 + span; ++l) {
            ++g_checks;
            if (bank[(addr[l] % window) / 8]++) fail(s, "16-bit B transposing read bank conflict", kb, sl0);
          }
        }
      }
    }
}

void check_mixed16_layouts() {
  const Shape s{256, 256, 64, 0, 0, 0, "16-bit direct-load layouts"};
  std::vector<char> seen(256 * 8, 0);
  for (int r = 0; r < 256; ++r)
    for (int c = 0; c < 8; ++c) {
      const int pos = m16_a_pos(r, c);
      ++g_checks;
      if (pos < 0 || pos >= 2048 || seen[pos]++) fail(s, "16-bit A layout not a bijection", r, c);
    }
  const long long ld = 1000;
  for (int j = 0; j < 2048; ++j) {
    const long long e = m16_dma_a_elem(j, ld);
    const int r = (int)(e / ld), col = (int)(e % ld);
    ++g_checks;
    if (col % 8 != 0 || col / 8 >= 8 || m16_a_pos(r, col / 8) != j)
      fail(s, "16-bit A load position", j, e);
  }
  for (int r0 = 0; r0 < 256; r0 += 16)
    for (int c = 0; c < 8; ++c) {
      std::vector<char> bank(16, 0);
      for (int l = 0; l < 16; ++l) {
        ++g_checks;
        if (bank[m16_a_pos(r0 + l, c) % 16]++) fail(s, "16-bit A fragment read bank conflict", r0 + l, c);
      }
    }
  check_mixed16_b<false>(s);
  check_mixed16_b<true>(s);
  // the guard: 256 rows of A and 64 k rows of B, 2-byte codes
  const long long lda = (1LL << 32) / (256 * 2LL), ldb = (1LL << 32) / (64 * 2LL);
  if (!lane_offsets_fit(256, lda, 2) || lane_offsets_fit(256, lda + 1, 2))
    fail(s, "guard boundary (16-bit A)", lda, 256);
  if (!lane_offsets_fit(64, ldb, 2) || lane_offsets_fit(64, ldb + 1, 2))
    fail(s, "guard boundary (16-bit B)", ldb, 64);
  for (int j = 0; j < 2048; ++j) check_voff16(s, m16_dma_a_elem(j, lda), "16-bit A lane offset");
  for (int j = 0; j < 2048; ++j) {
    check_voff16(s, m16_dma_b_elem<false>(j, ldb), "16-bit B lane offset (16x16x32)");
    check_voff16(s, m16_dma_b_elem<true>(j, ldb), "16-bit B lane offset (32x32x16)");
  }
}

// ---- windows, exhaustively on small sizes ---------------------------------------
void check_windows() {
  const Shape s{0, 0, 0, 0, 0, 0, "windows"};
  for (int rows = 1; rows <= 6; ++rows)
    for (int cols = 4; cols <= 40; ++cols)
      for (long long ld = cols; ld <= cols + 5; ld += 5)
        for (int row = 0; row < rows + 2; ++row)
          for (int col = 0; col < cols + 8; col += 4) {
            int meta = -1;
            const long long off = guarded_window(row, rows, col, cols, ld, meta);
            const int valid = meta >> 2, shift = meta & 3;
            ++g_checks;
            const long long r = off / ld, cc = off % ld;
            if (r >= rows || cc + 4 > cols) fail(s, "guarded window outside", off, meta);
            const int want = row < rows && col < cols ? (col + 4 <= cols ? 4 : cols - col) : 0;
            if (valid != want) fail(s, "guarded window count", valid, want);
            if (valid > 0 && (r != row || cc + shift != col)) fail(s, "guarded window place", r, cc);
          }
  for (int K = 4; K <= 100; ++K)
    for (int kc = 0; kc < K + 36; kc += 4) {
      int valid = -1, shift = -1;
      const int col = tail_window(kc, K, valid, shift);
      ++g_checks;
      if (col < 0 || col + 4 > K) fail(s, "tail window outside", kc, K);
      const int want = kc + 4 <= K ? 4 : (kc < K ? K - kc : 0);
      if (valid != want || (valid > 0 && col + shift != kc)) fail(s, "tail window place", kc, K);
    }
}

// ---- workgroup order ---------------------------------------------------------------
void check_orders() {
  const Shape s{0, 0, 0, 0, 0, 0, "orders"};
  for (int G = 1; G <= 1100; G += (G < 64 ? 1 : 37)) {
    std::vector<char> seen(G, 0);
    for (int b = 0; b < G; ++b) {
      const int l = xcd_remap(b, G);
      ++g_checks;
      if (l < 0 || l >= G || seen[l]) fail(s, "xcd_remap not a permutation", G, b);
      else seen[l] = 1;
    }
  }
  for (int tm = 1; tm <= 20; ++tm)
    for (int tn = 1; tn <= 20; ++tn) {
      std::vector<char> seen(tm * tn, 0);
      for (int t = 0; t < tm * tn; ++t) {
        int r = -1, c = -1;
        tile_coords(t, tm, tn, r, c);
        ++g_checks;
        if (r < 0 || r >= tm || c < 0 || c >= tn || seen[r * tn + c]) fail(s, "tile_coords", t, r);
        else seen[r * tn + c] = 1;
      }
    }
}

// ---- plan invariants ------------------------------------------------------------------
void check_plan(const Shape &s) {
  ++g_checks;
  const int e = prod_choose(s.M, s.N, s.K);
  if (e < 0 || e >= prod_num_configs()) return fail(s, "choice out of range", e, 0);
  for (int dim : {s.M, s.N})
    for (int tile : {64, 128, 192, 256}) {
      const int r = thin_remainder(dim, tile);
      ++g_checks;
      if (r < 0 || r * 8 > tile || (r > 0 && (dim <= tile || dim % tile != r)))
        fail(s, "thin remainder", dim, r);
    }
  const int rr = region_rows(s.M, s.N, s.K);
  ++g_checks;
  if (rr < 0 || (rr > 0 && (256LL * rr >= s.M || s.M - 256LL * rr < 128))) fail(s, "row cut", rr, 0);
  for (int cfg : {-1, 0, 3, 12, 23})
    for (int sp : {0, 1, 2, 7, 64}) {
      SplitPlan p{};
      ++g_checks;
      if (!splitk_plan(s.M, s.N, s.K, cfg, sp, &p)) {
        fail(s, "split plan refused", cfg, sp);
        continue;
      }
      if (p.splits < 1 || p.kc < 1 || (s.K > 0 && (long long)p.splits * p.kc < s.K) ||
          (s.K > 0 && (long long)(p.splits - 1) * p.kc >= s.K))
        fail(s, "split chunks do not cover K once", p.splits, p.kc);
      const long long ws = p.splits > 1 ? (long long)p.splits * s.M * s.N * 4 : 0;
      if (p.workspace_bytes != ws) fail(s, "split workspace", p.workspace_bytes, ws);
      if (!prod_supports(p.config, s.M, s.N, s.K)) fail(s, "split entry refuses", p.config, 0);
    }
}

}  // namespace

int main(int argc, char **argv) {
  bool quick = false;
  for (int i = 1; i < argc; ++i) {
    if (std::strcmp(argv[i], "--quick") == 0) quick = true;
    if (std::strcmp(argv[i], "--plant-unclamped") == 0) g_plant_unclamped = true;
  }
  std::vector<Shape> shapes = {
      {256, 256, 256, 256, 256, 256, "square_256"},
      {1024, 1024, 1024, 1024, 1024, 1024, "square_1024_int"},
      {4096, 4096, 4096, 4096, 4096, 4096, "square_4096"},
      {4097, 4095, 2049, 2049, 4095, 4095, "ragged"},
      {16384, 16384, 64, 64, 16384, 16384, "skinny_k64"},
      {4097, 4095, 2049, 2053, 4099, 4100, "ragged, padded ld"},
      {8192, 8192, 33, 33, 8192, 8192, "K below two steps"},
      {1, 4095, 2049, 2049, 4095, 4095, "one-row strip product"},
      {8, 8191, 4097, 4099, 8193, 8191, "8-row strip product, padded ld"},
      {4, 16384, 1027, 1027, 16384, 16384, "4-row strip product"},
      {2, 17, 2051, 2053, 19, 17, "2-row strip, partial column group"},
      {5, 300, 3, 3, 300, 300, "5-row strip, K below one quad"},
      {4097, 1, 4096, 4096, 1, 1, "one-column product"},
      {4096, 8, 4097, 4099, 9, 11, "8-column product, padded ld"},
      {300, 3, 1023, 1023, 3, 3, "3-column product, K below one chunk"},
      {17, 5, 2049, 2051, 5, 7, "5-column product, partial row group"},
      {9, 2, 1, 1, 2, 2, "2-column product, K = 1"},
  };
  // edge sweep: sizes around multiples of 16 .. 256, and K tails
  const int sizes[] = {1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257,
                       300, 511, 512, 513, 1000, 1025};
  for (int M : sizes)
    for (int N : sizes)
      for (int K : {1, 4, 31, 32, 33, 64, 65, 100, 257})
        if (!quick || (M % 7 == 0 && N % 5 == 0))
          shapes.push_back({M, N, K, K, N, N, "edge"});
  for (int M : {256, 512, 768, 1280})
    for (int N : {128, 256, 1024})
      shapes.push_back({M, N, 64, 64, N, N, "small K"});
  for (const Shape &s : shapes) {
    check_plan(s);
    replay_product(s);
  }
  // every family's guard at its boundary
  boundary_a<8>(256, "256-row A tiles, BK 32");
  boundary_a<8>(192, "192-row A tiles, BK 32");
  boundary_a<8>(128, "128-row A tiles, BK 32");
  boundary_a<16>(256, "256-row A panel, BK 64");
  boundary_a<16>(128, "128-row A tiles, BK 64");
  boundary_a<16>(64, "64-row A tiles, BK 64");
  boundary_b<64>(32, "256-column B steps, BK 32");
  boundary_b<48>(32, "192-column B steps, BK 32");
  boundary_b<32>(32, "128-column B steps, BK 32");
  boundary_b<32>(64, "128-column B steps, BK 64");
  boundary_b<16>(64, "64-column B steps, BK 64");
  check_ksplit_quarters();
  check_mixed16_layouts();
  check_windows();
  check_orders();
  std::printf("replay: %d shapes, %lld checks, %d failures\n", (int)shapes.size(), g_checks,
              g_failures);
  return g_failures == 0 ? 0 : 1;
}
