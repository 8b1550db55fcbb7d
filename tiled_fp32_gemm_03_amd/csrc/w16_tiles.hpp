// Shared pieces of the 16x16-MFMA kernels with direct-to-LDS operand loads
// (gfx950): the W16 tile family, its LDS layouts and fragment readers, the
// inline-assembly direct load and the barrier they use, and the 128x128-wave
// kernel template (big16_kernel), which is instantiated in more than one
// translation unit because its best register form differs with the wave
// tile.  Everything here has internal linkage.
#pragma once

#include "gemm_internal.hpp"
#include "launch_util.hpp"
#include "addr_math.hpp"

#include <atomic>
#include <cstdint>

namespace gemm_f32_impl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kLdsBytes = 160 * 1024;  // LDS of one gfx950 CU

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_void_t;

// Tile t's origin (edge_tile_origin: a tile that would overhang C is moved
// back inside it), and whether the whole tile lies inside C -- only a
// product narrower than one tile keeps guarded edges.
template <class S>
__device__ inline void tile_origin(int t, int tiles_m, int tiles_n, int &m0,
                                   int &n0, bool &interior, const Problem &p) {
  edge_tile_origin(t, tiles_m, tiles_n, S::BM, S::BN, p.M, p.N, m0, n0);
  interior = (m0 + S::BM <= p.M) && (n0 + S::BN <= p.N);
}

// s_waitcnt immediate that waits until at most `n` vector-memory operations
// of this wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt and lgkmcnt left at their "no wait" maxima).
constexpr int vmcnt_wait_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// The direct loads of this kernel are issued from inline assembly, with an
// SGPR base address, a per-lane 32-bit byte offset and the wave's LDS
// destination in M0, so that the compiler does not see them as LDS writes:
// it would otherwise wait for every outstanding one (vmcnt(0)) before each
// later LDS read, which would serialise the pipeline.  The kernel orders
// them itself: explicit vmcnt waits before each barrier, and every LDS read
// of a stage happens after the barrier that follows its loads.  M0 is named
// as clobbered; the compiler warns that it reserves M0 for itself, and in
// the kernels that use this load nothing else sets or reads M0 (the
// generated code touches M0 only in these sequences), so no value of the
// compiler's is lost.  tests/test_m0_guard.py disassembles the built code
// objects and fails if any other instruction in such a kernel writes M0 or
// reads it implicitly.  The s_nop gives the one wait state the hardware
// needs between writing M0 and an LDS DMA that reads it.
__device__ inline void ks_load_to_lds16(unsigned voff, const float *sbase, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

// Waits until this wave's LDS operations have completed (as a builtin, so
// the compiler knows the fragment registers are ready), then the workgroup
// barrier.  Unlike __syncthreads() it does not wait for outstanding
// vector-memory loads, so direct loads of later steps stay in flight; the
// memory clobber keeps the compiler from moving memory accesses across it.
constexpr int kLgkmWait0 = 0xF | (0x3 << 14) | (0x7 << 4);  // lgkmcnt(0) only

__device__ inline void ks_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kLgkmWait0);
  asm volatile("s_barrier" ::: "memory");
}

// ---- one wave per SIMD, 16x16x4 MFMAs, direct-load pipeline -----------
// The large-product form of the K-split kernel's recipe: a BM x BN tile
// (BM = 2 WTM, BN = 2 WTN) over 4 waves, each computing a WTM x WTN sub-tile
// as 16x16 blocks with v_mfma_f32_16x16x4_f32 -- (WTM/16)(WTN/16)
// independent accumulator chains, so a lone wave keeps the matrix pipe busy.
// Operands arrive by direct loads (ks_load_to_lds16)
// into STAGES LDS stages of BK-deep k steps: the loads of step
// i + STAGES - 1 are issued during step i, into the stage that step i - 1
// used.  Inside a step the fragments are read 16 k at a time, one chunk
// ahead of the MFMAs.  Within a 16-deep chunk h, MFMA t takes
// k = 16 h + 4 g + t for lane group g = l / 16.  LDS layouts (16-byte
// chunks): A rows of BK floats, chunk c of row r at c ^ ((r >> 1) & 7) for
// BK = 32 and at c ^ (r & 15) for BK = 64; B rows of BN floats,
// chunk c of k row k at c ^ (4 ((k >> 2) & 3)).  Each element is summed in
// one fp32 accumulator in ascending k steps, but the k order inside a step
// differs from the 32x32-MFMA kernels, so the bits may differ from theirs.
template <int WTM_, int WTN_, int BK_, int STAGES_>
struct W16 {
  static constexpr int WTM = WTM_, WTN = WTN_, BK = BK_, STAGES = STAGES_;
  static constexpr int BM = 2 * WTM, BN = 2 * WTN;
  static constexpr int TBM = WTM / 16, TBN = WTN / 16;
  static constexpr int NQ = BK / 16;      // 16-deep chunks per step
  static constexpr int ACH = BK / 4;      // 16-byte chunks per A row
  static constexpr int ARPI = 64 / ACH;   // A rows per 1 KB instruction
  static constexpr int BCH = BN / 4;      // 16-byte chunks per B row
  // B: instruction q of the step fills LDS chunks 64 q .. 64 q + 63 in k-row
  // order (BCH chunks per row), so it may span parts of several rows.
  static constexpr int A_FLOATS = BM * BK, B_FLOATS = BK * BN, STAGE = A_FLOATS + B_FLOATS;
  static constexpr int A_DMA = A_FLOATS / 256 / 4;  // instructions per wave and step
  static constexpr int B_DMA = B_FLOATS / 256 / 4;
  static constexpr int DMA = A_DMA + B_DMA;
  static_assert(BK == 32 || BK == 64, "A rows of 32 or 64 floats");
  static_assert(BCH % 16 == 0, "B rows of whole 16-chunk groups (the permutation stays in one)");
  static_assert(A_FLOATS % 1024 == 0 && B_FLOATS % 1024 == 0, "whole instructions per wave");
  static_assert(STAGES >= 2 && STAGES * STAGE * 4 <= kLdsBytes, "LDS budget");
};

// LDS chunk layouts (w16_a_pos, w16_b_pos): addr_math.hpp.

// Fragments, per lane (l16 = lane % 16, g = lane / 16): for 16-deep chunk
// h, A[row l16 of block bm][k = 16 h + 4 g .. + 3] as one 16-byte read,
// and for MFMA t of the chunk B[k = 16 h + 4 g + t][column l16 of block bn].
template <class W>
__device__ inline void w16_read_a(f32x4 (&a)[W::TBM], const float *st, int h, int lane, int wm) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int bm = 0; bm < W::TBM; ++bm)
    a[bm] = *reinterpret_cast<const f32x4 *>(
        st + 4 * w16_a_pos<W::ACH>(wm * W::WTM + 16 * bm + l16, 4 * h + g));
}

template <class W>
__device__ inline void w16_read_b(float (&b)[W::TBN], const float *st, int h, int t, int lane,
                                  int wn) {
  const int l16 = lane & 15, g = lane >> 4;
  const int k = 16 * h + 4 * g + t;
#pragma unroll
  for (int bn = 0; bn < W::TBN; ++bn) {
    const int n = wn * W::WTN + 16 * bn + l16;
    b[bn] = st[W::A_FLOATS + 4 * w16_b_pos<W::BCH>(k, n >> 2) + (n & 3)];
  }
}

// MFMA t of a chunk over all blocks of the wave tile, from separately held
// A (chunk) and B (MFMA t) fragments.
// One v_mfma_f32_16x16x4_f32 accumulating in place (FIRST: from 0, so a
// tile needs no zeroed accumulators), for the A-resident kernel, the
// whole-step K-split kernel and the tail forms of the 128x128-wave kernel.
// Issued as inline assembly with the
// accumulator tied to the destination: with the builtin, the register
// allocator renamed destinations away from their sources and copied the
// accumulators back inside the MFMA stream (about 600 accumulator moves per
// two tiles of the A-resident kernel: measured 294 -> 288 us on 16384 x
// 16384 x 64).  The compiler does not see these as MFMAs, so it inserts no
// wait states after them: the callers take their sources straight from LDS
// reads (waited for by lgkmcnt, which the compiler does track), keep each
// chain's next MFMA 16 or more MFMAs later, and issue 24 wait states after
// the stream before anything reads a result.
template <bool FIRST>
__device__ __forceinline__ void mfma_inplace(f32x4 &acc, float b, float a) {
  if constexpr (FIRST)
    asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, 0" : "=a"(acc) : "v"(b), "v"(a));
  else
    asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
}

template <class W, bool IN_PLACE = false>
__device__ inline void w16_mfma_t(f32x4 (&acc)[W::TBM][W::TBN], const f32x4 (&a)[W::TBM],
                                  const float (&b)[W::TBN], int t) {
#pragma unroll
  for (int bm = 0; bm < W::TBM; ++bm)
#pragma unroll
    for (int bn = 0; bn < W::TBN; ++bn)
      if constexpr (IN_PLACE)
        mfma_inplace<false>(acc[bm][bn], b[bn], a[bm][t]);
      else
        acc[bm][bn] = __builtin_amdgcn_mfma_f32_16x16x4f32(b[bn], a[bm][t], acc[bm][bn], 0, 0, 0);
}

// Guarded fill of one stage for the partial k step of a tile (k0 < K <
// k0 + BK), in the direct-load layout, by all 256 threads: A is read as
// 4-float windows (an A chunk that straddles K is the window ending at K,
// shifted into place; chunks past K are zero), B rows at or past K are
// zero, and every load stays inside the matrices (rows need 4-byte
// alignment, K >= 4).  The tile lies inside C.  Elements past K enter the
// MFMAs as exact zeros, so the per-element k order is that of a full step.
// Element e of the result is w[e + shift] for e < valid, else 0 (shift <=
// 3, valid <= 4 - shift).  The shift runs as two stages of selects (by 2,
// then by 1): an index select per element compiles to branches on the
// per-lane shift, which made the fill several times slower.
__device__ inline f32x4 w16_place_window(const f32x4 &w, int valid, int shift) {
  const bool s2 = (shift & 2) != 0, s1 = (shift & 1) != 0;
  const float a0 = s2 ? w[2] : w[0], a1 = s2 ? w[3] : w[1];
  const float a2 = s2 ? 0.f : w[2], a3 = s2 ? 0.f : w[3];
  const float b0 = s1 ? a1 : a0, b1 = s1 ? a2 : a1, b2 = s1 ? a3 : a2, b3 = s1 ? 0.f : a3;
  return f32x4{valid > 0 ? b0 : 0.f, valid > 1 ? b1 : 0.f, valid > 2 ? b2 : 0.f,
               valid > 3 ? b3 : 0.f};
}

template <class W>
__device__ inline void w16_fill_partial(float *st, const Problem &p, int m0, int n0, int k0,
                                        int tid) {
  constexpr int A_ROWS = 256 / W::ACH, B_ROWS = 256 / W::BCH;  // rows per pass of 256 threads
  constexpr int A_CHUNKS = W::BM / A_ROWS, B_CHUNKS = W::BK / B_ROWS;
  static_assert(W::BM % A_ROWS == 0 && W::BK % B_ROWS == 0, "whole passes");
  const int arow = tid / W::ACH, ac = tid % W::ACH;
  const int bkr = tid / W::BCH, bc = tid % W::BCH;
  int valid = 0, shift = 0;
  const int col = tail_window(k0 + 4 * ac, p.K, valid, shift);
  f32x4 ra[A_CHUNKS], rb[B_CHUNKS];
  const float *as = p.A + (long long)(m0 + arow) * p.lda + col;
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i)
    ra[i] = *reinterpret_cast<const f32x4u *>(as + (long long)i * A_ROWS * p.lda);
  int b_ok = 0;
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    const int k = k0 + bkr + i * B_ROWS;
    const bool ok = k < p.K;
    b_ok |= (int)ok << i;
    rb[i] = *reinterpret_cast<const f32x4u *>(p.B + (long long)(ok ? k : p.K - 1) * p.ldb + n0 +
                                              4 * bc);
  }
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i)
    *reinterpret_cast<f32x4 *>(st + 4 * w16_a_pos<W::ACH>(arow + i * A_ROWS, ac)) =
        w16_place_window(ra[i], valid, shift);
  const f32x4 z{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i)
    *reinterpret_cast<f32x4 *>(st + W::A_FLOATS + 4 * w16_b_pos<W::BCH>(bkr + i * B_ROWS, bc)) =
        (b_ok >> i) & 1 ? rb[i] : z;
}

// Workgroups of a kernel resident on the whole device at once (cached per
// kernel and device; computed on first use).
constexpr int kMaxDevices = 64;

template <auto KERNEL, int NT>
int resident_workgroups() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERNEL, NT, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) !=
          hipSuccess ||
      cus < 1)
    cus = 1;
  const int total = per_cu * cus;
  if (dev >= 0) cache[dev].store(total, std::memory_order_relaxed);
  return total;
}

// ---- one wave per SIMD, 128x128 wave tiles -----------------------------
// For large products whose K is a whole number of k steps: a 256x256 tile
// over 4 waves (2 x 2), each computing a 128x128 sub-tile as 8 x 8 blocks
// of v_mfma_f32_16x16x4_f32.  The 64 accumulator chains (256 registers per
// lane) live in the accumulation registers; per 32-deep k step a wave
// issues 512 MFMAs (16384 matrix-pipe cycles) against 16 direct loads,
// 16 A and 64 B fragment reads and one barrier, so the non-matrix work of
// a step is small and one barrier per step is cheap among 4 waves.  Two
// LDS stages: the loads of step i + 1 are issued during step i, into the
// stage step i - 1 used.  The k loop has no branch: the stage alternates
// by parity, the step after a tile's last is the next tile's first, and
// the workgroup's very last step reloads its own tile's first operands
// into the idle stage.  LDS layouts and the per-element k order are those
// of w16_kernel.
//
// With TAIL, K is not a multiple of the k step (K > BK): each tile's last
// step is partial.  The step before it issues its direct loads as usual but
// from the last whole step inside the matrices (A columns and B rows
// [K - BK, K)), so the MFMA stream is the plain kernel's; after its MFMAs
// each wave waits for its loads, a barrier, and then every thread rewrites
// the whole idle stage through registers with the partial step zero-filled
// (w16_fill_partial) -- once per tile, outside the MFMA stream -- and the
// top-of-step barrier publishes it.  Direct loads need only 4-byte aligned
// rows (checked on gfx950: a 16-byte direct load from a dword-aligned
// address delivers the 16 bytes at that address, at the same speed).
//
// The body is shared by the plain kernel and the split-K kernel (which runs
// it on one chunk of K per grid row); `bid` of `G` is the workgroup's place
// in the persistent grid.
template <class W, int VQ = 0>
__device__ __forceinline__ void big16_body(Problem p, int tiles_m, int tiles_n, int bid, int G) {
  static_assert(W::STAGES == 2, "two stages");
  // VQ = 0: K is a whole number of steps.  VQ = 1, 2 or 4: the partial
  // last step of each tile runs only its first VQ MFMA groups (group 4 h + u
  // takes k = 16 h + u + {0, 4, 8, 12} of the step; the launcher picks VQ so
  // that every group holding a k below K runs), inside the step before it.
  // VQ = BK / 4: the partial step runs the pinned loop.
  constexpr bool TAIL = VQ > 0;
  constexpr bool PEEL = TAIL && VQ < W::BK / 4;
  // The tail forms' MFMAs accumulate in place (mfma_inplace): with the
  // builtin, the register allocator copied one accumulator block out and
  // back every step of their loop (24 moves; measured 2 us of the 4096 x
  // 4096 x 2049 product).  The plain form keeps the builtin, which is
  // faster there (930 against 935 us on 4096^3).  The accumulators are
  // zeroed ahead of the k loop, whose first MFMA follows a wait, a barrier
  // and the fragment reads (37 instructions or more in the built code), so
  // the zeroing needs no wait states of its own.
  constexpr bool kInPlace = TAIL && W::TBM * W::TBN * 4 == 256;
  static_assert(VQ == 0 || VQ == 1 || VQ == 2 || VQ == 4 || VQ == W::BK / 4, "k quads");
  __shared__ __attribute__((aligned(16))) float lds[2 * W::STAGE];
  const unsigned lds_u = (unsigned)(uintptr_t)(lds_void_t *)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int ntiles = tiles_m * tiles_n;
  const int nk = (p.K + W::BK - 1) / W::BK;
  const int nk_full = PEEL ? nk - 1 : nk;  // steps of the pinned loop
  const int lid = xcd_remap(bid, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int my_tiles = (ntiles - lid + G - 1) / G;

  // Per-lane byte offsets of this wave's direct loads from a step's base
  // addresses (chunks permuted as in the LDS layouts).
  unsigned voff[W::DMA];
#pragma unroll
  for (int q = 0; q < W::A_DMA; ++q)
    voff[q] = (unsigned)(dma_a_elem<W::ACH>(wave * W::A_DMA + q, lane, p.lda) * 4);
#pragma unroll
  for (int q = 0; q < W::B_DMA; ++q)
    voff[W::A_DMA + q] = (unsigned)(dma_b_elem<W::BCH>(64 * (wave * W::B_DMA + q) + lane, p.ldb) * 4);
  const unsigned wave_a = (unsigned)(wave * W::A_DMA * 1024);
  const unsigned wave_b = (unsigned)(W::A_FLOATS * 4 + wave * W::B_DMA * 1024);
  const long long b_step = (long long)W::BK * p.ldb;
  // From the step before a partial one to the last whole step inside the
  // matrices, which starts at column (A) or row (B) K - BK.
  const long long a_inc_tail = p.K - (long long)(nk - 1) * W::BK;
  const long long b_inc_tail = a_inc_tail * p.ldb;

  auto tile_base = [&](int t, const float *&ab, const float *&bb) __attribute__((always_inline)) {
    int m0, n0;
    bool interior;
    tile_origin<W>(lid + t * G, tiles_m, tiles_n, m0, n0, interior, p);
    ab = p.A + (long long)m0 * p.lda;
    bb = p.B + n0;
  };
  auto tile_m0n0 = [&](int t, int &m0, int &n0) __attribute__((always_inline)) {
    bool interior;
    tile_origin<W>(lid + t * G, tiles_m, tiles_n, m0, n0, interior, p);
  };
  auto issue = [&](unsigned st, const float *ab, const float *bb, int q0, int q1)
      __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < W::DMA; ++q) {
      if (q < q0 || q >= q1) continue;
      if (q < W::A_DMA)
        ks_load_to_lds16(voff[q], ab, st + wave_a + q * 1024);
      else
        ks_load_to_lds16(voff[q], bb, st + wave_b + (q - W::A_DMA) * 1024);
    }
  };

  const float *is_a, *is_b;  // operands of the step most recently issued
  tile_base(0, is_a, is_b);
  issue(lds_u, is_a, is_b, 0, W::DMA);
  int stage = 0;

  f32x4 acc[W::TBM][W::TBN];
  for (int t = 0; t < my_tiles; ++t) {
    const float *nt_a, *nt_b;  // the next tile's first step (this tile's on the last)
    tile_base(t + 1 < my_tiles ? t + 1 : t, nt_a, nt_b);
#pragma unroll
    for (int i = 0; i < W::TBM; ++i)
#pragma unroll
      for (int j = 0; j < W::TBN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kk = 0; kk < nk_full; ++kk) {
      const bool last = !PEEL && kk + 1 == nk;     // a peeled partial step is the last
      const bool pre_tail = TAIL && kk + 2 == nk;  // the next step is the partial one
      // Step kk + 1's operands; before a partial step, the last whole step
      // inside the matrices (A columns and B rows [K - BK, K)), which the
      // fill below replaces.  Only a select per step: the increments are
      // fixed per product.
      const float *ia = last ? nt_a : is_a + (pre_tail ? a_inc_tail : (long long)W::BK);
      const float *ib = last ? nt_b : is_b + (pre_tail ? b_inc_tail : b_step);
      __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));  // this step's loads (own)
      ks_lds_barrier();                                // everyone's; stage stage^1 free
      const float *st = lds + stage * W::STAGE;
      const unsigned nst = lds_u + (stage ^ 1) * W::STAGE * 4;

      // Fragments: A one chunk ahead, B one MFMA group ahead.  After the
      // barrier, group 0's operands are read in the order its MFMAs use
      // them (B, then A row block by row block), so the first MFMAs wait
      // for two reads rather than for the whole group's.  Inside a group,
      // the next group's reads are issued after its first half, and the
      // next step's 16 direct loads one after every other row of 8 MFMAs
      // over the first two groups.  sched_barrier pins these positions.
      f32x4 a0[W::TBM], a1[W::TBM];
      float b0[W::TBN], b1[W::TBN];
      w16_read_b<W>(b0, st, 0, 0, lane, wn);
      __builtin_amdgcn_sched_barrier(0);
      {
        const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
        for (int bm = 0; bm < W::TBM; ++bm) {
          a0[bm] = *reinterpret_cast<const f32x4 *>(
              st + 4 * w16_a_pos<W::ACH>(wm * W::WTM + 16 * bm + l16, g));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int h = 0; h < W::NQ; ++h) {
        f32x4(&ac)[W::TBM] = (h & 1) ? a1 : a0;
        f32x4(&an)[W::TBM] = (h & 1) ? a0 : a1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int grp = 4 * h + u;
          float(&bc)[W::TBN] = (grp & 1) ? b1 : b0;
          float(&bnx)[W::TBN] = (grp & 1) ? b0 : b1;
#pragma unroll
          for (int bm = 0; bm < W::TBM; ++bm) {
#pragma unroll
            for (int bn = 0; bn < W::TBN; ++bn)
              if constexpr (kInPlace)
                mfma_inplace<false>(acc[bm][bn], bc[bn], ac[bm][u]);
              else
                acc[bm][bn] =
                    __builtin_amdgcn_mfma_f32_16x16x4f32(bc[bn], ac[bm][u], acc[bm][bn], 0, 0, 0);
            constexpr int kRowsPerLoad = 2;
            const int row = grp * W::TBM + bm;
            if (row % kRowsPerLoad == 0 && row / kRowsPerLoad < W::DMA) {
              __builtin_amdgcn_sched_barrier(0);
              issue(nst, ia, ib, row / kRowsPerLoad, row / kRowsPerLoad + 1);
              __builtin_amdgcn_sched_barrier(0);
            }
            if (bm == W::TBM / 2 - 1) {
              __builtin_amdgcn_sched_barrier(0);
              if (u < 3)
                w16_read_b<W>(bnx, st, h, u + 1, lane, wn);
              else if (h + 1 < W::NQ)
                w16_read_b<W>(bnx, st, h + 1, 0, lane, wn);
              if (u == 1 && h + 1 < W::NQ) w16_read_a<W>(an, st, h + 1, lane, wm);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      if constexpr (TAIL) {
        if (pre_tail) {  // every wave's loads into the idle stage landed; rewrite it
          __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));
          ks_lds_barrier();
          int m0, n0;
          tile_m0n0(t, m0, n0);
          w16_fill_partial<W>(lds + (stage ^ 1) * W::STAGE, p, m0, n0, (nk - 1) * W::BK, tid);
          if constexpr (PEEL) {
            // The partial step itself, here: the next tile's first loads
            // go into the stage this step just read (every wave is past
            // the barrier above, so done with it) -- none after the last
            // tile, where nothing reads them and the final wait would sit
            // on their latency (7 us of the 4096 x 4096 x 2049 product);
            // then only the first VQ MFMA groups (the others hold no k
            // below K and would add exact zeros), with fragments read as
            // they go.
            ks_lds_barrier();  // the fill is everyone's
            const float *pst = lds + (stage ^ 1) * W::STAGE;
            if (t + 1 < my_tiles) issue(lds_u + stage * W::STAGE * 4, nt_a, nt_b, 0, W::DMA);
            f32x4 a[W::TBM];
            float b[W::TBN];
#pragma unroll
            for (int grp = 0; grp < VQ; ++grp) {
              if (grp % 4 == 0) w16_read_a<W>(a, pst, grp / 4, lane, wm);
              w16_read_b<W>(b, pst, grp / 4, grp % 4, lane, wn);
              w16_mfma_t<W, kInPlace>(acc, a, b, grp % 4);
            }
            ia = nt_a;    // the operands most recently issued
            ib = nt_b;
            stage ^= 1;   // with the flip below: the next tile reads `stage`
          }
        }
      }
      is_a = ia;
      is_b = ib;
      stage ^= 1;
      // With 256 accumulators per lane, hand every one to the next step in
      // an accumulation register (an empty asm with an "a" operand):
      // without it the register allocator keeps part of them in ordinary
      // VGPRs across the loop and copies them to and from the accumulation
      // registers around the MFMAs every step.  (Smaller wave tiles are
      // built with the MFMAs' VGPR form, where no such copies arise.)
      if constexpr (W::TBM * W::TBN * 4 == 256) {
#pragma unroll
        for (int i = 0; i < W::TBM; ++i)
#pragma unroll
          for (int j = 0; j < W::TBN; ++j) asm volatile("" : "+a"(acc[i][j]));
      }
    }
    if constexpr (kInPlace) {
      // 24 wait states after the last MFMA before its results are read
      // (mfma_inplace).
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
      __builtin_amdgcn_sched_barrier(0);
    }
    int m0, n0;
    bool interior;
    tile_origin<W>(lid + t * G, tiles_m, tiles_n, m0, n0, interior, p);
    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int bm = 0; bm < W::TBM; ++bm) {
      float *crow = p.C + (long long)(m0 + wm * W::WTM + 16 * bm + l16) * p.ldc + n0 +
                    wn * W::WTN + 4 * g;
#pragma unroll
      for (int bn = 0; bn < W::TBN; ++bn)
        *reinterpret_cast<f32x4u *>(crow + 16 * bn) = acc[bm][bn];
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));  // the redundant last reload
}

template <class W, int VQ = 0>
__global__ void __launch_bounds__(256) big16_kernel(Problem p, int tiles_m, int tiles_n) {
  big16_body<W, VQ>(p, tiles_m, tiles_n, blockIdx.x, gridDim.x);
}

// Split-K: grid row y computes the partial product over k in
// [y * kc, min(K, (y + 1) * kc)) into its own M x N slab of `ws` (row pitch
// N), one tile per workgroup; the caller sums the slabs.  kc and K are
// multiples of the k step.
template <class W>
__global__ void __launch_bounds__(256)
    big16_split_kernel(Problem p, int tiles_m, int tiles_n, int kc, float *ws) {
  const int y = blockIdx.y;
  const int k0 = y * kc;
  Problem ps = p;
  ps.A = p.A + k0;
  ps.B = p.B + (long long)k0 * p.ldb;
  ps.K = p.K - k0 < kc ? p.K - k0 : kc;
  ps.C = ws + (long long)y * p.M * p.N;
  ps.ldc = p.N;
  big16_body<W>(ps, tiles_m, tiles_n, blockIdx.x, gridDim.x);
}

template <class W, auto KERNEL>
hipError_t launch_big16_grid(const Problem &p, hipStream_t s) {
  const long long tiles_m = ceil_div(p.M, W::BM), tiles_n = ceil_div(p.N, W::BN);
  const long long ntiles = tiles_m * tiles_n;
  if (ntiles > 0x7fffffffLL) return hipErrorInvalidValue;
  long long grid = resident_workgroups<KERNEL, 256>();
  if (grid > ntiles) grid = ntiles;
  return launch_kernel(KERNEL, dim3((unsigned)grid), dim3(256), s, p, (int)tiles_m, (int)tiles_n);
}

}  // namespace
}  // namespace gemm_f32_impl
