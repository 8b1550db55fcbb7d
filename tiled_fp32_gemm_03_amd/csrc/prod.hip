// Rung 3 of the kernel ladder: the production fp32 kernel for gfx950.
//
// It keeps the pages' structure -- one workgroup owns one C tile, A and B
// tiles are staged on chip once per k step and re-used there, the running
// sums live in registers (geek-doc.cn "矩阵乘法 tiling", sections 二-四;
// mayulu.co "CUDA 编程系列之三", section 6) -- and takes the further steps the
// pages only name: one thread owns many outputs and the tiling becomes a
// pyramid of register, wave and instruction blocks (geek-doc.cn sections 三
// and 五).  On CDNA4 the instruction block is the fp32 matrix-core op
// v_mfma_f32_32x32x2_f32.
//
// Per workgroup: BM x BN tiles of C, WGM x WGN waves, each wave a
// (BM/WGM) x (BN/WGN) sub-tile made of 32 x 32 MFMA blocks whose
// accumulators stay in registers for the whole k loop of a tile.
//
// Data path per k step (depth BK):
//   global -> registers: the next step's A and B tiles as 128-bit loads,
//     consecutive lanes on consecutive addresses.  Rows only need 4-byte
//     alignment (CDNA accepts dword-aligned multi-dword accesses), so odd
//     leading dimensions take the same path;
//   registers -> LDS: into the stage not being read (two stages), rows padded
//     so that the fragment reads below do not collide in LDS banks;
//   LDS -> MFMA: per 8-deep k group a lane reads one 128-bit A fragment per
//     32-row block and four B scalars per 32-column block.
//   One barrier per k step suffices with two stages: a stage is rewritten
//   only after the barrier that follows its last read.  (The pages' single
//   buffer needs its two barriers per step; the two-stage form here is a
//   departure from them.)
//
// Persistent schedule.  The grid holds at most as many workgroups as fit on
// the chip at once; each walks its tiles' k steps as one flat sequence, so
// the loads of the next tile's first step are in flight while the current
// tile finishes, and its C stores drain while the next tile computes.
//
// Operand roles.  An MFMA lane supplies one element of each operand: lane l
// gives row l%32 of the first operand and column l%32 of the second at k
// slot l/32, and holds output rows 8q + 4(l/32) + r, column l%32 (q, r in
// 0..3).  The kernel feeds B as the first operand and A as the second, so
// each MFMA block computes a transposed 32 x 32 block of C; then every lane
// holds four runs of four consecutive columns of one C row, stored with
// 128-bit writes.  The k order inside an 8-deep group is permuted (lane half
// h, step s takes k = 4h + s) so that both operands read 4 consecutive k per
// lane; a sum's value does not depend on which k is added in which step
// except through fp32 rounding.
//
// Edges.  Steps and tiles that overhang K, M or N use guarded loads that
// write 0 for elements outside the matrices (geek-doc.cn section 六; mayulu.co
// section 7), per element where a 4-wide chunk straddles an edge, and
// guarded stores that leave C outside M x N untouched.  Interior steps take
// unguarded loads.
//
// Workgroup order.  Workgroups are dealt to the 8 XCDs round robin by
// launch index; the index is remapped so that each XCD receives a contiguous
// run of tiles, and runs are laid out in groups of 8 tile rows so that the
// tiles sharing an XCD's L2 also share A rows and B columns.
#include "gemm_internal.hpp"
#include "launch_util.hpp"
#include "addr_math.hpp"
#include "w16_tiles.hpp"

#include <atomic>
#include <cstdint>
#include <type_traits>

namespace gemm_f32_impl {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPadA = 4;  // floats after each LDS row of A (k-contiguous rows)
constexpr int kPadB = 8;  // floats after each LDS row of B (n-contiguous rows)

template <int BM_, int BN_, int BK_, int WGM_, int WGN_, bool NT_STORE_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
  static constexpr bool NT_STORE = NT_STORE_;
  static constexpr int NT = 64 * WGM * WGN;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave sub-tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;    // MFMA blocks per wave
  static constexpr int SA = BK + kPadA;                  // LDS row stride of A
  static constexpr int SB = BN + kPadB;                  // LDS row stride of B
  static constexpr int A_STAGE = BM * SA;
  static constexpr int B_STAGE = BK * SB;
  static constexpr int LDS_FLOATS = 2 * (A_STAGE + B_STAGE);
  static constexpr int A_CHUNKS = BM * BK / 4 / NT;  // 4-float chunks per thread
  static constexpr int B_CHUNKS = BK * BN / 4 / NT;
  static constexpr int A_ROWS_PER_PASS = NT / (BK / 4);
  static constexpr int B_ROWS_PER_PASS = NT / (BN / 4);

  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
  static_assert(BK % 8 == 0, "BK must be a multiple of 8");
  static_assert(NT % (BK / 4) == 0 && NT % (BN / 4) == 0, "staging map");
  static_assert((BM * BK) % (4 * NT) == 0 && (BK * BN) % (4 * NT) == 0,
                "tile must split evenly over threads");
};


// Register staging map of a W16 tile (the K-tail and narrow-product path
// of the 16x16-MFMA kernels).
template <class W>
using W16Staging = Tile<W::BM, W::BN, W::BK, 2, 2, false>;

template <class S>
struct Stage {
  // registers holding one k step of A and B on their way to LDS, and per
  // chunk how to place the loaded 4-float window: (valid << 2) | shift --
  // element e of the chunk is window[e + shift] if e < valid, else 0.
  f32x4 a[S::A_CHUNKS];
  f32x4 b[S::B_CHUNKS];
  int ameta[S::A_CHUNKS];
  int bmeta[S::B_CHUNKS];
};

constexpr int kMetaFull = 4 << 2;  // four valid elements, no shift

__device__ inline f32x4 load4(const float *src) {
  return *reinterpret_cast<const f32x4u *>(src);
}

// Branch-free guarded chunk load.  Every lane issues one 128-bit load at an
// address that is always inside the matrix: a chunk wholly inside its row is
// loaded in place; one that straddles the row end loads the 4-float window
// ending at the row end (so no byte past the row is touched) and records the
// shift; a chunk outside the matrix loads from the matrix origin and is
// marked empty.  The zeroing happens when the stage is written to LDS, after
// the data has arrived, so no lane's path waits on another's load.
// Needs row length >= 4 (the caller takes the per-element path otherwise).
__device__ inline f32x4 load_chunk_guarded(const float *base, long long ld,
                                           int row, int rows, int col,
                                           int cols, int &meta) {
  return load4(base + guarded_window(row, rows, col, cols, ld, meta));
}

// Four elements src[0..3] with those at index >= valid read as 0 (per
// element; used only for rows shorter than 4 elements).
__device__ inline f32x4 load_partial(const float *src, int valid) {
  f32x4 v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (e < valid) v[e] = src[e];
  return v;
}

// Place a loaded window according to its meta code (see Stage): element e
// is w[e + shift] for e < valid, else 0 -- the w16 fill's branch-free select
// network (an index select per element compiles to branches on the per-lane
// shift).
__device__ inline f32x4 place(const f32x4 &w, int meta) {
  return w16_place_window(w, meta >> 2, meta & 3);
}

template <class S, bool GUARD, bool DO_A = true, bool DO_B = true>
__device__ inline void load_global(Stage<S> &st, const Problem &p, int m0,
                                   int n0, int k0, int tid) {
  const int arow = tid / (S::BK / 4), akq = (tid % (S::BK / 4)) * 4;
  const int bkr = tid / (S::BN / 4), bnq = (tid % (S::BN / 4)) * 4;
  if (!GUARD) {
#pragma unroll
    for (int i = 0; i < (DO_A ? S::A_CHUNKS : 0); ++i) {
      const int gm = m0 + arow + i * S::A_ROWS_PER_PASS;
      st.a[i] = load4(p.A + (long long)gm * p.lda + k0 + akq);
      st.ameta[i] = kMetaFull;
    }
#pragma unroll
    for (int i = 0; i < (DO_B ? S::B_CHUNKS : 0); ++i) {
      const int gk = k0 + bkr + i * S::B_ROWS_PER_PASS;
      st.b[i] = load4(p.B + (long long)gk * p.ldb + n0 + bnq);
      st.bmeta[i] = kMetaFull;
    }
  } else if (p.K >= 4 && p.N >= 4) {
#pragma unroll
    for (int i = 0; i < (DO_A ? S::A_CHUNKS : 0); ++i)
      st.a[i] = load_chunk_guarded(p.A, p.lda, m0 + arow + i * S::A_ROWS_PER_PASS, p.M,
                                   k0 + akq, p.K, st.ameta[i]);
#pragma unroll
    for (int i = 0; i < (DO_B ? S::B_CHUNKS : 0); ++i)
      st.b[i] = load_chunk_guarded(p.B, p.ldb, k0 + bkr + i * S::B_ROWS_PER_PASS, p.K,
                                   n0 + bnq, p.N, st.bmeta[i]);
  } else {
    // rows shorter than one chunk: per-element loads (tiny problems only)
#pragma unroll
    for (int i = 0; i < (DO_A ? S::A_CHUNKS : 0); ++i) {
      const int gm = m0 + arow + i * S::A_ROWS_PER_PASS;
      const int gk = k0 + akq;
      st.a[i] = load_partial(p.A + (long long)gm * p.lda + gk, gm < p.M ? p.K - gk : 0);
      st.ameta[i] = kMetaFull;
    }
#pragma unroll
    for (int i = 0; i < (DO_B ? S::B_CHUNKS : 0); ++i) {
      const int gk = k0 + bkr + i * S::B_ROWS_PER_PASS;
      const int gn = n0 + bnq;
      st.b[i] = load_partial(p.B + (long long)gk * p.ldb + gn, gk < p.K ? p.N - gn : 0);
      st.bmeta[i] = kMetaFull;
    }
  }
}

// Write one staged k step to LDS.  PLACED: the stage came from guarded loads
// and each chunk is placed by its meta code; otherwise it is stored as is.
template <class S, bool PLACED, bool DO_A = true, bool DO_B = true>
__device__ inline void store_lds_as(const Stage<S> &st, float *as, float *bs,
                                    int tid) {
  const int arow = tid / (S::BK / 4), akq = (tid % (S::BK / 4)) * 4;
#pragma unroll
  for (int i = 0; i < (DO_A ? S::A_CHUNKS : 0); ++i)
    *reinterpret_cast<f32x4 *>(as + (arow + i * S::A_ROWS_PER_PASS) * S::SA + akq) =
        PLACED ? place(st.a[i], st.ameta[i]) : st.a[i];
  const int bkr = tid / (S::BN / 4), bnq = (tid % (S::BN / 4)) * 4;
#pragma unroll
  for (int i = 0; i < (DO_B ? S::B_CHUNKS : 0); ++i)
    *reinterpret_cast<f32x4 *>(bs + (bkr + i * S::B_ROWS_PER_PASS) * S::SB + bnq) =
        PLACED ? place(st.b[i], st.bmeta[i]) : st.b[i];
}

template <class S>
__device__ inline void store_lds(const Stage<S> &st, float *as, float *bs,
                                 int tid, bool guarded) {
  if (guarded)
    store_lds_as<S, true>(st, as, bs, tid);
  else
    store_lds_as<S, false>(st, as, bs, tid);
}

// All MFMAs of one k step out of one LDS stage.
// k groups [KG0, KG1) of one stage (8 k values per group).
template <class S, int KG0 = 0, int KG1 = S::BK / 8>
__device__ inline void compute_stage(f32x16 (&acc)[S::TM][S::TN],
                                     const float *as, const float *bs,
                                     int wm, int wn, int lane) {
  const int l32 = lane & 31, h = lane >> 5;
  const float *a_base = as + (wm * S::WTM + l32) * S::SA + 4 * h;
  const float *b_base = bs + (4 * h) * S::SB + wn * S::WTN + l32;
#pragma unroll
  for (int kg = KG0; kg < KG1; ++kg) {
    f32x4 af[S::TM];
    float bf[S::TN][4];
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
      af[tm] = *reinterpret_cast<const f32x4 *>(a_base + tm * 32 * S::SA + kg * 8);
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        bf[tn][s] = b_base[(kg * 8 + s) * S::SB + tn * 32];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(
              bf[tn][s], af[tm][s], acc[tm][tn], 0, 0, 0);
  }
}

template <bool NT>
__device__ inline void store4(float *dst, const f32x4 &v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4u *>(dst));
  else
    *reinterpret_cast<f32x4u *>(dst) = v;
}

template <class S>
__device__ inline void store_c(const f32x16 (&acc)[S::TM][S::TN],
                               const Problem &p, int m0, int n0, int wm,
                               int wn, int lane, bool guard) {
  const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int tm = 0; tm < S::TM; ++tm) {
    const int row = m0 + wm * S::WTM + tm * 32 + l32;
    float *crow = p.C + (long long)row * p.ldc;
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * S::WTN + tn * 32 + 8 * q + 4 * h;
        const f32x4 v{acc[tm][tn][4 * q + 0], acc[tm][tn][4 * q + 1],
                      acc[tm][tn][4 * q + 2], acc[tm][tn][4 * q + 3]};
        if (!guard || (row < p.M && col + 4 <= p.N)) {
          store4<S::NT_STORE>(crow + col, v);
        } else if (row < p.M) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (col + r < p.N) crow[col + r] = v[r];
        }
      }
    }
  }
}

// Load one k step; returns whether the guarded path was taken (uniform).
template <class S>
__device__ inline bool load_step(Stage<S> &st, const Problem &p, int m0,
                                 int n0, int k0, bool interior, int tid) {
  if (interior && k0 + S::BK <= p.K) {
    load_global<S, false>(st, p, m0, n0, k0, tid);
    return false;
  }
  load_global<S, true>(st, p, m0, n0, k0, tid);
  return true;
}

// The persistent tile loop of one product: workgroup `bid` of `G` walks
// tiles bid, bid + G, ... (after the XCD renumbering), each over all of p.K.
template <class S>
__device__ __forceinline__ void prod_body(Problem p, int tiles_m, int tiles_n, int bid, int G) {
  static_assert(S::LDS_FLOATS * 4 <= kLdsBytes, "two stages must fit in LDS");
  __shared__ __attribute__((aligned(16))) float lds[S::LDS_FLOATS];
  float *const as0 = lds;
  float *const bs0 = lds + 2 * S::A_STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int ntiles = tiles_m * tiles_n;
  const int nk = (p.K + S::BK - 1) / S::BK;
  const int lid = xcd_remap(bid, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  // This workgroup's tiles are lid, lid + G, lid + 2G, ...
  const int my_tiles = (ntiles - lid + G - 1) / G;
  const long long steps = (long long)my_tiles * nk;

  int t = lid, kt = 0;
  int m0, n0;
  bool interior;
  tile_origin<S>(t, tiles_m, tiles_n, m0, n0, interior, p);

  f32x16 acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Stage<S> st;
  bool guarded = load_step<S>(st, p, m0, n0, 0, interior, tid);
  store_lds<S>(st, as0, bs0, tid, guarded);
  __syncthreads();

  for (long long it = 0; it < steps; ++it) {
    const int cur = (int)(it & 1);
    const bool more = it + 1 < steps;
    // Coordinates of the next step in this workgroup's flat sequence.
    int nt = t, nkt = kt + 1;
    int nm0 = m0, nn0 = n0;
    bool ninterior = interior;
    if (nkt == nk) {
      nkt = 0;
      nt = t + G;
      if (more) tile_origin<S>(nt, tiles_m, tiles_n, nm0, nn0, ninterior, p);
    }
    if (more) guarded = load_step<S>(st, p, nm0, nn0, nkt * S::BK, ninterior, tid);

    // First half of this step's matrix work, then the next stage's LDS
    // write (that buffer was last read before the previous barrier), then
    // the second half: the write leaves the barrier's critical path.
    compute_stage<S, 0, S::BK / 16>(acc, as0 + cur * S::A_STAGE, bs0 + cur * S::B_STAGE, wm,
                                    wn, lane);
    if (more)
      store_lds<S>(st, as0 + (cur ^ 1) * S::A_STAGE,
                   bs0 + (cur ^ 1) * S::B_STAGE, tid, guarded);
    compute_stage<S, S::BK / 16, S::BK / 8>(acc, as0 + cur * S::A_STAGE,
                                            bs0 + cur * S::B_STAGE, wm, wn, lane);

    if (kt == nk - 1) {
      // Tile done: stores drain while the next tile computes.
      store_c<S>(acc, p, m0, n0, wm, wn, lane, !interior);
#pragma unroll
      for (int i = 0; i < S::TM; ++i)
#pragma unroll
        for (int j = 0; j < S::TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }
    __syncthreads();
    t = nt;
    kt = nkt;
    m0 = nm0;
    n0 = nn0;
    interior = ninterior;
  }
}

template <class S>
__global__ void __launch_bounds__(S::NT)
    prod_kernel(Problem p, int tiles_m, int tiles_n) {
  prod_body<S>(p, tiles_m, tiles_n, blockIdx.x, gridDim.x);
}

// Split-K: grid row y computes the partial product over k in
// [y * kc, min(K, (y + 1) * kc)) into its own M x N slab of `ws` (row pitch
// N), by the same tile loop on the sub-problem.  The slabs are summed by
// splitk_reduce_kernel.
template <class S>
__global__ void __launch_bounds__(S::NT)
    prod_split_kernel(Problem p, int tiles_m, int tiles_n, int kc, float *ws) {
  const int y = blockIdx.y;
  const int k0 = y * kc;
  Problem ps = p;
  ps.A = p.A + k0;
  ps.B = p.B + (long long)k0 * p.ldb;
  ps.K = p.K - k0 < kc ? p.K - k0 : kc;
  ps.C = ws + (long long)y * p.M * p.N;
  ps.ldc = p.N;
  prod_body<S>(ps, tiles_m, tiles_n, blockIdx.x, gridDim.x);
}

constexpr int kReduceThreads = 256;

// C[i][j] = sum over y = 0 .. splits-1, in that order, of ws[y][i][j]: one
// thread per 4 consecutive columns of a row, grid-stride.
__global__ void __launch_bounds__(kReduceThreads)
    splitk_reduce_kernel(const float *ws, int splits, int M, int N, float *C, long long ldc) {
  const long long slab = (long long)M * N;
  const int nq = (N + 3) / 4;
  const long long total = (long long)M * nq;
  const long long stride = (long long)gridDim.x * kReduceThreads;
  for (long long e = (long long)blockIdx.x * kReduceThreads + threadIdx.x; e < total;
       e += stride) {
    const long long i = e / nq;
    const int j = (int)(e - i * nq) * 4;
    const float *w = ws + i * N + j;
    float *c = C + i * ldc + j;
    if (j + 4 <= N) {
      // Loads of 8 slabs are issued together; the additions keep slab order.
      f32x4 acc = *reinterpret_cast<const f32x4u *>(w);
      int y = 1;
      for (; y + 8 <= splits; y += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4u *>(w + (y + u) * slab);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
      }
      for (; y < splits; ++y) acc += *reinterpret_cast<const f32x4u *>(w + y * slab);
      *reinterpret_cast<f32x4u *>(c) = acc;
    } else {
      for (int e2 = 0; j + e2 < N; ++e2) {
        float acc = w[e2];
        for (int y = 1; y < splits; ++y) acc += w[e2 + y * slab];
        c[e2] = acc;
      }
    }
  }
}

// ---- k-loop kernel with direct-to-LDS operand loads ---------------------
// global_load_lds_dwordx4 writes each lane's 16 bytes straight into LDS at
// the wave's base address + 16 * lane.  An interior k step then needs no
// staging registers, no LDS write instructions and no wait in the middle of
// the step: the next stage's loads are issued at the top of the step and
// waited for just before the step's barrier.  One instruction fills 1 KB of
// LDS, so A (rows of BK = 32 k-contiguous floats) is stored without padding,
// with the 16-byte chunks of each row permuted (chunk c of row r sits at
// position c ^ ((r >> 1) & 7)) so that the fragment reads of 16 consecutive
// rows fall on distinct banks; a B row of BN = 256 floats is exactly one
// instruction and keeps the padded pitch of the register-staged kernel.
// Steps that cannot use it (the K tail, and every step of a tile that
// overhangs a product narrower than one tile) go through registers and write
// the same layout before the step's MFMAs.  Each element is summed in the
// same k order as in prod_kernel, so the two give identical bits.

__device__ inline void load_to_lds16(const float *src, float *lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_t *)src, (lds_void_t *)lds_dst, 16, 0, 0);
}

template <class S>
struct LdsDma {
  static constexpr int CPR = S::BK / 4;           // 16-byte chunks per A row
  static constexpr int RPB = 64 / CPR;            // A rows per 1 KB instruction
  static constexpr int NW = S::NT / 64;
  static constexpr int A_BLK = S::BM / RPB / NW;  // A instructions per wave
  static constexpr int B_ROWS = S::BK / NW;       // B instructions (rows) per wave
  static constexpr int A_STAGE = S::BM * S::BK;   // unpadded
  static constexpr int B_STAGE = S::B_STAGE;
  static_assert(S::BN == 256, "one B row per instruction");
  static_assert(CPR == 8, "the row permutation is written for 8 chunks per A row");
  static_assert(S::BM % (RPB * NW) == 0 && S::BK % NW == 0, "instructions split evenly");
  static_assert(S::WTM % 16 == 0, "the permutation is the same for every 32-row block");
};

__device__ inline int a_chunk_perm(int r) { return (r >> 1) & 7; }

template <class S>
__device__ inline void lds_dma_issue(const Problem &p, int m0, int n0, int k0, float *as,
                                     float *bs, int lane, int wave) {
  using D = LdsDma<S>;
  const int pos = lane % D::CPR;
#pragma unroll
  for (int j = 0; j < D::A_BLK; ++j) {
    const int blk = wave * D::A_BLK + j;
    const int r = blk * D::RPB + lane / D::CPR;
    const int c = pos ^ a_chunk_perm(r);
    load_to_lds16(p.A + (long long)(m0 + r) * p.lda + k0 + 4 * c, as + blk * 256);
  }
#pragma unroll
  for (int j = 0; j < D::B_ROWS; ++j) {
    const int k = wave * D::B_ROWS + j;
    load_to_lds16(p.B + (long long)(k0 + k) * p.ldb + n0 + 4 * lane, bs + k * S::SB);
  }
}

// Register-path write of one staged k step into the direct-load layout.
template <class S, bool PLACED>
__device__ inline void store_lds_perm_as(const Stage<S> &st, float *as, float *bs, int tid) {
  const int arow = tid / (S::BK / 4), c = tid % (S::BK / 4);
#pragma unroll
  for (int i = 0; i < S::A_CHUNKS; ++i) {
    const int r = arow + i * S::A_ROWS_PER_PASS;
    *reinterpret_cast<f32x4 *>(as + r * S::BK + 4 * (c ^ a_chunk_perm(r))) =
        PLACED ? place(st.a[i], st.ameta[i]) : st.a[i];
  }
  const int bkr = tid / (S::BN / 4), bnq = (tid % (S::BN / 4)) * 4;
#pragma unroll
  for (int i = 0; i < S::B_CHUNKS; ++i)
    *reinterpret_cast<f32x4 *>(bs + (bkr + i * S::B_ROWS_PER_PASS) * S::SB + bnq) =
        PLACED ? place(st.b[i], st.bmeta[i]) : st.b[i];
}

// All MFMAs of one k step from the direct-load layout (A chunks permuted).
template <class S>
__device__ inline void compute_stage_perm(f32x16 (&acc)[S::TM][S::TN], const float *as,
                                          const float *bs, int wm, int wn, int lane) {
  const int l32 = lane & 31, h = lane >> 5;
  const int perm = a_chunk_perm(l32);
  const float *a_row = as + (wm * S::WTM + l32) * S::BK;
  const float *b_base = bs + (4 * h) * S::SB + wn * S::WTN + l32;
#pragma unroll
  for (int kg = 0; kg < S::BK / 8; ++kg) {
    f32x4 af[S::TM];
    float bf[S::TN][4];
    const int pos = (2 * kg + h) ^ perm;
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
      af[tm] = *reinterpret_cast<const f32x4 *>(a_row + tm * 32 * S::BK + 4 * pos);
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
      for (int s = 0; s < 4; ++s) bf[tn][s] = b_base[(kg * 8 + s) * S::SB + tn * 32];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(bf[tn][s], af[tm][s], acc[tm][tn],
                                                             0, 0, 0);
  }
}

// The persistent tile loop of prod_kernel with direct-to-LDS loads.  The
// launcher guarantees 16-byte aligned rows of A and B (pointers and leading
// dimensions) and N % 4 == 0, so every tile origin is 16-byte aligned.
template <class S>
__global__ void __launch_bounds__(S::NT) lds_dma_kernel(Problem p, int tiles_m, int tiles_n) {
  using D = LdsDma<S>;
  static_assert(2 * (D::A_STAGE + D::B_STAGE) * 4 <= kLdsBytes, "two stages must fit in LDS");
  __shared__ __attribute__((aligned(16))) float lds[2 * (D::A_STAGE + D::B_STAGE)];
  float *const as0 = lds;
  float *const bs0 = lds + 2 * D::A_STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int ntiles = tiles_m * tiles_n;
  const int nk = (p.K + S::BK - 1) / S::BK;
  const int G = gridDim.x;
  const int lid = xcd_remap(blockIdx.x, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int my_tiles = (ntiles - lid + G - 1) / G;
  const long long steps = (long long)my_tiles * nk;

  int t = lid, kt = 0;
  int m0, n0;
  bool interior;
  tile_origin<S>(t, tiles_m, tiles_n, m0, n0, interior, p);

  f32x16 acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Stage<S> st;
  if (interior && S::BK <= p.K) {
    lds_dma_issue<S>(p, m0, n0, 0, as0, bs0, lane, wave);
  } else {
    const bool g = load_step<S>(st, p, m0, n0, 0, interior, tid);
    if (g)
      store_lds_perm_as<S, true>(st, as0, bs0, tid);
    else
      store_lds_perm_as<S, false>(st, as0, bs0, tid);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));
  __syncthreads();

  for (long long it = 0; it < steps; ++it) {
    const int cur = (int)(it & 1);
    const bool more = it + 1 < steps;
    int nt = t, nkt = kt + 1;
    int nm0 = m0, nn0 = n0;
    bool ninterior = interior;
    if (nkt == nk) {
      nkt = 0;
      nt = t + G;
      if (more) tile_origin<S>(nt, tiles_m, tiles_n, nm0, nn0, ninterior, p);
    }
    if (more) {
      // The other stage was last read before the previous barrier.
      float *const an = as0 + (cur ^ 1) * D::A_STAGE;
      float *const bn = bs0 + (cur ^ 1) * D::B_STAGE;
      const int nk0 = nkt * S::BK;
      if (ninterior && nk0 + S::BK <= p.K) {
        lds_dma_issue<S>(p, nm0, nn0, nk0, an, bn, lane, wave);
      } else {  // rare: written before this step's MFMAs, so no stage stays live
        const bool g = load_step<S>(st, p, nm0, nn0, nk0, ninterior, tid);
        if (g)
          store_lds_perm_as<S, true>(st, an, bn, tid);
        else
          store_lds_perm_as<S, false>(st, an, bn, tid);
      }
    }
    compute_stage_perm<S>(acc, as0 + cur * D::A_STAGE, bs0 + cur * D::B_STAGE, wm, wn, lane);
    if (kt == nk - 1) {
      store_c<S>(acc, p, m0, n0, wm, wn, lane, !interior);
#pragma unroll
      for (int i = 0; i < S::TM; ++i)
#pragma unroll
        for (int j = 0; j < S::TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));  // this wave's direct loads landed
    __syncthreads();
    t = nt;
    kt = nkt;
    m0 = nm0;
    n0 = nn0;
    interior = ninterior;
  }
}

// ---- the direct-to-LDS k loop on 16x16x4 MFMAs -------------------------
// lds_dma_kernel with each wave's WTM x WTN sub-tile computed as 16x16
// blocks on v_mfma_f32_16x16x4_f32 instead of 32x32 blocks on 32x32x2: the
// same matrix-pipe time and the same LDS traffic, but (WTM/16)(WTN/16)
// independent accumulator chains per wave instead of (WTM/32)(WTN/32).
// Within a 16-deep chunk h of a step, MFMA t takes k = 16 h + 4 g + t for
// lane group g = l / 16; the A layout is lds_dma_kernel's, B rows use a
// pitch of BN + 4 floats so that the four lane groups, reading k rows 4
// apart, fall on distinct banks.  The k order inside a step differs from
// prod_kernel, so the bits may differ.
template <class S>
struct LdsDma16 {
  static constexpr int SB = S::BN + 4;
  static constexpr int A_STAGE = S::BM * S::BK;
  static constexpr int B_STAGE = S::BK * SB;
  static constexpr int TBM = S::WTM / 16, TBN = S::WTN / 16;
};

template <class S>
__device__ inline void lds_dma16_issue(const Problem &p, int m0, int n0, int k0, float *as,
                                       float *bs, int lane, int wave) {
  using D = LdsDma<S>;
  const int pos = lane % D::CPR;
#pragma unroll
  for (int j = 0; j < D::A_BLK; ++j) {
    const int blk = wave * D::A_BLK + j;
    const int r = blk * D::RPB + lane / D::CPR;
    const int c = pos ^ a_chunk_perm(r);
    load_to_lds16(p.A + (long long)(m0 + r) * p.lda + k0 + 4 * c, as + blk * 256);
  }
#pragma unroll
  for (int j = 0; j < D::B_ROWS; ++j) {
    const int k = wave * D::B_ROWS + j;
    load_to_lds16(p.B + (long long)(k0 + k) * p.ldb + n0 + 4 * lane,
                  bs + k * LdsDma16<S>::SB);
  }
}

template <class S, bool PLACED>
__device__ inline void store_lds_perm16_as(const Stage<S> &st, float *as, float *bs, int tid) {
  const int arow = tid / (S::BK / 4), c = tid % (S::BK / 4);
#pragma unroll
  for (int i = 0; i < S::A_CHUNKS; ++i) {
    const int r = arow + i * S::A_ROWS_PER_PASS;
    *reinterpret_cast<f32x4 *>(as + r * S::BK + 4 * (c ^ a_chunk_perm(r))) =
        PLACED ? place(st.a[i], st.ameta[i]) : st.a[i];
  }
  const int bkr = tid / (S::BN / 4), bnq = (tid % (S::BN / 4)) * 4;
#pragma unroll
  for (int i = 0; i < S::B_CHUNKS; ++i)
    *reinterpret_cast<f32x4 *>(bs + (bkr + i * S::B_ROWS_PER_PASS) * LdsDma16<S>::SB + bnq) =
        PLACED ? place(st.b[i], st.bmeta[i]) : st.b[i];
}

template <class S>
__device__ inline void compute_stage16(f32x4 (&acc)[LdsDma16<S>::TBM][LdsDma16<S>::TBN],
                                       const float *as, const float *bs, int wm, int wn,
                                       int lane) {
  using D = LdsDma16<S>;
  const int l16 = lane & 15, g = lane >> 4;
  const int perm = a_chunk_perm(l16);  // rows of a wave differ by multiples of 16
  const float *a_row = as + (wm * S::WTM + l16) * S::BK;
  const float *b_base = bs + (4 * g) * D::SB + wn * S::WTN + l16;
#pragma unroll
  for (int h = 0; h < S::BK / 16; ++h) {
    f32x4 af[D::TBM];
    float bf[D::TBN][4];
    const int pos = (4 * h + g) ^ perm;
#pragma unroll
    for (int bm = 0; bm < D::TBM; ++bm)
      af[bm] = *reinterpret_cast<const f32x4 *>(a_row + bm * 16 * S::BK + 4 * pos);
#pragma unroll
    for (int bn = 0; bn < D::TBN; ++bn)
#pragma unroll
      for (int t = 0; t < 4; ++t) bf[bn][t] = b_base[(16 * h + t) * D::SB + bn * 16];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int bm = 0; bm < D::TBM; ++bm)
#pragma unroll
        for (int bn = 0; bn < D::TBN; ++bn)
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[bn][t], af[bm][t], acc[bm][bn],
                                                             0, 0, 0);
  }
}

template <class S>
__device__ inline void store_c16(const f32x4 (&acc)[LdsDma16<S>::TBM][LdsDma16<S>::TBN],
                                 const Problem &p, int m0, int n0, int wm, int wn, int lane,
                                 bool guard) {
  using D = LdsDma16<S>;
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int bm = 0; bm < D::TBM; ++bm) {
    const int row = m0 + wm * S::WTM + 16 * bm + l16;
    float *crow = p.C + (long long)row * p.ldc;
#pragma unroll
    for (int bn = 0; bn < D::TBN; ++bn) {
      const int col = n0 + wn * S::WTN + 16 * bn + 4 * g;
      const f32x4 v = acc[bm][bn];
      if (!guard || (row < p.M && col + 4 <= p.N)) {
        *reinterpret_cast<f32x4u *>(crow + col) = v;
      } else if (row < p.M) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (col + r < p.N) crow[col + r] = v[r];
      }
    }
  }
}

template <class S>
__global__ void __launch_bounds__(S::NT) lds_dma16_kernel(Problem p, int tiles_m, int tiles_n) {
  using D = LdsDma16<S>;
  static_assert(2 * (D::A_STAGE + D::B_STAGE) * 4 <= kLdsBytes, "two stages must fit in LDS");
  __shared__ __attribute__((aligned(16))) float lds[2 * (D::A_STAGE + D::B_STAGE)];
  float *const as0 = lds;
  float *const bs0 = lds + 2 * D::A_STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int ntiles = tiles_m * tiles_n;
  const int nk = (p.K + S::BK - 1) / S::BK;
  const int G = gridDim.x;
  const int lid = xcd_remap(blockIdx.x, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int my_tiles = (ntiles - lid + G - 1) / G;
  const long long steps = (long long)my_tiles * nk;

  int t = lid, kt = 0;
  int m0, n0;
  bool interior;
  tile_origin<S>(t, tiles_m, tiles_n, m0, n0, interior, p);

  f32x4 acc[D::TBM][D::TBN];
#pragma unroll
  for (int i = 0; i < D::TBM; ++i)
#pragma unroll
    for (int j = 0; j < D::TBN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Stage<S> st;
  if (interior && S::BK <= p.K) {
    lds_dma16_issue<S>(p, m0, n0, 0, as0, bs0, lane, wave);
  } else {
    const bool g = load_step<S>(st, p, m0, n0, 0, interior, tid);
    if (g)
      store_lds_perm16_as<S, true>(st, as0, bs0, tid);
    else
      store_lds_perm16_as<S, false>(st, as0, bs0, tid);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));
  __syncthreads();

  for (long long it = 0; it < steps; ++it) {
    const int cur = (int)(it & 1);
    const bool more = it + 1 < steps;
    int nt = t, nkt = kt + 1;
    int nm0 = m0, nn0 = n0;
    bool ninterior = interior;
    if (nkt == nk) {
      nkt = 0;
      nt = t + G;
      if (more) tile_origin<S>(nt, tiles_m, tiles_n, nm0, nn0, ninterior, p);
    }
    if (more) {
      float *const an = as0 + (cur ^ 1) * D::A_STAGE;
      float *const bn = bs0 + (cur ^ 1) * D::B_STAGE;
      const int nk0 = nkt * S::BK;
      if (ninterior && nk0 + S::BK <= p.K) {
        lds_dma16_issue<S>(p, nm0, nn0, nk0, an, bn, lane, wave);
      } else {
        const bool g = load_step<S>(st, p, nm0, nn0, nk0, ninterior, tid);
        if (g)
          store_lds_perm16_as<S, true>(st, an, bn, tid);
        else
          store_lds_perm16_as<S, false>(st, an, bn, tid);
      }
    }
    compute_stage16<S>(acc, as0 + cur * D::A_STAGE, bs0 + cur * D::B_STAGE, wm, wn, lane);
    if (kt == nk - 1) {
      store_c16<S>(acc, p, m0, n0, wm, wn, lane, !interior);
#pragma unroll
      for (int i = 0; i < D::TBM; ++i)
#pragma unroll
        for (int j = 0; j < D::TBN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));
    __syncthreads();
    t = nt;
    kt = nkt;
    m0 = nm0;
    n0 = nn0;
    interior = ninterior;
  }
}

// ---- 64x64 tiles with K split over the waves, 3-stage direct-load pipe --
// For products with about one 64x64 tile per CU (1024^3 has 256), where a
// k step of a 64x64 tile is too short to hide the latency of its loads.
// Each of the 4 waves computes the whole 64x64 tile over its own quarter of
// every 64-deep k step (k in [16w, 16w + 16) of the step) with
// v_mfma_f32_16x16x4_f32: 16 independent 16x16 accumulator blocks per wave,
// so one wave per SIMD keeps the matrix pipe busy.  The four partial tiles
// are added in wave order through LDS at the end of the tile, so the result
// is deterministic (but summed in a different order from the other entries).
//
// A wave loads exactly the operands it reads -- its k quarter of the tile's
// 64 A rows and its 16 k rows of B -- into LDS regions of its own, so the k
// loop has no workgroup barrier: each wave waits only for its own loads and
// runs at its own pace until the tile's partial sums meet.  Operands arrive
// by global_load_lds_dwordx4 into three LDS stages: the loads for step i + 3
// are issued during step i, into the stage whose fragments the wave already
// holds in registers (fragments are read one step ahead), so each load has
// two steps to land.  A partial last k step goes through registers, zero
// past K, into the same regions.
//
// MFMA operand roles: B is the first operand, A the second, so lane l of
// block (bm, bn) holds C[m = 16 bm + l % 16][n = 16 bn + 4 (l / 16) + r],
// r = 0..3.  Within a wave's 16 k of a step, MFMA t takes k = 4 g + t for
// lane group g = l / 16, so a lane's A operand for t = 0..3 is one 128-bit
// LDS read.  LDS layouts of a stage (16-byte chunks):
//   A: wave w's quarter at float 1024 w, chunk c of row r at ks_a_pos(r, c);
//   B: from float 4096, chunk c of k row k at 16 k + (c ^ (4 ((k >> 2) & 3))).
// Both make the fragment reads of a wave conflict-free.  The partial tiles
// use rows of 16 chunks, chunk c of row r at 16 r + (c ^ (r & 15)).
using KsTile = Tile<64, 64, 64, 2, 2, false>;  // tile origins
constexpr int kKsStages = 3;
constexpr int kKsStageFloats = 64 * 64 * 2;   // A and B, unpadded
constexpr int kKsQuarterFloats = 64 * 16;     // a wave's A quarter
constexpr int kKsRedFloats = 4 * 64 * 64;     // the four partial tiles
constexpr int kKsDmaPerWave = 8;              // 4 A + 4 B instructions of 1 KB

__device__ inline int ks_red_pos(int r, int c) { return r * 16 + (c ^ (r & 15)); }
__device__ inline int ks_b_pos(int k, int c) { return k * 16 + (c ^ (4 * ((k >> 2) & 3))); }

// A partial k step through registers: wave `wave` loads its quarter of the
// step starting at column k0 -- A rows m0 .. m0 + 63, columns k0 + 16 w ..
// + 15, and B rows k0 + 16 w .. + 15, columns n0 .. n0 + 63 -- with zeros
// for k >= K, and writes it to its own regions of stage `st`.  Rows of A and
// B are 16-byte aligned and chunks start at multiples of 4, so a chunk lies
// wholly inside K (one 128-bit load), partly (per-element loads) or outside.
__device__ inline void ks_fill_partial(const Problem &p, int m0, int n0, int k0, float *st,
                                       int lane, int wave) {
  f32x4 a[4], b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 16 * q + lane / 4, kc = k0 + 16 * wave + 4 * (lane & 3);
    const int valid = chunk_valid(kc, p.K);
    const float *src = p.A + (long long)(m0 + r) * p.lda + kc;
    a[q] = valid == 4 ? load4(src) : load_partial(src, valid);
    const int k = k0 + 16 * wave + 4 * q + lane / 16;
    b[q] = k < p.K ? load4(p.B + (long long)k * p.ldb + n0 + 4 * (lane & 15))
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float *sa = st + wave * kKsQuarterFloats;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    *reinterpret_cast<f32x4 *>(sa + 4 * ks_a_pos(16 * q + lane / 4, lane & 3)) = a[q];
    *reinterpret_cast<f32x4 *>(st + 64 * 64 +
                               4 * ks_b_pos(16 * wave + 4 * q + lane / 16, lane & 15)) = b[q];
  }
}

struct KsFrag {
  f32x4 a[4];     // per row block bm: A[16 bm + l%16][16 w + 4 g + t], t = 0..3
  float b[4][4];  // per column block bn and t: B[16 w + 4 g + t][16 bn + l%16]
};

__device__ inline void ks_read_frag(KsFrag &f, const float *st, int lane, int wave) {
  const int l16 = lane & 15, g = lane >> 4;
  const float *sa = st + wave * kKsQuarterFloats;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
    f.a[bm] = *reinterpret_cast<const f32x4 *>(sa + 4 * ks_a_pos(16 * bm + l16, g));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int k = 16 * wave + 4 * g + t;
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int n = 16 * bn + l16;
      f.b[bn][t] = st[64 * 64 + 4 * ks_b_pos(k, n >> 2) + (n & 3)];
    }
  }
}

// The step's 64 MFMAs in 8 groups of 8; with DMA, direct load q of the next
// stage is issued after group q, so its issue overlaps the matrix work of a
// lone wave.
// ACC: how the MFMAs accumulate -- kKsBuiltin (the compiler's MFMA),
// kKsInPlace or kKsFromZero (mfma_inplace, the latter starting the tile).
enum KsAcc { kKsBuiltin, kKsInPlace, kKsFromZero };
template <bool DMA, KsAcc ACC = kKsBuiltin>
__device__ inline void ks_mfma(f32x4 (&acc)[4][4], const KsFrag &f, const unsigned (&voff)[8],
                               const float *abase, const float *bbase, unsigned lds_a,
                               unsigned lds_b) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int bm = 2 * half; bm < 2 * half + 2; ++bm)
#pragma unroll
        for (int bn = 0; bn < 4; ++bn) {
          if constexpr (ACC == kKsBuiltin)
            acc[bm][bn] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.b[bn][t], f.a[bm][t],
                                                               acc[bm][bn], 0, 0, 0);
          else if (ACC == kKsFromZero && t == 0)
            mfma_inplace<true>(acc[bm][bn], f.b[bn][t], f.a[bm][t]);
          else
            mfma_inplace<false>(acc[bm][bn], f.b[bn][t], f.a[bm][t]);
        }
      if constexpr (DMA) {
        __builtin_amdgcn_sched_barrier(0);  // keep each load after its group
        const int q = 2 * t + half;
        if (q < 4)
          ks_load_to_lds16(voff[q], abase, lds_a + q * 4 * 64 * 4);
        else
          ks_load_to_lds16(voff[q], bbase, lds_b + (q - 4) * 4 * 64 * 4);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
}

// Waits for this wave's vector-memory operations down to `n` outstanding
// (n is 0, 8 or 16: one step's direct loads per 8).  A wave reads only LDS
// its own loads wrote, so this wait -- no barrier -- makes a stage readable;
// the empty assembly keeps the compiler from moving LDS reads above it.
__device__ inline void ks_wait_own(int n) {
  if (n >= 16)
    __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(16));
  else if (n >= 8)
    __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(8));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));
  asm volatile("" ::: "memory");
}

// The end of a tile: each wave writes its partial 64x64 tile to LDS, and
// after a barrier wave w adds rows 16 w .. 16 w + 15 of the four in wave
// order (lane (row, q) takes chunks 4 j + q, j = 0..3, of its row) and
// stores them to C.
__device__ inline void ks_finish_tile(const f32x4 (&acc)[4][4], float *red, const Problem &p,
                                      int m0, int n0, int lane, int wave) {
  const int l16 = lane & 15, g = lane >> 4;
  float *mine = red + wave * 64 * 64;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
      *reinterpret_cast<f32x4 *>(mine + 4 * ks_red_pos(16 * bm + l16, 4 * bn + g)) = acc[bm][bn];
  ks_lds_barrier();
  const int row = 16 * wave + (lane >> 2), q = lane & 3;
  const int gm = m0 + row;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 4 * j + q;
    f32x4 v = *reinterpret_cast<const f32x4 *>(red + 4 * ks_red_pos(row, c));
#pragma unroll
    for (int w = 1; w < 4; ++w)
      v += *reinterpret_cast<const f32x4 *>(red + w * 64 * 64 + 4 * ks_red_pos(row, c));
    *reinterpret_cast<f32x4u *>(p.C + (long long)gm * p.ldc + n0 + 4 * c) = v;
  }
}

// The launcher guarantees M, N >= 64 (every tile lies inside C after the
// edge shift), N % 4 == 0, 16-byte aligned rows of A and B, and per-lane
// byte offsets that fit in 32 bits (lane_offsets_fit over 64 rows of each).
__global__ void __launch_bounds__(256) ksplit_kernel(Problem p, int tiles_m, int tiles_n) {
  static_assert((kKsStages * kKsStageFloats + kKsRedFloats) * 4 <= kLdsBytes, "LDS budget");
  __shared__ __attribute__((aligned(16))) float lds[kKsStages * kKsStageFloats + kKsRedFloats];
  float *const red = lds + kKsStages * kKsStageFloats;
  const unsigned lds_u = (unsigned)(uintptr_t)(lds_void_t *)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntiles = tiles_m * tiles_n;
  const int nk = (p.K + 63) / 64;
  const int G = gridDim.x;
  const int lid = xcd_remap(blockIdx.x, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int my_tiles = (ntiles - lid + G - 1) / G;
  const int steps = my_tiles * nk;
  const bool k_tail = (p.K & 63) != 0;  // the last step of every tile is partial

  // Per-lane byte offsets of this wave's direct loads from the step's base
  // addresses: q < 4 fill its A quarter (rows 16 q + l / 4), the others its
  // B k rows 16 w + 4 (q - 4) + l / 16; chunks permuted as in the layouts.
  unsigned voff[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    voff[q] = (unsigned)(ks_dma_a_elem(q, lane, wave, p.lda) * 4);
    voff[4 + q] = (unsigned)(dma_b_elem<16>(64 * (4 * wave + q) + lane, p.ldb) * 4);
  }
  const unsigned wave_a = (unsigned)(wave * kKsQuarterFloats * 4);  // LDS bytes
  const unsigned wave_b = (unsigned)((64 * 64 + 16 * wave * 64) * 4);

  // The issue side walks steps it + 3 ahead of the consumer: its tile, k
  // step and tile origin are kept incrementally.
  int is_t = 0, is_k = 0, is_m0 = 0, is_n0 = 0;
  auto issue_origin = [&]() __attribute__((always_inline)) {
    bool interior;
    tile_origin<KsTile>(lid + is_t * G, tiles_m, tiles_n, is_m0, is_n0, interior, p);
  };
  auto issue_advance = [&]() __attribute__((always_inline)) {
    if (++is_k == nk) {
      is_k = 0;
      ++is_t;
      if (is_t < my_tiles) issue_origin();
    }
  };
  auto issue_direct = [&]() __attribute__((always_inline)) {
    return !k_tail || is_k != nk - 1;
  };
  // Register path for one step (the K tail).  Nothing of it stays
  // outstanding: without this wait the compiler, merging paths, would wait
  // on all vector memory before later LDS reads, which includes the direct
  // loads in flight.
  auto issue_regs = [&](float *st) __attribute__((always_inline)) {
    ks_fill_partial(p, is_m0, is_n0, is_k * 64, st, lane, wave);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));
  };
  auto abase_of = [&]() __attribute__((always_inline)) {
    return p.A + (long long)is_m0 * p.lda + is_k * 64;
  };
  auto bbase_of = [&]() __attribute__((always_inline)) {
    return p.B + (long long)(is_k * 64) * p.ldb + is_n0;
  };

  f32x4 acc[4][4];
  issue_origin();
  // Prologue: steps 0..2 in flight; wait for step 0 only.  `after` counts
  // the direct loads issued after step 0's (a register step completes
  // everything before it).
  int after = 0;
  for (int s = 0; s < kKsStages && s < steps; ++s) {
    const unsigned st = lds_u + s * kKsStageFloats * 4;
    if (issue_direct()) {
      const float *ab = abase_of(), *bb = bbase_of();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ks_load_to_lds16(voff[q], ab, st + wave_a + q * 4 * 64 * 4);
        ks_load_to_lds16(voff[4 + q], bb, st + wave_b + q * 4 * 64 * 4);
      }
      if (s > 0) after += kKsDmaPerWave;
    } else {
      issue_regs(lds + s * kKsStageFloats);
      after = 0;
    }
    issue_advance();
  }
  ks_wait_own(after);
  KsFrag f0, f1;
  ks_read_frag(f0, lds, lane, wave);

  // One step: `fc` holds this step's fragments, `fn` receives the next's.
  auto step = [&](int it, KsFrag &fc, KsFrag &fn) __attribute__((always_inline)) {
    const int cur = it % kKsStages;
    // This wave's reads of stage `cur` (the fragments of step it) are
    // complete, so the stage may be refilled; once step it + 1's loads have
    // landed its stage may be read.  Step it + 2 is the issue side's
    // previous step.
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);
    if (it + 1 < steps) {
      const bool next2_direct =
          it + 2 < steps && (!k_tail || (is_k + nk - 1) % nk != nk - 1);
      ks_wait_own(next2_direct ? kKsDmaPerWave : 0);
      ks_read_frag(fn, lds + ((it + 1) % kKsStages) * kKsStageFloats, lane, wave);
    }
    // Step it + 3 goes into stage `cur`: direct loads spread over this
    // step's MFMAs, or (for a K tail) the register path before them.
    if (it + kKsStages < steps) {
      const unsigned st = lds_u + cur * kKsStageFloats * 4;
      if (issue_direct()) {
        ks_mfma<true>(acc, fc, voff, abase_of(), bbase_of(), st + wave_a, st + wave_b);
      } else {
        issue_regs(lds + cur * kKsStageFloats);
        ks_mfma<false>(acc, fc, voff, nullptr, nullptr, 0, 0);
      }
      issue_advance();
    } else {
      ks_mfma<false>(acc, fc, voff, nullptr, nullptr, 0, 0);
    }
  };
  // Tile done: add the four partial tiles in wave order and store.  The
  // next tile's partial tiles overwrite the buffer: every wave must have
  // read it first (the k loop has no barrier of its own).
  auto finish_tile = [&](int t) __attribute__((always_inline)) {
    int m0, n0;
    bool interior;
    tile_origin<KsTile>(lid + t * G, tiles_m, tiles_n, m0, n0, interior, p);
    ks_finish_tile(acc, red, p, m0, n0, lane, wave);
    if (t + 1 < my_tiles) ks_lds_barrier();
  };

  // Tile loop outside, k steps inside (unrolled by two so that the fragment
  // sets keep fixed registers); the accumulators stay in one register class.
  int it = 0;
  for (int t = 0; t < my_tiles; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk + 1 < nk; kk += 2, it += 2) {
      step(it, f0, f1);
      step(it + 1, f1, f0);
    }
    if (nk & 1) {
      step(it, f0, f1);
      ++it;
      f0 = f1;  // the next step's fragments are read into f1
    }
    finish_tile(t);
  }
}

// ksplit_kernel for K a multiple of 64, without its per-step conditions.
// The issue side never runs past the last step: having reached it, it
// issues that step's loads again (in bounds; nothing reads them), so every
// step waits for the same count, reads the next step's fragments and issues
// one step of loads, and the loop's only branches are its own and the issue
// side's move to the next tile.  Same launch conditions as ksplit_kernel.
__global__ void __launch_bounds__(256) ksplit_whole_kernel(Problem p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) float lds[kKsStages * kKsStageFloats + kKsRedFloats];
  float *const red = lds + kKsStages * kKsStageFloats;
  const unsigned lds_u = (unsigned)(uintptr_t)(lds_void_t *)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntiles = tiles_m * tiles_n;
  const int nk = p.K / 64;
  const int G = gridDim.x;
  const int lid = xcd_remap(blockIdx.x, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int my_tiles = (ntiles - lid + G - 1) / G;

  unsigned voff[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    voff[q] = (unsigned)(ks_dma_a_elem(q, lane, wave, p.lda) * 4);
    voff[4 + q] = (unsigned)(dma_b_elem<16>(64 * (4 * wave + q) + lane, p.ldb) * 4);
  }
  const unsigned wave_a = (unsigned)(wave * kKsQuarterFloats * 4);  // LDS bytes
  const unsigned wave_b = (unsigned)((64 * 64 + 16 * wave * 64) * 4);

  // Issue side: tile is_t, k step is_k, and that step's base addresses.
  int is_t = 0, is_k = 0;
  const float *a_is = p.A, *b_is = p.B;
  const long long b_step = 64LL * p.ldb;
  auto issue_origin = [&]() __attribute__((always_inline)) {
    int m0, n0;
    bool interior;
    tile_origin<KsTile>(lid + is_t * G, tiles_m, tiles_n, m0, n0, interior, p);
    a_is = p.A + (long long)m0 * p.lda;
    b_is = p.B + n0;
  };
  auto issue_advance = [&]() __attribute__((always_inline)) {
    if (++is_k < nk) {
      a_is += 64;
      b_is += b_step;
    } else if (is_t + 1 < my_tiles) {
      is_k = 0;
      ++is_t;
      issue_origin();
    } else {
      is_k = nk - 1;  // past the last step: repeat its loads
    }
  };
  // Stages of steps it, it + 1 and it + 2 (float offsets into lds).
  int o_c = 0, o_1 = kKsStageFloats, o_2 = 2 * kKsStageFloats;
  auto issue_into = [&](int o) __attribute__((always_inline)) {
    const unsigned st = lds_u + o * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ks_load_to_lds16(voff[q], a_is, st + wave_a + q * 4 * 64 * 4);
      ks_load_to_lds16(voff[4 + q], b_is, st + wave_b + q * 4 * 64 * 4);
    }
    issue_advance();
  };

  f32x4 acc[4][4];
  issue_origin();
  issue_into(o_c);
  issue_into(o_1);
  issue_into(o_2);
  ks_wait_own(2 * kKsDmaPerWave);
  KsFrag f0, f1;
  ks_read_frag(f0, lds + o_c, lane, wave);

  // One step: wait for step it + 1 (step it + 2's loads stay in flight),
  // read its fragments, and run step it's MFMAs with step it + 3's loads
  // going into step it's stage, whose fragments this wave already holds.
  auto step = [&](auto acc_mode, KsFrag &fc, KsFrag &fn) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);
    ks_wait_own(kKsDmaPerWave);
    ks_read_frag(fn, lds + o_1, lane, wave);
    const unsigned st = lds_u + o_c * 4;
    ks_mfma<true, decltype(acc_mode)::value>(acc, fc, voff, a_is, b_is, st + wave_a,
                                              st + wave_b);
    issue_advance();
    const int o = o_c;
    o_c = o_1;
    o_1 = o_2;
    o_2 = o;
  };
  using First = std::integral_constant<KsAcc, kKsFromZero>;
  using Next = std::integral_constant<KsAcc, kKsInPlace>;

  for (int t = 0; t < my_tiles; ++t) {
    // The tile's first step starts its accumulators from 0.
    if (nk == 1) {
      step(First{}, f0, f1);
      f0 = f1;  // the next step's fragments are read into f1
    } else {
      step(First{}, f0, f1);
      step(Next{}, f1, f0);
      for (int kk = 2; kk + 1 < nk; kk += 2) {
        step(Next{}, f0, f1);
        step(Next{}, f1, f0);
      }
      if (nk & 1) {
        step(Next{}, f0, f1);
        f0 = f1;
      }
    }
    // 24 wait states after the last MFMA before its results are read
    // (mfma_inplace); the repeated loads of the last tile land before the
    // workgroup ends.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 == my_tiles) ks_wait_own(0);
    int m0, n0;
    bool interior;
    tile_origin<KsTile>(lid + t * G, tiles_m, tiles_n, m0, n0, interior, p);
    ks_finish_tile(acc, red, p, m0, n0, lane, wave);
    if (t + 1 < my_tiles) ks_lds_barrier();
  }
}

template <class W, bool PLACED>
__device__ inline void w16_store_stage(const Stage<W16Staging<W>> &sg, float *st, int tid) {
  using T = W16Staging<W>;
  const int arow = tid / (T::BK / 4), ac = tid % (T::BK / 4);
#pragma unroll
  for (int i = 0; i < T::A_CHUNKS; ++i) {
    const int r = arow + i * T::A_ROWS_PER_PASS;
    *reinterpret_cast<f32x4 *>(st + 4 * w16_a_pos<W::ACH>(r, ac)) =
        PLACED ? place(sg.a[i], sg.ameta[i]) : sg.a[i];
  }
  const int bkr = tid / (T::BN / 4), bc = tid % (T::BN / 4);
#pragma unroll
  for (int i = 0; i < T::B_CHUNKS; ++i) {
    const int k = bkr + i * T::B_ROWS_PER_PASS;
    *reinterpret_cast<f32x4 *>(st + W::A_FLOATS + 4 * w16_b_pos<W::BCH>(k, bc)) =
        PLACED ? place(sg.b[i], sg.bmeta[i]) : sg.b[i];
  }
}

// All fragments of one chunk, read together (w16_kernel reads a chunk
// ahead of its MFMAs).
template <class W>
struct W16Frag {
  f32x4 a[W::TBM];     // A[row][16 h + 4 g .. + 3]
  float b[W::TBN][4];  // B[16 h + 4 g + t][col]
};

template <class W>
__device__ inline void w16_read_frag(W16Frag<W> &f, const float *st, int h, int lane, int wm,
                                     int wn) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int bm = 0; bm < W::TBM; ++bm)
    f.a[bm] = *reinterpret_cast<const f32x4 *>(
        st + 4 * w16_a_pos<W::ACH>(wm * W::WTM + 16 * bm + l16, 4 * h + g));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int k = 16 * h + 4 * g + t;
#pragma unroll
    for (int bn = 0; bn < W::TBN; ++bn) {
      const int n = wn * W::WTN + 16 * bn + l16;
      f.b[bn][t] = st[W::A_FLOATS + 4 * w16_b_pos<W::BCH>(k, n >> 2) + (n & 3)];
    }
  }
}

template <class W>
__device__ inline void w16_mfma(f32x4 (&acc)[W::TBM][W::TBN], const W16Frag<W> &f, int t) {
#pragma unroll
  for (int bm = 0; bm < W::TBM; ++bm)
#pragma unroll
    for (int bn = 0; bn < W::TBN; ++bn)
      acc[bm][bn] =
          __builtin_amdgcn_mfma_f32_16x16x4f32(f.b[bn][t], f.a[bm][t], acc[bm][bn], 0, 0, 0);
}

// The launcher guarantees M >= BM, N >= BN (every tile lies inside C after
// the edge shift), N % 4 == 0, 16-byte aligned rows of A and B, and per-lane
// byte offsets that fit in 32 bits (lane_offsets_fit over BM rows of A and
// BK rows of B).
template <class W>
__global__ void __launch_bounds__(256) w16_kernel(Problem p, int tiles_m, int tiles_n) {
  using T = W16Staging<W>;
  __shared__ __attribute__((aligned(16))) float lds[W::STAGES * W::STAGE];
  const unsigned lds_u = (unsigned)(uintptr_t)(lds_void_t *)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int ntiles = tiles_m * tiles_n;
  const int nk = (p.K + W::BK - 1) / W::BK;
  const int G = gridDim.x;
  const int lid = xcd_remap(blockIdx.x, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int my_tiles = (ntiles - lid + G - 1) / G;
  const int steps = my_tiles * nk;
  const bool k_tail = (p.K % W::BK) != 0;  // the last step of every tile is partial

  // Per-lane byte offsets of this wave's direct loads from the step's base
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

  // The issue side runs STAGES - 1 steps ahead of the consumer.
  int is_t = 0, is_k = 0, is_m0 = 0, is_n0 = 0;
  auto issue_origin = [&]() __attribute__((always_inline)) {
    bool interior;
    tile_origin<T>(lid + is_t * G, tiles_m, tiles_n, is_m0, is_n0, interior, p);
  };
  auto issue_advance = [&]() __attribute__((always_inline)) {
    if (++is_k == nk) {
      is_k = 0;
      ++is_t;
      if (is_t < my_tiles) issue_origin();
    }
  };
  auto k_direct = [&](int k) __attribute__((always_inline)) { return !k_tail || k != nk - 1; };
  auto issue_regs = [&](float *st) __attribute__((always_inline)) {
    Stage<T> sg;
    const bool g = load_step<T>(sg, p, is_m0, is_n0, is_k * W::BK, true, tid);
    if (g)
      w16_store_stage<W, true>(sg, st, tid);
    else
      w16_store_stage<W, false>(sg, st, tid);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));  // nothing of this path outstanding
  };
  auto issue_dma = [&](unsigned st, int q0, int q1) __attribute__((always_inline)) {
    const float *ab = p.A + (long long)is_m0 * p.lda + is_k * W::BK;
    const float *bb = p.B + (long long)(is_k * W::BK) * p.ldb + is_n0;
#pragma unroll
    for (int q = 0; q < W::DMA; ++q) {
      if (q < q0 || q >= q1) continue;
      if (q < W::A_DMA)
        ks_load_to_lds16(voff[q], ab, st + wave_a + q * 1024);
      else
        ks_load_to_lds16(voff[q], bb, st + wave_b + (q - W::A_DMA) * 1024);
    }
  };

  f32x4 acc[W::TBM][W::TBN];
  issue_origin();
  for (int s = 0; s < W::STAGES - 1 && s < steps; ++s) {
    if (k_direct(is_k))
      issue_dma(lds_u + s * W::STAGE * 4, 0, W::DMA);
    else
      issue_regs(lds + s * W::STAGE);
    issue_advance();
  }

  // One step: wait for its stage (own loads; loads of later steps may stay
  // in flight), barrier, then the MFMAs chunk by chunk with the next chunk's
  // fragments read ahead and the direct loads of step it + STAGES - 1
  // spread over the first half of the step.
  auto step = [&](int it) __attribute__((always_inline)) {
    const int cur = it % W::STAGES;
    {
      // Outstanding younger steps: it + 1 .. it + STAGES - 2.
      int younger = 0;
      for (int d = 1; d <= W::STAGES - 2; ++d)
        if (it + d < steps && k_direct((it + d) % nk)) ++younger;
      if (younger == W::STAGES - 2 && W::STAGES > 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm((W::STAGES - 2) * W::DMA));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));
    }
    ks_lds_barrier();
    const float *st = lds + cur * W::STAGE;
    const int ns = it + W::STAGES - 1;
    const bool issue = ns < steps;
    const bool direct = issue && k_direct(is_k);
    const unsigned nst = lds_u + (ns % W::STAGES) * W::STAGE * 4;
    if (issue && !direct) issue_regs(lds + (ns % W::STAGES) * W::STAGE);
    W16Frag<W> fa, fb;
    w16_read_frag<W>(fa, st, 0, lane, wm, wn);
#pragma unroll
    for (int h = 0; h < W::NQ; ++h) {
      W16Frag<W> &fc = (h & 1) ? fb : fa;
      W16Frag<W> &fn = (h & 1) ? fa : fb;
      if (h + 1 < W::NQ) w16_read_frag<W>(fn, st, h + 1, lane, wm, wn);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        w16_mfma<W>(acc, fc, t);
        // direct loads over the first half of the step's MFMA groups
        constexpr int GROUPS = 4 * W::NQ, SPREAD = GROUPS / 2 > 0 ? GROUPS / 2 : 1;
        const int grp = 4 * h + t;
        if (direct && grp < SPREAD) {
          __builtin_amdgcn_sched_barrier(0);
          issue_dma(nst, grp * W::DMA / SPREAD, (grp + 1) * W::DMA / SPREAD);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (issue) issue_advance();
  };
  auto store_tile = [&](int t) __attribute__((always_inline)) {
    int m0, n0;
    bool interior;
    tile_origin<T>(lid + t * G, tiles_m, tiles_n, m0, n0, interior, p);
    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int bm = 0; bm < W::TBM; ++bm) {
      float *crow = p.C + (long long)(m0 + wm * W::WTM + 16 * bm + l16) * p.ldc + n0 +
                    wn * W::WTN + 4 * g;
#pragma unroll
      for (int bn = 0; bn < W::TBN; ++bn)
        *reinterpret_cast<f32x4u *>(crow + 16 * bn) = acc[bm][bn];
    }
  };

  int it = 0;
  for (int t = 0; t < my_tiles; ++t) {
#pragma unroll
    for (int i = 0; i < W::TBM; ++i)
#pragma unroll
      for (int j = 0; j < W::TBN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < nk; ++kk, ++it) step(it);
    store_tile(t);
  }
}

// ---- the same tiles with operands staged through registers --------------
// For products whose rows are not 16-byte aligned or whose K is not a whole
// number of k steps (direct loads need both): big16_kernel's tile, waves,
// LDS layout and MFMA schedule, with each step's operands loaded into
// registers by 128-bit loads (4-byte alignment suffices) during the first
// rows of MFMAs of the previous step and written to the idle stage during
// its second half.  Rows and columns need no guard: C is at least one tile
// each way and edge tiles are moved inside it.  The K tail does: the step
// that loads a tile's partial last step keeps its loads inside the
// matrices (A columns clamped to the last 4-float window of the row, every
// B chunk read from row 0) and then, after its MFMAs, rewrites that stage
// from guarded loads -- an A chunk that straddles K is loaded as the window
// ending at K and shifted into place, A chunks past K and B rows at or
// past K are zeroed.  Full steps thus carry no per-element selects, and
// the one rewrite per tile sits outside the MFMA stream.  Per-element k
// order as in big16_kernel (the zeroed tail adds exact zeros).
template <class W>
__global__ void __launch_bounds__(256) big16r_kernel(Problem p, int tiles_m, int tiles_n) {
  using T = W16Staging<W>;
  static_assert(W::STAGES == 2, "two stages");
  __shared__ __attribute__((aligned(16))) float lds[2 * W::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int ntiles = tiles_m * tiles_n;
  const int nk = (p.K + W::BK - 1) / W::BK;
  const bool k_tail = p.K % W::BK != 0;  // the last step of every tile is partial
  const int G = gridDim.x;
  const int lid = xcd_remap(blockIdx.x, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int my_tiles = (ntiles - lid + G - 1) / G;

  // Staging map: A chunk i of this thread is row arow + A_ROWS_PER_PASS i,
  // k chunk ac; B chunk i is k row bkr + B_ROWS_PER_PASS i, column chunk bc.
  const int arow = tid / W::ACH, ac = tid % W::ACH;
  const int bkr = tid / W::BCH, bc = tid % W::BCH;
  constexpr int kChunks = T::A_CHUNKS + T::B_CHUNKS;
  f32x4 ra[T::A_CHUNKS], rb[T::B_CHUNKS];
  const long long a_stride = (long long)T::A_ROWS_PER_PASS * p.lda;

  // Unguarded loads of the step at (m0, n0, k0), kept inside the matrices
  // when the step is the partial one (clamp).
  const float *a_src = p.A, *b_src = p.B;
  long long b_stride = 0;
  auto load_setup = [&](int m0, int n0, int k0) __attribute__((always_inline)) {
    const bool partial = k0 + W::BK > p.K;  // uniform
    const int kc = k0 + 4 * ac;
    a_src = p.A + (long long)(m0 + arow) * p.lda + (partial ? min(kc, p.K - 4) : kc);
    b_src = p.B + (partial ? 0LL : (long long)(k0 + bkr) * p.ldb) + n0 + 4 * bc;
    b_stride = partial ? 0LL : (long long)T::B_ROWS_PER_PASS * p.ldb;
  };
  auto load_chunk = [&](int q) __attribute__((always_inline)) {
    if (q < T::A_CHUNKS)
      ra[q] = load4(a_src + q * a_stride);
    else
      rb[q - T::A_CHUNKS] = load4(b_src + (q - T::A_CHUNKS) * b_stride);
  };
  auto store_chunk = [&](float *st, int q) __attribute__((always_inline)) {
    if (q < T::A_CHUNKS)
      *reinterpret_cast<f32x4 *>(
          st + 4 * w16_a_pos<W::ACH>(arow + q * T::A_ROWS_PER_PASS, ac)) = ra[q];
    else
      *reinterpret_cast<f32x4 *>(
          st + W::A_FLOATS +
          4 * w16_b_pos<W::BCH>(bkr + (q - T::A_CHUNKS) * T::B_ROWS_PER_PASS, bc)) =
          rb[q - T::A_CHUNKS];
  };
  // The guarded form of one step, loaded and written in one go.
  auto write_guarded = [&](float *st, int m0, int n0, int k0) __attribute__((always_inline)) {
    int valid = 0, shift = 0;
    const int col = tail_window(k0 + 4 * ac, p.K, valid, shift);
    const int a_meta = (valid << 2) | shift;
    const float *as = p.A + (long long)(m0 + arow) * p.lda + col;
#pragma unroll
    for (int i = 0; i < T::A_CHUNKS; ++i) ra[i] = load4(as + i * a_stride);
    int b_ok = 0;
#pragma unroll
    for (int i = 0; i < T::B_CHUNKS; ++i) {
      const int k = k0 + bkr + i * T::B_ROWS_PER_PASS;
      const bool ok = k < p.K;
      b_ok |= (int)ok << i;
      rb[i] = load4(p.B + (long long)(ok ? k : p.K - 1) * p.ldb + n0 + 4 * bc);
    }
    const f32x4 z{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < T::A_CHUNKS; ++i) ra[i] = place(ra[i], a_meta);
#pragma unroll
    for (int i = 0; i < T::B_CHUNKS; ++i) rb[i] = (b_ok >> i) & 1 ? rb[i] : z;
#pragma unroll
    for (int q = 0; q < kChunks; ++q) store_chunk(st, q);
  };

  int is_m0, is_n0, is_k0 = 0;  // operands of the step most recently loaded
  {
    bool interior;
    tile_origin<T>(lid, tiles_m, tiles_n, is_m0, is_n0, interior, p);
  }
  write_guarded(lds, is_m0, is_n0, 0);
  int stage = 0;

  f32x4 acc[W::TBM][W::TBN];
  for (int t = 0; t < my_tiles; ++t) {
    const int cur_m0 = is_m0, cur_n0 = is_n0;
    int nt_m0, nt_n0;
    {
      bool interior;
      tile_origin<T>(lid + (t + 1 < my_tiles ? t + 1 : t) * G, tiles_m, tiles_n, nt_m0, nt_n0,
                     interior, p);
    }
#pragma unroll
    for (int i = 0; i < W::TBM; ++i)
#pragma unroll
      for (int j = 0; j < W::TBN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kk = 0; kk < nk; ++kk) {
      const bool last = kk + 1 == nk;
      is_m0 = last ? nt_m0 : cur_m0;
      is_n0 = last ? nt_n0 : cur_n0;
      is_k0 = last ? 0 : is_k0 + W::BK;
      ks_lds_barrier();  // this stage written by every wave; the other one free
      const float *st = lds + stage * W::STAGE;
      float *nst = lds + (stage ^ 1) * W::STAGE;
      load_setup(is_m0, is_n0, is_k0);

      // As big16_kernel, with register loads and LDS writes of the next
      // step in place of its direct loads: one 128-bit load after each of
      // the step's first rows of 8 MFMAs (from the second on), one LDS
      // write after every second row of its second half.
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
        f32x4(&acur)[W::TBM] = (h & 1) ? a1 : a0;
        f32x4(&anext)[W::TBM] = (h & 1) ? a0 : a1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int grp = 4 * h + u;
          float(&bcur)[W::TBN] = (grp & 1) ? b1 : b0;
          float(&bnext)[W::TBN] = (grp & 1) ? b0 : b1;
#pragma unroll
          for (int bm = 0; bm < W::TBM; ++bm) {
#pragma unroll
            for (int bn = 0; bn < W::TBN; ++bn)
              acc[bm][bn] = __builtin_amdgcn_mfma_f32_16x16x4f32(bcur[bn], acur[bm][u],
                                                                 acc[bm][bn], 0, 0, 0);
            const int lrow = grp * W::TBM + bm - 1;
            if (lrow >= 0 && lrow < kChunks) {
              __builtin_amdgcn_sched_barrier(0);
              load_chunk(lrow);
              __builtin_amdgcn_sched_barrier(0);
            }
            constexpr int kRowsPerWrite = 2;
            constexpr int kFirstRow = 2 * W::NQ * W::TBM;  // the step's second half
            const int row = grp * W::TBM + bm - kFirstRow;
            if (row >= 0 && row % kRowsPerWrite == 0 && row / kRowsPerWrite < kChunks) {
              __builtin_amdgcn_sched_barrier(0);
              store_chunk(nst, row / kRowsPerWrite);
              __builtin_amdgcn_sched_barrier(0);
            }
            if (bm == W::TBM / 2 - 1) {
              __builtin_amdgcn_sched_barrier(0);
              if (u < 3)
                w16_read_b<W>(bnext, st, h, u + 1, lane, wn);
              else if (h + 1 < W::NQ)
                w16_read_b<W>(bnext, st, h + 1, 0, lane, wn);
              if (u == 1 && h + 1 < W::NQ) w16_read_a<W>(anext, st, h + 1, lane, wm);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      // The stage just written holds a partial step: rewrite it zero-filled
      // (same thread, same addresses, so the rewrite lands last).
      if (k_tail && kk + 2 == nk) write_guarded(nst, is_m0, is_n0, is_k0);
      stage ^= 1;
      // accumulators handed on in accumulation registers (see big16_kernel)
#pragma unroll
      for (int i = 0; i < W::TBM; ++i)
#pragma unroll
        for (int j = 0; j < W::TBN; ++j) asm volatile("" : "+a"(acc[i][j]));
    }

    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int bm = 0; bm < W::TBM; ++bm) {
      float *crow = p.C + (long long)(cur_m0 + wm * W::WTM + 16 * bm + l16) * p.ldc + cur_n0 +
                    wn * W::WTN + 4 * g;
#pragma unroll
      for (int bn = 0; bn < W::TBN; ++bn)
        *reinterpret_cast<f32x4u *>(crow + 16 * bn) = acc[bm][bn];
    }
  }
}

// Small-K kernel: the whole K (<= BK) of a tile fits one LDS stage, so each
// iteration of the persistent loop is one complete tile.  It covers only
// whole tiles (the launcher sends edge strips to the k-loop kernel), which
// keeps the loop straight-line.  Order per tile: issue the next tile's loads
// into registers, run all MFMAs, issue this tile's TM*TN*4 C stores per
// lane, barrier (every wave done reading LDS), wait until at most those
// stores are outstanding -- the vector-memory counter retires in issue
// order, so this waits for the loads but leaves the stores draining while
// the next tile computes -- write the stage, barrier.  The last iteration
// reloads its own tile so every iteration has the same shape.
template <class S, bool KFULL>
__global__ void __launch_bounds__(S::NT)
    panel_kernel(Problem p, int tiles_m, int tiles_n) {
  static_assert((S::A_STAGE + S::B_STAGE) * 4 <= kLdsBytes, "stage must fit in LDS");
  __shared__ __attribute__((aligned(16))) float lds[S::A_STAGE + S::B_STAGE];
  float *const as = lds;
  float *const bs = lds + S::A_STAGE;
  constexpr int kStoresPerTile = S::TM * S::TN * 4;
  static_assert(kStoresPerTile < 64, "vmcnt holds at most 63");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int ntiles = tiles_m * tiles_n;
  const int G = gridDim.x;
  const int lid = xcd_remap(blockIdx.x, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int my_tiles = (ntiles - lid + G - 1) / G;

  int t = lid, m0, n0;
  bool interior;  // always true: the launcher passes whole tiles only
  tile_origin<S>(t, tiles_m, tiles_n, m0, n0, interior, p);
  Stage<S> st;
  load_global<S, !KFULL>(st, p, m0, n0, 0, tid);
  store_lds_as<S, !KFULL>(st, as, bs, tid);
  __syncthreads();

  for (int i = 0; i < my_tiles; ++i) {
    const int tnext = i + 1 < my_tiles ? t + G : t;
    int nm0, nn0;
    tile_origin<S>(tnext, tiles_m, tiles_n, nm0, nn0, interior, p);
    load_global<S, !KFULL>(st, p, nm0, nn0, 0, tid);
    // Keep the loads ahead of the MFMAs so their latency hides under them.
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc[S::TM][S::TN];
#pragma unroll
    for (int a = 0; a < S::TM; ++a)
#pragma unroll
      for (int b = 0; b < S::TN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    compute_stage<S>(acc, as, bs, wm, wn, lane);
    store_c<S>(acc, p, m0, n0, wm, wn, lane, false);
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(kStoresPerTile));
    store_lds_as<S, !KFULL>(st, as, bs, tid);
    __syncthreads();
    t = tnext;
    m0 = nm0;
    n0 = nn0;
  }
}

// One tile of the pipelined small-K kernel: issue the next tile's loads,
// run this tile's MFMAs into `acc` while the previous tile's results in
// `prev` go out as C stores, one store after every 8 MFMAs (the ratio of a
// 64 x 64 wave tile at K = 64), then refill the stage.  Stores that drain
// beside matrix work instead of in a burst after it keep the store path
// busy through the whole tile.
template <class S, bool KFULL, bool STORE>
__device__ __forceinline__ void panel_pipe_step(f32x16 (&acc)[S::TM][S::TN],
                                                const f32x16 (&prev)[S::TM][S::TN],
                                                const Problem &p, int pm0, int pn0, int nm0,
                                                int nn0, Stage<S> &st, float *as, float *bs,
                                                int wm, int wn, int lane, int tid) {
  constexpr int kStores = S::TM * S::TN * 4;
  constexpr int kMfmas = S::TM * S::TN * (S::BK / 2);
  static_assert(kMfmas % kStores == 0, "MFMAs must split evenly between stores");
  load_global<S, !KFULL>(st, p, nm0, nn0, 0, tid);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int a = 0; a < S::TM; ++a)
#pragma unroll
    for (int b = 0; b < S::TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  compute_stage<S>(acc, as, bs, wm, wn, lane);
  if constexpr (STORE) {
    store_c<S>(prev, p, pm0, pn0, wm, wn, lane, false);
#pragma unroll
    for (int g = 0; g < kStores; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, kMfmas / kStores, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);                 // VMEM write
    }
  }
  __syncthreads();
  // Loads done; this tile's stores (issued after them) may still drain.
  __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(STORE ? kStores : 0));
  store_lds_as<S, !KFULL>(st, as, bs, tid);
  __syncthreads();
}

// Small-K kernel with the C stores of tile i interleaved into the MFMAs of
// tile i + 1 (two accumulator sets, alternating; the loop is unrolled by two
// so each set has fixed registers).  Otherwise as panel_kernel: whole tiles
// only, persistent, the last tile reloads itself.
template <class S, bool KFULL>
__global__ void __launch_bounds__(S::NT)
    panel_pipe_kernel(Problem p, int tiles_m, int tiles_n) {
  static_assert((S::A_STAGE + S::B_STAGE) * 4 <= kLdsBytes, "stage must fit in LDS");
  __shared__ __attribute__((aligned(16))) float lds[S::A_STAGE + S::B_STAGE];
  float *const as = lds;
  float *const bs = lds + S::A_STAGE;
  static_assert(S::TM * S::TN * 4 < 64, "vmcnt holds at most 63");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int ntiles = tiles_m * tiles_n;
  const int G = gridDim.x;
  const int lid = xcd_remap(blockIdx.x, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int n = (ntiles - lid + G - 1) / G;  // this workgroup's tiles: lid, lid + G, ...

  bool interior;  // always true: the launcher passes whole tiles only
  int m0, n0;
  tile_origin<S>(lid, tiles_m, tiles_n, m0, n0, interior, p);
  Stage<S> st;
  load_global<S, !KFULL>(st, p, m0, n0, 0, tid);
  store_lds_as<S, !KFULL>(st, as, bs, tid);
  __syncthreads();

  f32x16 acc0[S::TM][S::TN], acc1[S::TM][S::TN];
  // Tile i sits in LDS; (m0, n0) is its origin, (pm0, pn0) the previous one.
  int pm0 = m0, pn0 = n0, nm0, nn0;
  tile_origin<S>(n > 1 ? lid + G : lid, tiles_m, tiles_n, nm0, nn0, interior, p);
  panel_pipe_step<S, KFULL, false>(acc0, acc0, p, 0, 0, nm0, nn0, st, as, bs, wm, wn, lane, tid);
  int i = 1;
  for (; i + 1 < n; i += 2) {
    pm0 = m0, pn0 = n0, m0 = nm0, n0 = nn0;
    tile_origin<S>(lid + (i + 1) * G, tiles_m, tiles_n, nm0, nn0, interior, p);
    panel_pipe_step<S, KFULL, true>(acc1, acc0, p, pm0, pn0, nm0, nn0, st, as, bs, wm, wn, lane,
                                    tid);
    pm0 = m0, pn0 = n0, m0 = nm0, n0 = nn0;
    tile_origin<S>(i + 2 < n ? lid + (i + 2) * G : lid + (i + 1) * G, tiles_m, tiles_n, nm0,
                   nn0, interior, p);
    panel_pipe_step<S, KFULL, true>(acc0, acc1, p, pm0, pn0, nm0, nn0, st, as, bs, wm, wn, lane,
                                    tid);
  }
  if (i < n) {  // one tile left: compute it while the previous one drains
    pm0 = m0, pn0 = n0, m0 = nm0, n0 = nn0;
    panel_pipe_step<S, KFULL, true>(acc1, acc0, p, pm0, pn0, m0, n0, st, as, bs, wm, wn, lane,
                                    tid);
    store_c<S>(acc1, p, m0, n0, wm, wn, lane, false);
  } else {
    store_c<S>(acc0, p, m0, n0, wm, wn, lane, false);
  }
}

// One column tile of the A-resident small-K kernel: load the next tile's B
// (the last tile reloads its own, so every step has the same shape), run
// the first half of this tile's MFMAs from the resident A and B buffer `cur`
// into `acc` while `prev` goes out as C stores (one per 4 MFMAs), write the
// next B into the other buffer -- last read before the previous barrier --
// run the second half, and synchronise.
template <class S, bool KFULL, bool STORE>
__device__ __forceinline__ void panel_arow_step(f32x16 (&acc)[S::TM][S::TN],
                                                const f32x16 (&prev)[S::TM][S::TN],
                                                const Problem &p, int m0, int pn0, int nn0,
                                                Stage<S> &st, const float *as, const float *bcur,
                                                float *bnext, int wm, int wn, int lane,
                                                int tid) {
  constexpr int kStores = S::TM * S::TN * 4;
  constexpr int kMfmas = S::TM * S::TN * (S::BK / 2);
  static_assert(kMfmas % kStores == 0, "MFMAs must split evenly between stores");
  load_global<S, !KFULL, false, true>(st, p, m0, nn0, 0, tid);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int a = 0; a < S::TM; ++a)
#pragma unroll
    for (int b = 0; b < S::TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  compute_stage<S, 0, S::BK / 16>(acc, as, bcur, wm, wn, lane);
  if constexpr (STORE) {
    store_c<S>(prev, p, m0, pn0, wm, wn, lane, false);
#pragma unroll
    for (int g = 0; g < kStores; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, kMfmas / kStores / 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);                     // VMEM write
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // The B loads are done; the stores issued after them may still drain.
  __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(STORE ? kStores : 0));
  store_lds_as<S, !KFULL, false, true>(st, nullptr, bnext, tid);
  compute_stage<S, S::BK / 16, S::BK / 8>(acc, as, bcur, wm, wn, lane);
  __syncthreads();
}

// Small-K kernel with A resident in LDS.  Workgroup (panel, chunk) owns the
// BM rows of panel `panel` -- all of K (<= BK), loaded once -- and the chunk
// of BN-column tiles [t0, t1) of that panel.  Per tile only B moves (one of
// two LDS buffers, written while the other is read), so a tile costs one
// barrier and a third of the staging traffic of panel_pipe_kernel; C stores
// drain during the next tile's MFMAs as there.  Whole tiles only.
template <class S, bool KFULL>
__global__ void __launch_bounds__(S::NT)
    panel_arow_kernel(Problem p, int panels, int chunks, int tiles_n) {
  static_assert((S::A_STAGE + 2 * S::B_STAGE) * 4 <= kLdsBytes, "A and two B buffers must fit");
  __shared__ __attribute__((aligned(16))) float lds[S::A_STAGE + 2 * S::B_STAGE];
  float *const as = lds;
  float *const bs0 = lds + S::A_STAGE;
  float *const bs1 = bs0 + S::B_STAGE;
  static_assert(S::TM * S::TN * 4 < 64, "vmcnt holds at most 63");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int panel = lid / chunks, chunk = lid % chunks;
  if (panel >= panels) return;  // uniform per workgroup
  const int t0 = (int)((long long)chunk * tiles_n / chunks);
  const int t1 = (int)((long long)(chunk + 1) * tiles_n / chunks);
  const int n = t1 - t0;  // >= 1: the launcher keeps chunks <= tiles_n
  const int m0 = panel * S::BM;

  Stage<S> st;
  load_global<S, !KFULL>(st, p, m0, (t0 + panel % n) * S::BN, 0, tid);
  store_lds_as<S, !KFULL>(st, as, bs0, tid);
  __syncthreads();

  f32x16 acc0[S::TM][S::TN], acc1[S::TM][S::TN];
  // The i-th tile of this workgroup (in buffer i % 2) is column tile
  // t0 + (i + rot) % n: workgroups start their runs at different columns so
  // that the C rows written at any one time spread over all of C's columns
  // (in lockstep every workgroup would write the same few columns, whose
  // rows lie 4N bytes apart on a few memory channels).
  const int rot = panel % n;
  auto col = [&](int i) {
    const int k = i < n ? i : n - 1;
    return (t0 + (k + rot) % n) * S::BN;
  };
  panel_arow_step<S, KFULL, false>(acc0, acc0, p, m0, 0, col(1), st, as, bs0, bs1, wm, wn,
                                   lane, tid);
  int i = 1;
  for (; i + 1 < n; i += 2) {
    panel_arow_step<S, KFULL, true>(acc1, acc0, p, m0, col(i - 1), col(i + 1), st, as, bs1,
                                    bs0, wm, wn, lane, tid);
    panel_arow_step<S, KFULL, true>(acc0, acc1, p, m0, col(i), col(i + 2), st, as, bs0, bs1, wm,
                                    wn, lane, tid);
  }
  if (i < n) {  // one tile left, in buffer 1: compute it while the previous one drains
    panel_arow_step<S, KFULL, true>(acc1, acc0, p, m0, col(i - 1), col(i), st, as, bs1, bs0, wm,
                                    wn, lane, tid);
    store_c<S>(acc1, p, m0, col(i), wm, wn, lane, false);
  } else {
    store_c<S>(acc0, p, m0, col(i - 1), wm, wn, lane, false);
  }
}

// ---- A-resident small-K kernel on 16x16 MFMAs, one wave per SIMD ---------
// The skinny product's recipe (A panel resident, only B moves per column
// tile, C stores of one tile drained during the next tile's MFMAs) on the
// 128x128-wave kernel's machinery: a 256x128 tile over 4 waves (2 x 2),
// each computing 128x64 as 8 x 4 blocks of v_mfma_f32_16x16x4_f32 -- 32
// chains and 128 accumulators per set, two sets (256 accumulation
// registers) so that tile i computes into one set while tile i - 1 leaves
// from the other.  K is exactly 64.  LDS: the 256x64 A panel (64 KB, rows of
// 16 chunks at c ^ (r & 15)) loaded once, and two 64x128 B buffers (32 KB
// each, chunks of k row k at c ^ (4 ((k >> 2) & 3))), all by direct loads.
// Per tile a wave issues 512 MFMAs against 8 direct loads (the next tile's
// B, in the first rows), 32 C stores (spread over the rest) and one
// barrier; the wait before it lets the stores drain (the vector-memory
// counter retires in issue order and the loads went first).
struct Arow16 {
  static constexpr int WTM = 128, WTN = 64, BK = 64;
  static constexpr int BM = 2 * WTM, BN = 2 * WTN;
  static constexpr int TBM = WTM / 16, TBN = WTN / 16;
  static constexpr int NQ = BK / 16;
  static constexpr int ACH = BK / 4, BCH = BN / 4;
  static constexpr int A_FLOATS = BM * BK, B_FLOATS = BK * BN;
  static constexpr int A_DMA = A_FLOATS / 1024;  // per wave: (A_FLOATS * 4 / 1024) / 4
  static constexpr int B_DMA = B_FLOATS / 1024;
  static constexpr int STORES = TBM * TBN;  // 16-byte stores per lane and tile
  static_assert((A_FLOATS + 2 * B_FLOATS) * 4 <= kLdsBytes, "A and two B buffers fit");
  static_assert(STORES + B_DMA < 64, "vmcnt holds at most 63");
};

using Acc16 = f32x4[Arow16::TBM][Arow16::TBN];

__device__ inline void arow16_store(const Acc16 &acc, const Problem &p, int m0, int n0, int wm,
                                    int wn, int lane, int i) {
  const int l16 = lane & 15, g = lane >> 4;
  const int bm = i / Arow16::TBN, bn = i % Arow16::TBN;
  float *dst = p.C + (long long)(m0 + wm * Arow16::WTM + 16 * bm + l16) * p.ldc + n0 +
               wn * Arow16::WTN + 16 * bn + 4 * g;
  *reinterpret_cast<f32x4 *>(dst) = acc[bm][bn];
}

// One column tile: MFMAs of tile n0 from B buffer `buf` into `acc` (zeroed
// first), the next tile's B (column nn0) into the other buffer, and, with
// STORE, the previous tile (column pn0, in `prev`) out to C.
// Fragment reads from per-lane LDS pointers with the rest of each address
// a constant: a[h] points at the A chunk h of row block 0 (row block bm is
// bm * 1024 floats further), b[bn] at B column block bn, k row 4 g, of
// buffer 0 (k row 16 h + t is (16 h + t) * BN floats further, buffer 1
// B_FLOATS further).
struct Arow16Lane {
  const float *a[Arow16::NQ];
  const float *b[Arow16::TBN];
};

__device__ inline Arow16Lane arow16_lane(const float *lds, int lane, int wm, int wn) {
  using W = Arow16;
  const int l16 = lane & 15, g = lane >> 4;
  Arow16Lane o;
#pragma unroll
  for (int h = 0; h < W::NQ; ++h)
    o.a[h] = lds + 4 * w16_a_pos<W::ACH>(wm * W::WTM + l16, 4 * h + g);
#pragma unroll
  for (int bn = 0; bn < W::TBN; ++bn) {
    const int n = wn * W::WTN + 16 * bn + l16;
    o.b[bn] = lds + W::A_FLOATS + 4 * w16_b_pos<W::BCH>(4 * g, n >> 2) + (n & 3);
  }
  return o;
}

template <int H, int BUF>
__device__ inline void arow16_read_a(f32x4 (&a)[Arow16::TBM], const Arow16Lane &o) {
#pragma unroll
  for (int bm = 0; bm < Arow16::TBM; ++bm)
    a[bm] = *reinterpret_cast<const f32x4 *>(o.a[H] + bm * 1024);
}
template <int KROW, int BUF>
__device__ inline void arow16_read_b(float (&b)[Arow16::TBN], const Arow16Lane &o) {
#pragma unroll
  for (int bn = 0; bn < Arow16::TBN; ++bn)
    b[bn] = o.b[bn][KROW * Arow16::BN + BUF * Arow16::B_FLOATS];
}

template <bool STORE, int BUF>
__device__ __forceinline__ void arow16_tile(Acc16 &acc, Acc16 &prev, const Problem &p,
                                            int m0, int pn0, int nn0, const float *lds,
                                            unsigned lds_u, const unsigned (&voff)[Arow16::B_DMA],
                                            const Arow16Lane &o, int wave, int wm, int wn,
                                            int lane) {
  constexpr int buf = BUF;
  using W = Arow16;
  const float *bsrc = p.B + nn0;
  const unsigned bdst = lds_u + (W::A_FLOATS + (buf ^ 1) * W::B_FLOATS) * 4 + wave * W::B_DMA * 1024;
  f32x4 a0[W::TBM], a1[W::TBM];
  float b0[W::TBN], b1[W::TBN];
  arow16_read_b<0, BUF>(b0, o);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int bm = 0; bm < W::TBM; ++bm) {
    a0[bm] = *reinterpret_cast<const f32x4 *>(o.a[0] + bm * 1024);
    __builtin_amdgcn_sched_barrier(0);
  }
  auto mfma_rows = [&](auto hc, auto uc, f32x4(&acur)[W::TBM], f32x4(&anext)[W::TBM],
                       float(&bcur)[W::TBN], float(&bnext)[W::TBN]) __attribute__((always_inline)) {
    constexpr int h = decltype(hc)::value, u = decltype(uc)::value;
    constexpr int grp = 4 * h + u;
#pragma unroll
    for (int bm = 0; bm < W::TBM; ++bm) {
#pragma unroll
      for (int bn = 0; bn < W::TBN; ++bn)
        mfma_inplace<grp == 0>(acc[bm][bn], bcur[bn], acur[bm][u]);
      // rows of 4 MFMAs: the next B's direct loads after rows 0, 2, ..,
      // then one C store after every third row
      const int row = grp * W::TBM + bm;
      if (row % 2 == 0 && row / 2 < W::B_DMA) {
        __builtin_amdgcn_sched_barrier(0);
        ks_load_to_lds16(voff[row / 2], bsrc, bdst + (row / 2) * 1024);
        __builtin_amdgcn_sched_barrier(0);
      }
      constexpr int kFirstStoreRow = 2 * W::B_DMA;
      const int srow = row - kFirstStoreRow;
      if (STORE && srow >= 0 && srow % 3 == 0 && srow / 3 < W::STORES) {
        __builtin_amdgcn_sched_barrier(0);
        arow16_store(prev, p, m0, pn0, wm, wn, lane, srow / 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (bm == W::TBM / 2 - 1) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (u < 3)
          arow16_read_b<16 * h + u + 1, BUF>(bnext, o);
        else if constexpr (h + 1 < W::NQ)
          arow16_read_b<16 * (h + 1), BUF>(bnext, o);
        if constexpr (u == 1 && h + 1 < W::NQ)
          arow16_read_a<(h + 1 < W::NQ ? h + 1 : 0), BUF>(anext, o);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  static_assert(W::NQ == 4, "four 16-deep chunks");
  mfma_rows(I0{}, I0{}, a0, a1, b0, b1);
  mfma_rows(I0{}, I1{}, a0, a1, b1, b0);
  mfma_rows(I0{}, I2{}, a0, a1, b0, b1);
  mfma_rows(I0{}, I3{}, a0, a1, b1, b0);
  mfma_rows(I1{}, I0{}, a1, a0, b0, b1);
  mfma_rows(I1{}, I1{}, a1, a0, b1, b0);
  mfma_rows(I1{}, I2{}, a1, a0, b0, b1);
  mfma_rows(I1{}, I3{}, a1, a0, b1, b0);
  mfma_rows(I2{}, I0{}, a0, a1, b0, b1);
  mfma_rows(I2{}, I1{}, a0, a1, b1, b0);
  mfma_rows(I2{}, I2{}, a0, a1, b0, b1);
  mfma_rows(I2{}, I3{}, a0, a1, b1, b0);
  mfma_rows(I3{}, I0{}, a1, a0, b0, b1);
  mfma_rows(I3{}, I1{}, a1, a0, b1, b0);
  mfma_rows(I3{}, I2{}, a1, a0, b0, b1);
  mfma_rows(I3{}, I3{}, a1, a0, b1, b0);
  // 24 wait states after the last MFMA before anything may read its result
  // (mfma_inplace).
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
  // The next B is in (own loads; the stores issued after them may drain),
  // then every wave's, and every wave is done with this buffer.
  __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(STORE ? W::STORES : 0));
  ks_lds_barrier();
#pragma unroll
  for (int i = 0; i < W::TBM; ++i)
#pragma unroll
    for (int j = 0; j < W::TBN; ++j) {
      asm volatile("" : "+a"(acc[i][j]));
      asm volatile("" : "+a"(prev[i][j]));
    }
}

// Workgroup (panel, chunk) owns rows [256 panel, +256) and the column tiles
// [t0, t1) of that panel, walked from a rotated start as in
// panel_arow_kernel.  Each XCD's run of logical ids (xcd_remap) covers 8
// panels and all their chunks.  Giving an XCD one chunk of B instead (ids
// panel-fastest) does not keep that 1 MB chunk in the XCD's L2: the C
// stores stream through L2 and evict it, and on 16384 x 16384 x 64 the L2
// read traffic rose from 246 to 277 MB with no change in time.  The launcher
// guarantees K == 64, M % 256 == 0, N % 128 == 0, 16-byte aligned rows of A
// and B and byte offsets below 2^32 (rows of 256 A rows and 64 B rows).
__global__ void __launch_bounds__(256) arow16_kernel(Problem p, int panels, int chunks,
                                                     int tiles_n) {
  using W = Arow16;
  __shared__ __attribute__((aligned(16))) float lds[W::A_FLOATS + 2 * W::B_FLOATS];
  const unsigned lds_u = (unsigned)(uintptr_t)(lds_void_t *)lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int panel = lid / chunks, chunk = lid % chunks;
  if (panel >= panels) return;  // uniform per workgroup
  const int t0 = (int)((long long)chunk * tiles_n / chunks);
  const int t1 = (int)((long long)(chunk + 1) * tiles_n / chunks);
  const int n = t1 - t0;  // >= 1: the launcher keeps chunks <= tiles_n
  const int m0 = panel * W::BM;
  const int rot = panel % n;
  auto col = [&](int i) __attribute__((always_inline)) {
    const int k = i < n ? i : n - 1;
    return (t0 + (k + rot) % n) * W::BN;
  };

  // Direct-load offsets: the A panel (once) and a B tile (per tile).
  unsigned voff[W::B_DMA];
#pragma unroll
  for (int q = 0; q < W::B_DMA; ++q)
    voff[q] = (unsigned)(dma_b_elem<W::BCH>(64 * (wave * W::B_DMA + q) + lane, p.ldb) * 4);
  {
    const float *asrc = p.A + (long long)m0 * p.lda;
#pragma unroll
    for (int q = 0; q < W::A_DMA; ++q) {
      const int blk = wave * W::A_DMA + q;
      ks_load_to_lds16((unsigned)(dma_a_elem<W::ACH>(blk, lane, p.lda) * 4), asrc,
                       lds_u + blk * 1024);
    }
    const float *bsrc = p.B + col(0);
#pragma unroll
    for (int q = 0; q < W::B_DMA; ++q)
      ks_load_to_lds16(voff[q], bsrc, lds_u + W::A_FLOATS * 4 + (wave * W::B_DMA + q) * 1024);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));
    ks_lds_barrier();
  }

  const Arow16Lane o = arow16_lane(lds, lane, wm, wn);
  Acc16 acc0, acc1;
  arow16_tile<false, 0>(acc0, acc0, p, m0, 0, col(1), lds, lds_u, voff, o, wave, wm, wn, lane);
  int i = 1;
  for (; i + 1 < n; i += 2) {
    arow16_tile<true, 1>(acc1, acc0, p, m0, col(i - 1), col(i + 1), lds, lds_u, voff, o, wave,
                         wm, wn, lane);
    arow16_tile<true, 0>(acc0, acc1, p, m0, col(i), col(i + 2), lds, lds_u, voff, o, wave, wm,
                         wn, lane);
  }
  if (i < n) {  // one tile left, in buffer 1: compute it while the previous one drains
    arow16_tile<true, 1>(acc1, acc0, p, m0, col(i - 1), col(i), lds, lds_u, voff, o, wave, wm,
                         wn, lane);
#pragma unroll
    for (int q = 0; q < W::STORES; ++q) arow16_store(acc1, p, m0, col(i), wm, wn, lane, q);
  } else {
#pragma unroll
    for (int q = 0; q < W::STORES; ++q) arow16_store(acc0, p, m0, col(i - 1), wm, wn, lane, q);
  }
}

// Thin-M kernel for a strip of at most 32 rows: a bottom remainder strip, or
// a whole product of that few rows (a 64- to 256-row MFMA tile holding 1 to
// 32 valid rows would cost a whole tile's work per column block).  Its
// time is the stream of B, read once: each workgroup owns 16 columns, and
// its 512 threads are 4 column quads x 128 k-slices; slice s takes the
// quads of consecutive k starting at 4 s, 4 s + 512, ..., so a lane loads
// 4 B rows of its 4 columns and one 16-byte chunk per A row per quad.  A
// lane issues the loads of NB quads before it uses any of them (a loop
// whose every iteration may exit would wait for each load in turn, one
// memory round trip per quad); the last quads of a lane, any of them past
// K, go in one guarded batch.  Workgroups are dealt to the XCDs so that
// each XCD streams one contiguous band of B's columns, and the 128-byte
// lines that neighbouring 64-byte column groups share are fetched into one
// L2.  Each thread accumulates its R x 4 outputs in fp32 over its slice in
// ascending k; the 16 slices of a wave are added by a fixed butterfly of
// lane exchanges and the 8 waves' sums in wave order through LDS, so the
// result is deterministic.  Rows of A and B need only 4-byte alignment.
constexpr int kStripThreads = 512;
constexpr int kStripCols = 16;
constexpr int kStripSlices = kStripThreads / (kStripCols / 4);
constexpr int kStripWaves = kStripThreads / 64;

template <int R, int NB>
__global__ void __launch_bounds__(kStripThreads) strip_kernel(Problem p) {
  constexpr int KB = 4 * kStripSlices;  // k per quad round of the workgroup
  constexpr int RS = R <= 16 ? R : 8;   // rows whose A chunks a lane holds at once
  __shared__ float red[kStripWaves][R][kStripCols];
  const int tid = threadIdx.x;
  const int c4 = (tid & 3) * 4;  // first of this lane's 4 columns
  const int k0 = 4 * (tid >> 2);  // first k of this lane's first quad
  const long long n0 = (long long)xcd_remap(blockIdx.x, gridDim.x) * kStripCols;
  float acc[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[r][j] = 0.f;
  // Rows past M read row M - 1 (never stored), so no load is conditional.
  // Row starts are formed where they are used (32 held pointers would take
  // 64 registers).
  auto arow = [&](int r) __attribute__((always_inline)) {
    return p.A + (long long)(r < p.M ? r : p.M - 1) * p.lda;
  };
  const bool whole = n0 + kStripCols <= p.N;
  const int valid = (int)(p.N - n0) - c4;  // columns of this lane inside C (whole: >= 4)
  const float *bp = p.B + n0 + c4;
  auto load_b = [&](int k) __attribute__((always_inline)) {
    f32x4 v;
    if (whole) {
      v = *reinterpret_cast<const f32x4u *>(bp + (long long)k * p.ldb);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = j < valid ? bp[(long long)k * p.ldb + j] : 0.f;
    }
    return v;
  };
  int k = k0;
  // Whole batches: NB quads, every k inside K.  Rows go in sets of RS (all
  // R up to 16 rows; four sets of 8 for 32), each set's A chunks loaded
  // after the previous set's FMAs, so that the 32-row form fits its
  // registers beside its 128 accumulators.
  for (; k + (NB - 1) * KB + 3 < p.K; k += NB * KB) {
    f32x4 b[NB][4];
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) b[u][t] = load_b(k + u * KB + t);
#pragma unroll
    for (int r0 = 0; r0 < R; r0 += RS) {
      f32x4 a[NB][RS];
#pragma unroll
      for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int r = 0; r < RS; ++r)
          a[u][r] = *reinterpret_cast<const f32x4u *>(arow(r0 + r) + k + u * KB);
#pragma unroll
      for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < RS; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[r0 + r][j] += a[u][r][t] * b[u][t][j];
      // keep the next set's loads after these FMAs
      if constexpr (RS < R) __builtin_amdgcn_sched_barrier(0);
    }
  }
  // The rest of this slice (fewer than NB quads, the last possibly partial):
  // one batch, k past K loading row K - 1 and adding nothing.
  if (k < p.K) {
    f32x4 b[NB][4];
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kk = k + u * KB + t;
        b[u][t] = load_b(kk < p.K ? kk : p.K - 1);
      }
#pragma unroll
    for (int r0 = 0; r0 < R; r0 += RS) {
      f32x4 a[NB][RS];
#pragma unroll
      for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kk = k + u * KB + t;
          const int kc = kk < p.K ? kk : p.K - 1;
#pragma unroll
          for (int r = 0; r < RS; ++r) a[u][r][t] = arow(r0 + r)[kc];
        }
#pragma unroll
      for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (k + u * KB + t < p.K) {
#pragma unroll
            for (int r = 0; r < RS; ++r)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[r0 + r][j] += a[u][r][t] * b[u][t][j];
          }
      if constexpr (RS < R) __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Slices of one wave: lanes 4 s + q (s = 0..15) hold column quad q.  Row
  // by row, so that few exchanged values are in flight at once.
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int m = 4; m < 64; m <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[r][j] += __shfl_xor(acc[r][j], m);
    if constexpr (RS < R) __builtin_amdgcn_sched_barrier(0);
  }
  const int wave = tid >> 6;
  if ((tid & 63) < 4) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][r][c4 + j] = acc[r][j];
  }
  __syncthreads();
  if (tid < kStripCols * R) {
    const int r = tid / kStripCols, c = tid % kStripCols;
    if (r < p.M && n0 + c < p.N) {
      float sum = red[0][r][c];
#pragma unroll
      for (int w = 1; w < kStripWaves; ++w) sum += red[w][r][c];
      p.C[(long long)r * p.ldc + n0 + c] = sum;
    }
  }
}

hipError_t launch_strip(const Problem &p, hipStream_t s) {
  if (p.M < 1 || p.M > kStripMaxRows) return hipErrorInvalidValue;
  const dim3 grid((unsigned)ceil_div(p.N, kStripCols)), block(kStripThreads);
  switch (strip_rows(p.M)) {
    case 1: return launch_kernel(strip_kernel<1, strip_batch_quads(1)>, grid, block, s, p);
    case 2: return launch_kernel(strip_kernel<2, strip_batch_quads(2)>, grid, block, s, p);
    case 4: return launch_kernel(strip_kernel<4, strip_batch_quads(4)>, grid, block, s, p);
    case 8: return launch_kernel(strip_kernel<8, strip_batch_quads(8)>, grid, block, s, p);
    case 16: return launch_kernel(strip_kernel<16, strip_batch_quads(16)>, grid, block, s, p);
    default: return launch_kernel(strip_kernel<32, strip_batch_quads(32)>, grid, block, s, p);
  }
}


// Thin-N kernel for a whole product of at most 16 columns: a stream of A,
// read once (a 64- to 256-column MFMA tile holding one to eight valid
// columns would cost a whole tile's work per row block).  A workgroup of
// 512 threads owns 16 rows of C: 8 lanes per row read 128 consecutive bytes
// of it per load (one 16-byte quad of k each), the two row halves take one
// wave each, and 4 wave pairs split k (pair s takes k = 128 j + 32 s + 4 q
// for lane q of a row), so at each step a workgroup reads 512 bytes of each
// of its rows.  B goes through LDS a chunk of KC k at a time (1024, or 512
// for 16 columns), quad of k by quad of k: the 4 x NC values of a quad as
// NC runs of 4 k (column n's run at 4 n), a quad's block padded to 4 NC + 4
// floats for NC >= 2 so that the 8 quads a wave reads at once fall on
// distinct banks; a lane reads one 16-byte run per column per quad.  A lane
// loads a chunk's B values and A quads together, B first, and waits for the
// B values alone before writing them to LDS.  With PREFETCH it issues the
// next chunk's loads before it computes on the current one, holding them
// in registers until the next barrier: against loading each chunk when it
// starts, 4096 x 16 x 4096 35.4 -> 28.9 us, 16384 x 16 x 4096 120.7 ->
// 107.0, 4096 x 1 x 4096 17.5 -> 16.2 (the same prefetch made the thin-M
// strip slower, 10.5 -> 12.7 us on 1 x 4095 x 2049).  The extra registers
// can halve the workgroups resident per CU (2 columns: 90 -> 142 VGPRs;
// 100000 x 2 x 512 40.5 -> 69.1 us), so the launcher takes the prefetching
// form only where that costs no residency the grid would use.  Elements
// past K or N are zeros on both
// sides, and quads wholly past K are skipped.  Each lane sums its k in
// ascending order; the 8 lanes of a row are added by a fixed butterfly of
// lane exchanges and the 4 k-splits in split order through LDS, so the
// result is deterministic.  Rows of A and B need only 4-byte alignment.
constexpr int kColThreads = 512;
constexpr int kColRows = 16;
constexpr int kColSplits = 4;
constexpr int kColStep = 4 * 8 * kColSplits;  // k per step of a row: 8 lanes x 4 k x 4 splits

template <int NC>
constexpr int col_quad_floats() {
  return NC == 1 ? 4 : 4 * NC + 4;
}

template <int NC, bool PREFETCH>
__global__ void __launch_bounds__(kColThreads) colstrip_kernel(Problem p) {
  constexpr int QF = col_quad_floats<NC>();
  constexpr int KC = col_chunk(NC), NJ = KC / kColStep;
  constexpr int BV = KC * NC / kColThreads;  // B values a thread stages per chunk
  static_assert(KC % kColStep == 0 && (KC * NC) % kColThreads == 0, "chunk shape");
  __shared__ __attribute__((aligned(16))) float bq[KC / 4 * QF];
  __shared__ float red[kColSplits][kColRows][NC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = wave >> 1;
  const int r = 8 * (wave & 1) + (lane >> 3);  // row within the workgroup
  const int q = lane & 7;
  const long long m0 = (long long)blockIdx.x * kColRows;
  // Rows past M read row M - 1 (never stored), so no A load is conditional.
  const float *arow = p.A + (m0 + r < p.M ? m0 + r : p.M - 1) * p.lda;
  float acc[NC];
#pragma unroll
  for (int n = 0; n < NC; ++n) acc[n] = 0.f;
  auto load_chunk = [&](float(&bv)[BV], f32x4(&a)[NJ], int kc0) __attribute__((always_inline)) {
    const int kn = p.K - kc0 < KC ? p.K - kc0 : KC;
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int i = tid + kColThreads * v, k = i / NC, n = i % NC;
      bv[v] = k < kn && n < p.N ? p.B[(long long)(kc0 + k) * p.ldb + n] : 0.f;
    }
    if (kn == KC) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        a[j] = *reinterpret_cast<const f32x4u *>(arow + kc0 + kColStep * j + 32 * split + 4 * q);
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int k = kc0 + kColStep * j + 32 * split + 4 * q;
        if (k + 4 <= p.K) {
          a[j] = *reinterpret_cast<const f32x4u *>(arow + k);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) a[j][t] = k + t < p.K ? arow[k + t] : 0.f;
        }
      }
    }
  };
  float bv[BV];
  f32x4 a[NJ];
  if constexpr (PREFETCH) load_chunk(bv, a, 0);
  for (int kc0 = 0; kc0 < p.K; kc0 += KC) {
    const int kn = p.K - kc0 < KC ? p.K - kc0 : KC;
    if constexpr (!PREFETCH) load_chunk(bv, a, kc0);
    __syncthreads();  // every lane is done with the previous chunk's B
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int i = tid + kColThreads * v, k = i / NC, n = i % NC;
      bq[(k >> 2) * QF + 4 * n + (k & 3)] = bv[v];
    }
    __syncthreads();
    const bool more = PREFETCH && kc0 + KC < p.K;
    f32x4 an[NJ];
    if (more) load_chunk(bv, an, kc0 + KC);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int kl = kColStep * j + 32 * split + 4 * q;
      if (kl < kn) {
#pragma unroll
        for (int n = 0; n < NC; ++n) {
          const f32x4 b = *reinterpret_cast<const f32x4 *>(bq + (kl >> 2) * QF + 4 * n);
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[n] += a[j][t] * b[t];
        }
      }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) a[j] = an[j];
    }
  }
#pragma unroll
  for (int m = 1; m < 8; m <<= 1)
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[n] += __shfl_xor(acc[n], m);
  if (q == 0) {
#pragma unroll
    for (int n = 0; n < NC; ++n) red[split][r][n] = acc[n];
  }
  __syncthreads();
  if (tid < kColRows * NC) {
    const int rr = tid / NC, n = tid % NC;
    if (m0 + rr < p.M && n < p.N) {
      float sum = red[0][rr][n];
#pragma unroll
      for (int sp = 1; sp < kColSplits; ++sp) sum += red[sp][rr][n];
      p.C[(m0 + rr) * p.ldc + n] = sum;
    }
  }
}

// The prefetching form unless it holds fewer workgroups resident than the
// plain one while the grid needs more than it holds.
template <int NC>
hipError_t launch_colstrip_nc(const Problem &p, long long wgs, hipStream_t s) {
  const dim3 grid((unsigned)wgs), block(kColThreads);
  const long long with = resident_workgroups<colstrip_kernel<NC, true>, kColThreads>();
  const long long without = resident_workgroups<colstrip_kernel<NC, false>, kColThreads>();
  if (wgs <= with || with >= without)
    return launch_kernel(colstrip_kernel<NC, true>, grid, block, s, p);
  return launch_kernel(colstrip_kernel<NC, false>, grid, block, s, p);
}

hipError_t launch_colstrip(const Problem &p, hipStream_t s) {
  if (p.N < 1 || p.N > kStripMaxCols || p.M < 1) return hipErrorInvalidValue;
  const long long wgs = ceil_div(p.M, kColRows);
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  switch (strip_cols(p.N)) {
    case 1: return launch_colstrip_nc<1>(p, wgs, s);
    case 2: return launch_colstrip_nc<2>(p, wgs, s);
    case 4: return launch_colstrip_nc<4>(p, wgs, s);
    case 8: return launch_colstrip_nc<8>(p, wgs, s);
    default: return launch_colstrip_nc<16>(p, wgs, s);
  }
}

// ---- launch table (its entries and the automatic choice: host_plan.cpp) --

using C0 = Tile<128, 128, 32, 2, 2, false>;
using C1 = Tile<128, 128, 16, 2, 2, false>;
using C2 = Tile<256, 128, 16, 4, 2, false>;
using C3 = Tile<64, 64, 32, 2, 2, false>;
using C4 = Tile<128, 64, 32, 2, 2, false>;
using C5 = Tile<128, 128, 32, 2, 2, true>;
using C6 = Tile<128, 128, 16, 2, 2, true>;
using C7 = Tile<256, 128, 32, 4, 2, false>;
using P8 = Tile<128, 128, 64, 2, 2, false>;  // small-K panel kernel, K <= 64
using P9 = Tile<256, 128, 64, 4, 2, false>;  // small-K panel kernel, K <= 64
using C10 = Tile<256, 256, 16, 4, 4, false>;
using C11 = Tile<256, 256, 16, 4, 2, false>;
using C12 = Tile<256, 256, 32, 4, 4, false>;



template <class S, void (*KERNEL)(Problem, int, int)>
hipError_t launch_grid(const Problem &p, hipStream_t s) {
  const long long tiles_m = ceil_div(p.M, S::BM), tiles_n = ceil_div(p.N, S::BN);
  const long long ntiles = tiles_m * tiles_n;
  if (ntiles > 0x7fffffffLL) return hipErrorInvalidValue;
  long long grid = resident_workgroups<KERNEL, S::NT>();
  if (grid > ntiles) grid = ntiles;
  return launch_kernel(KERNEL, dim3((unsigned)grid), dim3(S::NT), s, p,
                       (int)tiles_m, (int)tiles_n);
}

template <class S>
hipError_t launch_kloop(const Problem &p, hipStream_t s) {
  return launch_grid<S, prod_kernel<S>>(p, s);
}

// K split over the waves of a 64x64 tile when A and B rows are 16-byte
// aligned, N % 4 == 0, C is at least one tile each way and the lane offsets
// fit in 32 bits -- the whole-step form (ksplit_whole_kernel) when K is a
// multiple of 64, else ksplit_kernel; otherwise the register-staged
// 64x64x32 kernel.
hipError_t launch_ksplit(const Problem &p, hipStream_t s) {
  const bool ok = (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && (p.lda & 3) == 0 &&
                  (p.ldb & 3) == 0 && (p.N & 3) == 0 && p.M >= 64 && p.N >= 64 &&
                  lane_offsets_fit(64, p.lda, 4) && lane_offsets_fit(64, p.ldb, 4);
  if (!ok) return launch_kloop<C3>(p, s);
  const long long tiles_m = ceil_div(p.M, 64), tiles_n = ceil_div(p.N, 64);
  const long long ntiles = tiles_m * tiles_n;
  if (ntiles > 0x7fffffffLL) return hipErrorInvalidValue;
  if (p.K % 64 == 0) {
    long long grid = resident_workgroups<ksplit_whole_kernel, 256>();
    if (grid > ntiles) grid = ntiles;
    return launch_kernel(ksplit_whole_kernel, dim3((unsigned)grid), dim3(256), s, p,
                         (int)tiles_m, (int)tiles_n);
  }
  long long grid = resident_workgroups<ksplit_kernel, 256>();
  if (grid > ntiles) grid = ntiles;
  return launch_kernel(ksplit_kernel, dim3((unsigned)grid), dim3(256), s, p, (int)tiles_m,
                       (int)tiles_n);
}

// One wave per SIMD with 16x16 MFMAs (w16_kernel) when A and B rows are
// 16-byte aligned, N % 4 == 0, C is at least one tile each way and the
// lane offsets fit in 32 bits; otherwise the register-staged kernel
// FALLBACK.
template <class W, class FALLBACK>
hipError_t launch_w16(const Problem &p, hipStream_t s) {
  const bool ok = (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && (p.lda & 3) == 0 &&
                  (p.ldb & 3) == 0 && (p.N & 3) == 0 && p.M >= W::BM && p.N >= W::BN &&
                  lane_offsets_fit(W::BM, p.lda, 4) && lane_offsets_fit(W::BK, p.ldb, 4);
  if (!ok) return launch_kloop<FALLBACK>(p, s);
  const long long tiles_m = ceil_div(p.M, W::BM), tiles_n = ceil_div(p.N, W::BN);
  const long long ntiles = tiles_m * tiles_n;
  if (ntiles > 0x7fffffffLL) return hipErrorInvalidValue;
  long long grid = resident_workgroups<w16_kernel<W>, 256>();
  if (grid > ntiles) grid = ntiles;
  return launch_kernel(w16_kernel<W>, dim3((unsigned)grid), dim3(256), s, p, (int)tiles_m,
                       (int)tiles_n);
}

// The 128x128-wave kernel with direct loads (big16_kernel) when C is at
// least one tile each way, K is at least one k step (a partial last step
// takes the kernel's tail form) and the lane offsets fit in 32 bits;
// otherwise FALLBACK (for the 256x256 tiles, the same tiles staged through
// registers).  Rows need only the 4-byte alignment every call has.
using Launcher = hipError_t (*)(const Problem &, hipStream_t);
template <class W, Launcher FALLBACK>
hipError_t launch_big16(const Problem &p, hipStream_t s);

// The direct-to-LDS kernel when A and B rows are 16-byte aligned and
// N % 4 == 0; otherwise the register-staged kernel with the same tiles.
template <class S>
hipError_t launch_lds_dma16(const Problem &p, hipStream_t s) {
  const bool aligned = (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && (p.lda & 3) == 0 &&
                       (p.ldb & 3) == 0 && (p.N & 3) == 0;
  if (!aligned) return launch_kloop<S>(p, s);
  return launch_grid<S, lds_dma16_kernel<S>>(p, s);
}

template <class S>
hipError_t launch_lds_dma(const Problem &p, hipStream_t s) {
  const bool aligned = (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && (p.lda & 3) == 0 &&
                       (p.ldb & 3) == 0 && (p.N & 3) == 0;
  if (!aligned) return launch_kloop<S>(p, s);
  return launch_grid<S, lds_dma_kernel<S>>(p, s);
}

// Split-K launch: every (tile, split) pair is one workgroup (grid y = the
// split), then the reduction over the slabs into C.
hipError_t launch_splitk_reduce(const Problem &p, int splits, const float *ws, hipStream_t s);

template <class S>
hipError_t launch_split(const Problem &p, int splits, int kc, float *ws, hipStream_t s) {
  const long long tiles_m = ceil_div(p.M, S::BM), tiles_n = ceil_div(p.N, S::BN);
  const long long ntiles = tiles_m * tiles_n;
  if (ntiles > 0x7fffffffLL || splits < 1 || splits > kMaxGridY) return hipErrorInvalidValue;
  hipError_t e = launch_kernel(prod_split_kernel<S>, dim3((unsigned)ntiles, (unsigned)splits),
                               dim3(S::NT), s, p, (int)tiles_m, (int)tiles_n, kc, ws);
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(p, splits, ws, s);
}

// The slab sum into C, after the partial products.
hipError_t launch_splitk_reduce(const Problem &p, int splits, const float *ws, hipStream_t s) {
  const long long quads = (long long)p.M * ((p.N + 3) / 4);
  long long blocks = ceil_div(quads, kReduceThreads);
  if (blocks > 4096) blocks = 4096;
  return launch_kernel(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(kReduceThreads), s,
                       static_cast<const float *>(ws), splits, p.M, p.N, p.C, p.ldc);
}

// Whole tiles only: the caller (launch_prod) splits edge strips off first.
template <class S, bool PIPE = false>
hipError_t launch_panel(const Problem &p, hipStream_t s) {
  if (p.K > S::BK || p.M % S::BM != 0 || p.N % S::BN != 0) return hipErrorInvalidValue;
  if constexpr (PIPE) {
    if (p.K == S::BK) return launch_grid<S, panel_pipe_kernel<S, true>>(p, s);
    return launch_grid<S, panel_pipe_kernel<S, false>>(p, s);
  }
  if (p.K == S::BK) return launch_grid<S, panel_kernel<S, true>>(p, s);
  return launch_grid<S, panel_kernel<S, false>>(p, s);
}

// A-resident small-K launch: one workgroup per (row panel, chunk of column
// tiles), enough chunks per panel to give every resident slot a workgroup.
template <class S>
hipError_t launch_arow(const Problem &p, hipStream_t s) {
  if (p.K > S::BK || p.M % S::BM != 0 || p.N % S::BN != 0) return hipErrorInvalidValue;
  const long long panels = p.M / S::BM, tiles_n = p.N / S::BN;
  if (panels * tiles_n > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool full = p.K == S::BK;
  const long long slots = full ? resident_workgroups<panel_arow_kernel<S, true>, S::NT>()
                               : resident_workgroups<panel_arow_kernel<S, false>, S::NT>();
  long long chunks = ceil_div(slots, panels);
  if (chunks > tiles_n) chunks = tiles_n;
  if (chunks < 1) chunks = 1;
  const dim3 grid((unsigned)(panels * chunks));
  if (full)
    return launch_kernel(panel_arow_kernel<S, true>, grid, dim3(S::NT), s, p, (int)panels,
                         (int)chunks, (int)tiles_n);
  return launch_kernel(panel_arow_kernel<S, false>, grid, dim3(S::NT), s, p, (int)panels,
                       (int)chunks, (int)tiles_n);
}

// 128x128-wave tiles with register staging (big16r_kernel) when C is at
// least one tile each way and K >= 4; otherwise the register-staged 32x32
// kernel with the same tiles.
template <class W>
hipError_t launch_big16r(const Problem &p, hipStream_t s) {
  if (p.M < W::BM || p.N < W::BN || p.K < 4) return launch_kloop<C12>(p, s);
  return launch_big16_grid<W, big16r_kernel<W>>(p, s);
}

template <class W, Launcher FALLBACK>
hipError_t launch_big16(const Problem &p, hipStream_t s) {
  const bool direct = p.M >= W::BM && p.N >= W::BN && p.K >= W::BK &&
                      lane_offsets_fit(W::BM, p.lda, 4) && lane_offsets_fit(W::BK, p.ldb, 4);
  if (!direct) return FALLBACK(p, s);
  // A partial last step of r = K mod 32 valid k values.  MFMA group
  // 4 h + u of a step covers k = 16 h + u + {0, 4, 8, 12}, so it holds a
  // valid k iff 16 h + u < r: for r <= 16 the first min(r, 4) groups (run
  // as 1, 2 or 4, extra groups adding exact zeros), after the fill; for
  // r > 16 the whole pinned step.
  static_assert(W::BK == 32, "eight MFMA groups of 16x16x4 per step");
  const int r = p.K % W::BK;
  if (r == 0) return launch_big16_grid<W, big16_kernel<W>>(p, s);
  if (r == 1) return launch_big16_grid<W, big16_kernel<W, 1>>(p, s);
  if (r == 2) return launch_big16_grid<W, big16_kernel<W, 2>>(p, s);
  if (r <= 16) return launch_big16_grid<W, big16_kernel<W, 4>>(p, s);
  return launch_big16_grid<W, big16_kernel<W, W::BK / 4>>(p, s);
}

// The A-resident kernel on 16x16 MFMAs (arow16_kernel) when K == 64, C is
// whole 256x128 tiles, A and B rows are 16-byte aligned and the lane
// offsets fit in 32 bits; otherwise the 32x32-MFMA A-resident kernel.
hipError_t launch_arow16(const Problem &p, hipStream_t s) {
  using W = Arow16;
  const bool ok = p.K == W::BK && p.M % W::BM == 0 && p.N % W::BN == 0 && p.M > 0 && p.N > 0 &&
                  (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && (p.lda & 3) == 0 &&
                  (p.ldb & 3) == 0 && lane_offsets_fit(W::BM, p.lda, 4) &&
                  lane_offsets_fit(W::BK, p.ldb, 4);
  if (!ok) return launch_arow<P9>(p, s);
  const long long panels = p.M / W::BM, tiles_n = p.N / W::BN;
  if (panels * tiles_n > 0x7fffffffLL) return hipErrorInvalidValue;
  const long long slots = resident_workgroups<arow16_kernel, 256>();
  long long chunks = ceil_div(slots, panels);
  if (chunks > tiles_n) chunks = tiles_n;
  if (chunks < 1) chunks = 1;
  return launch_kernel(arow16_kernel, dim3((unsigned)(panels * chunks)), dim3(256), s, p,
                       (int)panels, (int)chunks, (int)tiles_n);
}

hipError_t launch_one(int index, const Problem &p, hipStream_t s) {
  switch (index) {
    case 0: return launch_kloop<C0>(p, s);
    case 1: return launch_kloop<C1>(p, s);
    case 2: return launch_kloop<C2>(p, s);
    case 3: return launch_kloop<C3>(p, s);
    case 4: return launch_kloop<C4>(p, s);
    case 5: return launch_kloop<C5>(p, s);
    case 6: return launch_kloop<C6>(p, s);
    case 7: return launch_kloop<C7>(p, s);
    case 8: return launch_panel<P8>(p, s);
    case 9: return launch_panel<P9>(p, s);
    case 10: return launch_kloop<C10>(p, s);
    case 11: return launch_kloop<C11>(p, s);
    case 12: return launch_kloop<C12>(p, s);
    case 13: return launch_panel<P9, true>(p, s);
    case 14: return launch_arow<P9>(p, s);
    case 15: return launch_lds_dma<C12>(p, s);
    case 16: return launch_ksplit(p, s);
    case 17: return launch_w16<W16<64, 64, 64, 2>, C0>(p, s);
    case 18: return launch_lds_dma16<C12>(p, s);
    case 19: return launch_big16<W16<128, 128, 32, 2>, launch_big16r<W16<128, 128, 32, 2>>>(p, s);
    case 25: {  // rows in whole rounds of entry 19's tiles, the rest on its own entry
      const int r = region_rows(p.M, p.N, p.K);
      if (r == 0) return launch_prod(model_kloop(p.M, p.N, p.K).entry, p, s);
      Problem top = p, rest = p;
      top.M = 256 * r;
      rest.M = p.M - top.M;
      rest.A = p.A + (long long)top.M * p.lda;
      rest.C = p.C + (long long)top.M * p.ldc;
      const hipError_t e = launch_prod(19, top, s);
      return e != hipSuccess ? e : launch_prod(model_kloop(rest.M, rest.N, rest.K).entry, rest, s);
    }
    case 24:  // 192x256 direct-load tiles (built apart); else entry 19's launcher
      return big16_192x256_fits(p)
                 ? launch_big16_192x256(p, s)
                 : launch_big16<W16<128, 128, 32, 2>, launch_big16r<W16<128, 128, 32, 2>>>(p, s);
    case 20: return launch_big16r<W16<128, 128, 32, 2>>(p, s);
    case 21: return launch_arow16(p, s);
    case 22:  // 192x192 direct-load tiles (built apart); else the 256x256 register path
      return big16_192_fits(p) ? launch_big16_192(p, s)
                               : launch_big16r<W16<128, 128, 32, 2>>(p, s);
    case 23:  // 128x128 direct-load tiles (built apart); else entry 17's launcher
      return big16_128_fits(p) ? launch_big16_128(p, s) : launch_w16<W16<64, 64, 64, 2>, C0>(p, s);
    case kStripConfig: return launch_strip(p, s);
    case kColStripConfig: return launch_colstrip(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_split_one(int index, const Problem &p, int splits, int kc, float *ws,
                            hipStream_t s) {
  switch (index) {
    case 0: return launch_split<C0>(p, splits, kc, ws, s);
    case 1: return launch_split<C1>(p, splits, kc, ws, s);
    case 2: return launch_split<C2>(p, splits, kc, ws, s);
    case 3: return launch_split<C3>(p, splits, kc, ws, s);
    case 4: return launch_split<C4>(p, splits, kc, ws, s);
    case 7: return launch_split<C7>(p, splits, kc, ws, s);
    case 12: return launch_split<C12>(p, splits, kc, ws, s);
    case 23: {  // the VGPR-form 128x128 kernel where it fits, else entry 0's kernel
      if (!big16_128_split_fits(p, kc)) return launch_split<C0>(p, splits, kc, ws, s);
      const hipError_t e = launch_big16_128_split(p, splits, kc, ws, s);
      return e != hipSuccess ? e : launch_splitk_reduce(p, splits, ws, s);
    }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prod_split(const SplitPlan &plan, const Problem &p, float *ws, hipStream_t s) {
  if (plan.splits <= 1) return launch_prod(plan.config, p, s);
  return launch_split_one(plan.config, p, plan.splits, plan.kc, ws, s);
}

// One product with launch-table entry `index`.  Thin remainder strips along
// M or N (and, for the small-K panel entries, any remainder) go to separate
// launches with small tiles; all launches share the stream, so they run in
// order.  The strip entries are the thin-M and thin-N kernels on the whole
// product.
hipError_t launch_prod(int index, const Problem &p, hipStream_t s) {
  if (!prod_supports(index, p.M, p.N, p.K)) return hipErrorInvalidValue;
  if (prod_kind(index) == kStrip) return launch_strip(p, s);
  if (prod_kind(index) == kStripN) return launch_colstrip(p, s);
  const ProdConfig &c = prod_config(index);
  int rm = index == kRemainderConfig ? 0 : thin_remainder(p.M, c.BM);
  int rn = index == kRemainderConfig ? 0 : thin_remainder(p.N, c.BN);
  if (prod_kind(index) == kPanel) {  // whole tiles only; every remainder is a strip
    rm = p.M % c.BM;
    rn = p.N % c.BN;
    if (p.M < c.BM || p.N < c.BN) return launch_one(kRemainderConfig, p, s);
  }
  Problem main_part = p;
  main_part.M = p.M - rm;
  main_part.N = p.N - rn;
  hipError_t e = launch_one(index, main_part, s);
  if (e != hipSuccess) return e;
  if (rn > 0) {  // right strip beside the main block
    Problem strip = p;
    strip.M = main_part.M;
    strip.N = rn;
    strip.B = p.B + main_part.N;
    strip.C = p.C + main_part.N;
    e = launch_one(kRemainderConfig, strip, s);
    if (e != hipSuccess) return e;
  }
  if (rm > 0) {  // bottom strip, full width
    Problem strip = p;
    strip.M = rm;
    strip.A = p.A + (long long)main_part.M * p.lda;
    strip.C = p.C + (long long)main_part.M * p.ldc;
    e = rm <= kStripMaxRows ? launch_strip(strip, s) : launch_one(kRemainderConfig, strip, s);
  }
  return e;
}

}  // namespace gemm_f32_impl
