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
// Per workgroup: a BM x BN tile of C, WGM x WGN waves, each wave a
// (BM/WGM) x (BN/WGN) sub-tile made of 32 x 32 MFMA blocks whose
// accumulators stay in registers for the whole k loop.
//
// Data path per k step (depth BK):
//   global -> registers: the next step's A and B tiles, 128-bit loads where
//     rows are 16-byte aligned (scalar loads otherwise), consecutive lanes on
//     consecutive addresses;
//   registers -> LDS: into the stage not being read (two stages), rows padded
//     so that the fragment reads below do not collide in LDS banks;
//   LDS -> MFMA: per 8-deep k group a lane reads one 128-bit A fragment per
//     32-row block and four B scalars per 32-column block.
//   One barrier per k step suffices with two stages: a stage is rewritten
//   only after the barrier that follows its last read.  (The pages' single
//   buffer needs its two barriers per step; the two-stage form here is a
//   departure from them.)
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
// section 7), and guarded stores that leave C outside M x N untouched.
// Interior steps take unguarded loads.
//
// Workgroup order.  Workgroups are dealt to the 8 XCDs round robin by
// launch index; the index is remapped so that each XCD receives a contiguous
// run of tiles, and runs are laid out in groups of 8 tile rows so that the
// tiles sharing an XCD's L2 also share A rows and B columns.
#include "gemm_internal.hpp"
#include "launch_util.hpp"

#include <cstdint>

namespace gemm_f32_impl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPadA = 4;  // floats after each LDS row of A (k-contiguous rows)
constexpr int kPadB = 8;  // floats after each LDS row of B (n-contiguous rows)
constexpr int kXcds = 8;
constexpr int kGroupRows = 8;

template <int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
  static constexpr int NT = 64 * WGM * WGN;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave sub-tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;    // MFMA blocks per wave
  static constexpr int SA = BK + kPadA;                  // LDS row stride of A
  static constexpr int SB = BN + kPadB;                  // LDS row stride of B
  static constexpr int A_STAGE = BM * SA;
  static constexpr int B_STAGE = BK * SB;
  static constexpr int LDS_FLOATS = 2 * (A_STAGE + B_STAGE);
  // vector (128-bit) staging: chunks of 4 floats
  static constexpr int A_CHUNKS = BM * BK / 4 / NT;  // per thread
  static constexpr int B_CHUNKS = BK * BN / 4 / NT;
  static constexpr int A_ROWS_PER_PASS = NT / (BK / 4);
  static constexpr int B_ROWS_PER_PASS = NT / (BN / 4);
  // scalar staging
  static constexpr int A_ELEMS = BM * BK / NT;
  static constexpr int B_ELEMS = BK * BN / NT;
  static constexpr int A_ROWS_PER_PASS_S = NT / BK;
  static constexpr int B_ROWS_PER_PASS_S = NT / BN;

  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
  static_assert(BK % 8 == 0, "BK must be a multiple of 8");
  static_assert(NT % (BK / 4) == 0 && NT % (BN / 4) == 0, "vector staging map");
  static_assert(NT % BK == 0 && NT % BN == 0, "scalar staging map");
  static_assert((BM * BK) % (4 * NT) == 0 && (BK * BN) % (4 * NT) == 0,
                "tile must split evenly over threads");
  static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget of a gfx950 CU");
};

// Remap the launch index so each XCD gets a contiguous run of tile ids,
// then walk tiles in groups of kGroupRows tile rows, column by column.
__device__ inline void tile_of(int b, int G, int tiles_m, int tiles_n, int &tm,
                               int &tn) {
  const int per = G / kXcds, rem = G % kXcds, x = b % kXcds;
  const int lid = x * per + (x < rem ? x : rem) + b / kXcds;
  const int per_group = kGroupRows * tiles_n;
  const int g = lid / per_group;
  const int first = g * kGroupRows;
  const int rows = tiles_m - first < kGroupRows ? tiles_m - first : kGroupRows;
  const int r = lid - g * per_group;
  tm = first + r % rows;
  tn = r / rows;
}

template <class S, bool VEC>
struct Stage {
  // registers holding one k step of A and B on their way to LDS
  f32x4 a[VEC ? S::A_CHUNKS : S::A_ELEMS / 4];
  f32x4 b[VEC ? S::B_CHUNKS : S::B_ELEMS / 4];
};

template <class S, bool VEC, bool GUARD>
__device__ inline void load_global(Stage<S, VEC> &st, const Problem &p, int m0,
                                   int n0, int k0, int tid) {
  if constexpr (VEC) {
    const int arow = tid / (S::BK / 4), akq = (tid % (S::BK / 4)) * 4;
#pragma unroll
    for (int i = 0; i < S::A_CHUNKS; ++i) {
      const int gm = m0 + arow + i * S::A_ROWS_PER_PASS;
      const int gk = k0 + akq;
      const float *src = p.A + (long long)gm * p.lda + gk;
      if (!GUARD || (gm < p.M && gk < p.K))
        st.a[i] = *reinterpret_cast<const f32x4 *>(src);
      else
        st.a[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int bkr = tid / (S::BN / 4), bnq = (tid % (S::BN / 4)) * 4;
#pragma unroll
    for (int i = 0; i < S::B_CHUNKS; ++i) {
      const int gk = k0 + bkr + i * S::B_ROWS_PER_PASS;
      const int gn = n0 + bnq;
      const float *src = p.B + (long long)gk * p.ldb + gn;
      if (!GUARD || (gk < p.K && gn < p.N))
        st.b[i] = *reinterpret_cast<const f32x4 *>(src);
      else
        st.b[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  } else {
    const int arow = tid / S::BK, ak = tid % S::BK;
#pragma unroll
    for (int i = 0; i < S::A_ELEMS; ++i) {
      const int gm = m0 + arow + i * S::A_ROWS_PER_PASS_S;
      const int gk = k0 + ak;
      float v = 0.f;
      if (!GUARD || (gm < p.M && gk < p.K)) v = p.A[(long long)gm * p.lda + gk];
      st.a[i / 4][i % 4] = v;
    }
    const int bkr = tid / S::BN, bn = tid % S::BN;
#pragma unroll
    for (int i = 0; i < S::B_ELEMS; ++i) {
      const int gk = k0 + bkr + i * S::B_ROWS_PER_PASS_S;
      const int gn = n0 + bn;
      float v = 0.f;
      if (!GUARD || (gk < p.K && gn < p.N)) v = p.B[(long long)gk * p.ldb + gn];
      st.b[i / 4][i % 4] = v;
    }
  }
}

template <class S, bool VEC>
__device__ inline void store_lds(const Stage<S, VEC> &st, float *as, float *bs,
                                 int tid) {
  if constexpr (VEC) {
    const int arow = tid / (S::BK / 4), akq = (tid % (S::BK / 4)) * 4;
#pragma unroll
    for (int i = 0; i < S::A_CHUNKS; ++i)
      *reinterpret_cast<f32x4 *>(as + (arow + i * S::A_ROWS_PER_PASS) * S::SA + akq) = st.a[i];
    const int bkr = tid / (S::BN / 4), bnq = (tid % (S::BN / 4)) * 4;
#pragma unroll
    for (int i = 0; i < S::B_CHUNKS; ++i)
      *reinterpret_cast<f32x4 *>(bs + (bkr + i * S::B_ROWS_PER_PASS) * S::SB + bnq) = st.b[i];
  } else {
    const int arow = tid / S::BK, ak = tid % S::BK;
#pragma unroll
    for (int i = 0; i < S::A_ELEMS; ++i)
      as[(arow + i * S::A_ROWS_PER_PASS_S) * S::SA + ak] = st.a[i / 4][i % 4];
    const int bkr = tid / S::BN, bn = tid % S::BN;
#pragma unroll
    for (int i = 0; i < S::B_ELEMS; ++i)
      bs[(bkr + i * S::B_ROWS_PER_PASS_S) * S::SB + bn] = st.b[i / 4][i % 4];
  }
}

// All MFMAs of one k step out of one LDS stage.
template <class S>
__device__ inline void compute_stage(f32x16 (&acc)[S::TM][S::TN],
                                     const float *as, const float *bs,
                                     int wm, int wn, int lane) {
  const int l32 = lane & 31, h = lane >> 5;
  const float *a_base = as + (wm * S::WTM + l32) * S::SA + 4 * h;
  const float *b_base = bs + (4 * h) * S::SB + wn * S::WTN + l32;
#pragma unroll
  for (int kg = 0; kg < S::BK / 8; ++kg) {
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

template <class S, bool VEC_C>
__device__ inline void store_c(const f32x16 (&acc)[S::TM][S::TN],
                               const Problem &p, int m0, int n0, int wm,
                               int wn, int lane) {
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
        if constexpr (VEC_C) {
          // N % 4 == 0: a 4-column run is wholly inside or outside C.
          if (row < p.M && col < p.N) *reinterpret_cast<f32x4 *>(crow + col) = v;
        } else {
          if (row < p.M) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (col + r < p.N) crow[col + r] = v[r];
          }
        }
      }
    }
  }
}

template <class S, bool VEC_AB, bool VEC_C>
__global__ void __launch_bounds__(S::NT)
    prod_kernel(Problem p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) float lds[S::LDS_FLOATS];
  float *const as0 = lds;
  float *const bs0 = lds + 2 * S::A_STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int ntiles = tiles_m * tiles_n;
  const int nk = (p.K + S::BK - 1) / S::BK;

  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    int tm, tn;
    tile_of(t, ntiles, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * S::BM, n0 = tn * S::BN;
    const bool interior = (m0 + S::BM <= p.M) && (n0 + S::BN <= p.N);

    f32x16 acc[S::TM][S::TN];
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
#pragma unroll
      for (int j = 0; j < S::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    Stage<S, VEC_AB> st;
    if (interior && S::BK <= p.K)
      load_global<S, VEC_AB, false>(st, p, m0, n0, 0, tid);
    else
      load_global<S, VEC_AB, true>(st, p, m0, n0, 0, tid);
    store_lds<S, VEC_AB>(st, as0, bs0, tid);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        const int k1 = (kt + 1) * S::BK;
        if (interior && k1 + S::BK <= p.K)
          load_global<S, VEC_AB, false>(st, p, m0, n0, k1, tid);
        else
          load_global<S, VEC_AB, true>(st, p, m0, n0, k1, tid);
      }
      compute_stage<S>(acc, as0 + cur * S::A_STAGE, bs0 + cur * S::B_STAGE, wm,
                       wn, lane);
      if (more)
        store_lds<S, VEC_AB>(st, as0 + (cur ^ 1) * S::A_STAGE,
                             bs0 + (cur ^ 1) * S::B_STAGE, tid);
      __syncthreads();
    }
    store_c<S, VEC_C>(acc, p, m0, n0, wm, wn, lane);
  }
}

// ---- launch table ----------------------------------------------------

using T128x128x32 = Tile<128, 128, 32, 2, 2>;
using T128x128x16 = Tile<128, 128, 16, 2, 2>;
using T256x128x16 = Tile<256, 128, 16, 4, 2>;
using T64x64x32 = Tile<64, 64, 32, 2, 2>;
using T128x64x32 = Tile<128, 64, 32, 2, 2>;

const ProdConfig kConfigs[] = {
    {128, 128, 32, 2, 2, 2, "128x128x32_w2x2"},
    {128, 128, 16, 2, 2, 4, "128x128x16_w2x2"},
    {256, 128, 16, 4, 2, 2, "256x128x16_w4x2"},
    {64, 64, 32, 2, 2, 4, "64x64x32_w2x2"},
    {128, 64, 32, 2, 2, 4, "128x64x32_w2x2"},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

bool aligned16(const void *q) {
  return (reinterpret_cast<std::uintptr_t>(q) & 15u) == 0;
}

template <class S>
hipError_t launch_shape(const Problem &p, hipStream_t s) {
  const long long tiles_m = ceil_div(p.M, S::BM), tiles_n = ceil_div(p.N, S::BN);
  const long long ntiles = tiles_m * tiles_n;
  if (ntiles > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool vec_ab = p.K % 4 == 0 && p.N % 4 == 0 && p.lda % 4 == 0 &&
                      p.ldb % 4 == 0 && aligned16(p.A) && aligned16(p.B);
  const bool vec_c = p.N % 4 == 0 && p.ldc % 4 == 0 && aligned16(p.C);
  const dim3 grid((unsigned)ntiles), block(S::NT);
  const int tm = (int)tiles_m, tn = (int)tiles_n;
  if (vec_ab && vec_c)
    return launch_kernel(prod_kernel<S, true, true>, grid, block, s, p, tm, tn);
  if (vec_ab)
    return launch_kernel(prod_kernel<S, true, false>, grid, block, s, p, tm, tn);
  if (vec_c)
    return launch_kernel(prod_kernel<S, false, true>, grid, block, s, p, tm, tn);
  return launch_kernel(prod_kernel<S, false, false>, grid, block, s, p, tm, tn);
}

}  // namespace

int prod_num_configs() { return kNumConfigs; }

const ProdConfig &prod_config(int index) { return kConfigs[index]; }

// Shape-based choice: the largest tile that still gives every CU work.
int prod_choose(int M, int N, int K) {
  (void)K;
  const long long t128 = ceil_div(M, 128) * ceil_div(N, 128);
  if (t128 >= 512) return 0;
  const long long t64 = ceil_div(M, 128) * ceil_div(N, 64);
  if (t64 >= 256) return 4;
  return 3;
}

hipError_t launch_prod(int index, const Problem &p, hipStream_t s) {
  switch (index) {
    case 0: return launch_shape<T128x128x32>(p, s);
    case 1: return launch_shape<T128x128x16>(p, s);
    case 2: return launch_shape<T256x128x16>(p, s);
    case 3: return launch_shape<T64x64x32>(p, s);
    case 4: return launch_shape<T128x64x32>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gemm_f32_impl
