// 16-bit inputs, fp32 accumulation and result, on gfx950 matrix cores.
//
// The pages name this as the step after the fp32 tiled kernel: the same
// tiling, with the block pyramid extended down to register blocks and a
// matrix instruction block, fed FP16 or BF16 inputs (geek-doc.cn "矩阵乘法
// tiling", section 五: the Tensor Core row of its table and the paragraph
// after it).  Here the instruction block is v_mfma_f32_32x32x16_bf16 (or
// _f16): a 32 x 32 block of C per wave from 16 k values, 8 per lane.
//
// Workgroup tile BM x BN with k step 64, two LDS stages, one barrier per
// step, the next step's tile prefetched into registers (as in the fp32
// production kernel).  Both operands sit in LDS as rows of 64 k values
// (8 sixteen-byte units, one pad unit after each row), because each MFMA
// lane reads 8 consecutive k of one row of A and one column of B:
//   * A (row-major M x K) is copied as it lies;
//   * B (row-major K x N) is transposed on its way in: a thread loads an
//     8 (k) x 8 (n) block as 8 row pieces, transposes it in registers and
//     writes 8 column pieces.  The unit index of B row n is XORed with
//     (n / 16) % 8 so these writes, and the MFMA reads, hit distinct banks.
// Half the threads stage A, the other half B (whole waves each).
//
// B is fed as the MFMA's first operand and A as its second, so a lane ends
// with 4-long runs of one C row and stores them with 128-bit writes.
// Elements outside A or B are loaded as 0 and stores outside C are skipped
// (geek-doc.cn section 六; mayulu.co "CUDA 编程系列之三", section 7).
#include "gemm_internal.hpp"
#include "launch_util.hpp"
#include "addr_math.hpp"

#include <cstdint>
#include <type_traits>

namespace gemm_f32_impl {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// 16 bytes at any 2-byte-aligned address: gfx950 under ROCm runs with
// unaligned global access enabled, so this is still one global_load_dwordx4.
typedef unsigned int u32x4u __attribute__((ext_vector_type(4), aligned(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kMixedBK = 64;
constexpr int kUnits = kMixedBK / 8;  // 16-byte units per LDS row
constexpr int kPitch = kUnits + 1;    // units per LDS row, with one pad unit

// BKB: k depth of the B block one thread transposes (8, or 4 when there
// are twice as many threads as 8 x 8 blocks).
template <int BM_, int BN_, int WGM_, int WGN_, int BKB_ = 8>
struct MTile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, BKB = BKB_;
  static constexpr int NT = 64 * WGM * WGN;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int HALF = NT / 2;          // threads staging A (and B)
  static constexpr int A_ROWS = HALF / 8;      // A rows covered by one load pass
  static constexpr int A_PER = BM / A_ROWS;    // A pieces per staging thread
  static constexpr int B_NB = BN / 8;          // 8-column blocks of B
  static constexpr int A_UNITS = BM * kPitch;
  static constexpr int STAGE_UNITS = (BM + BN) * kPitch;
  static_assert(BKB == 8 || BKB == 4, "B blocks are 8 or 4 k deep");
  static_assert((kMixedBK / BKB) * B_NB == HALF, "one B block per staging thread");
  static_assert(A_PER * A_ROWS == BM && A_PER <= 8, "A rows split evenly over staging threads");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
  static_assert(2 * STAGE_UNITS * 16 <= 160 * 1024, "two stages must fit in LDS");
};

template <int FMT>
__device__ inline f32x16 mfma16(u32x4 x, u32x4 y, f32x16 acc) {
  if constexpr (FMT == kMixedBf16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                   __builtin_bit_cast(bf16x8, y), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x),
                                                  __builtin_bit_cast(f16x8, y), acc, 0, 0, 0);
}

__device__ inline int b_swizzle(int n) { return (n >> 4) & 7; }

// One k step of this thread's share: up to 8 sixteen-byte pieces of A or
// of B (S::A_PER or S::BKB of them are used).
struct MStage {
  u32x4 v[8];
};

__device__ inline unsigned int pack2(unsigned int lo, unsigned int hi) {
  return (lo & 0xffffu) | (hi << 16);
}

// 8 codes from p[0..7], zero where e >= valid (valid may be <= 0).
__device__ inline u32x4 load8_guarded(const uint16_t *p, int valid) {
  unsigned int c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) c[e] = e < valid ? p[e] : 0u;
  return u32x4{pack2(c[0], c[1]), pack2(c[2], c[3]), pack2(c[4], c[5]), pack2(c[6], c[7])};
}

// Element offset of a lane's piece from the tile's origin.  OFF32: the
// launcher has checked that the tile's span fits in 32 bits, so the origin
// stays a uniform (scalar) pointer and each lane keeps only a 32-bit offset
// -- fewer registers than one 64-bit pointer per piece.
template <bool OFF32>
using MOffset = typename std::conditional<OFF32, unsigned int, long long>::type;

template <class S, bool GUARD, bool OFF32>
__device__ inline void mixed_load(MStage &st, const MixedProblem &p, int m0, int n0,
                                  int k0, int tid) {
  using Off = MOffset<OFF32>;
  if (tid < S::HALF) {
    const int u = tid & 7, r0 = tid >> 3;
    const uint16_t *origin = p.A + (long long)m0 * p.lda + k0;
#pragma unroll
    for (int j = 0; j < S::A_PER; ++j) {
      const int r = r0 + j * S::A_ROWS;
      const uint16_t *src = origin + ((Off)r * (Off)p.lda + (Off)(8 * u));
      if (!GUARD) st.v[j] = *reinterpret_cast<const u32x4u *>(src);
      else st.v[j] = load8_guarded(src, m0 + r < p.M ? p.K - (k0 + 8 * u) : 0);
    }
  } else {
    const int t = tid - S::HALF;
    const int nb = t % S::B_NB, kb = t / S::B_NB;
    const uint16_t *origin = p.B + (long long)k0 * p.ldb + n0;
#pragma unroll
    for (int j = 0; j < S::BKB; ++j) {
      const int r = S::BKB * kb + j;
      const uint16_t *src = origin + ((Off)r * (Off)p.ldb + (Off)(8 * nb));
      if (!GUARD) st.v[j] = *reinterpret_cast<const u32x4u *>(src);
      else st.v[j] = load8_guarded(src, k0 + r < p.K ? p.N - (n0 + 8 * nb) : 0);
    }
  }
}

template <class S>
__device__ inline void mixed_store_lds(const MStage &st, u32x4 *stage, int tid) {
  if (tid < S::HALF) {
    const int u = tid & 7, r0 = tid >> 3;
#pragma unroll
    for (int j = 0; j < S::A_PER; ++j) stage[(r0 + j * S::A_ROWS) * kPitch + u] = st.v[j];
  } else {
    const int t = tid - S::HALF;
    const int nb = t % S::B_NB, kb = t / S::B_NB;
    u32x4 *bs = stage + S::A_UNITS;
    // st.v[j] holds B[k0 + BKB kb + j][n .. n+7]; column piece i gathers
    // element i of each of the BKB rows, two codes per dword.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int w = i >> 1;
      unsigned int col[S::BKB / 2];
#pragma unroll
      for (int d = 0; d < S::BKB / 2; ++d) {
        const unsigned int lo = st.v[2 * d][w], hi = st.v[2 * d + 1][w];
        col[d] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      const int n = 8 * nb + i;
      if constexpr (S::BKB == 8) {
        bs[n * kPitch + (kb ^ b_swizzle(n))] = u32x4{col[0], col[1], col[2], col[3]};
      } else {
        // 4 k values: one half of unit kb / 2.
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        u32x2 *half = reinterpret_cast<u32x2 *>(bs + n * kPitch + ((kb >> 1) ^ b_swizzle(n)));
        half[kb & 1] = u32x2{col[0], col[1]};
      }
    }
  }
}

// k slices [KK0, KK1) of one stage (16 k values per slice).
template <class S, int FMT, int KK0 = 0, int KK1 = kUnits / 2>
__device__ inline void mixed_compute(const u32x4 *stage, f32x16 (&acc)[S::TM][S::TN], int wm,
                                     int wn, int lane) {
  const u32x4 *as = stage;
  const u32x4 *bs = stage + S::A_UNITS;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kk = KK0; kk < KK1; ++kk) {
    const int u = 2 * kk + h;
    u32x4 af[S::TM], bf[S::TN];
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm) af[tm] = as[(wm * S::WTM + 32 * tm + r) * kPitch + u];
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn) {
      const int n = wn * S::WTN + 32 * tn + r;
      bf[tn] = bs[n * kPitch + (u ^ b_swizzle(n))];
    }
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < S::TN; ++tn)
        acc[tm][tn] = mfma16<FMT>(bf[tn], af[tm], acc[tm][tn]);
  }
}

template <class S, int FMT, bool OFF32>
__global__ void __launch_bounds__(S::NT)
    mixed_kernel(MixedProblem p, int tiles_m, int tiles_n) {
  __shared__ u32x4 lds[2 * S::STAGE_UNITS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % S::WGM, wn = wave / S::WGM;
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  // A last tile row or column that would overhang C is moved back to end at
  // C's edge (when C is at least one tile wide): it overlaps its neighbour,
  // both compute the shared elements in the same k order and store the same
  // values, and the tile avoids element-wise edge loads.
  int m0 = tm * S::BM, n0 = tn * S::BN;
  if (m0 + S::BM > p.M && p.M >= S::BM) m0 = p.M - S::BM;
  if (n0 + S::BN > p.N && p.N >= S::BN) n0 = p.N - S::BN;
  const bool fast = m0 + S::BM <= p.M && n0 + S::BN <= p.N;
  const int nk = (p.K + kMixedBK - 1) / kMixedBK;

  f32x16 acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  MStage st;
  if (fast && kMixedBK <= p.K) mixed_load<S, false, OFF32>(st, p, m0, n0, 0, tid);
  else mixed_load<S, true, OFF32>(st, p, m0, n0, 0, tid);
  mixed_store_lds<S>(st, lds, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k1 = (kt + 1) * kMixedBK;
      if (fast && k1 + kMixedBK <= p.K) mixed_load<S, false, OFF32>(st, p, m0, n0, k1, tid);
      else mixed_load<S, true, OFF32>(st, p, m0, n0, k1, tid);
    }
    // The next stage's buffer was last read before the previous barrier, so
    // its write goes between the two halves of this step's matrix work.
    mixed_compute<S, FMT, 0, kUnits / 4>(lds + cur * S::STAGE_UNITS, acc, wm, wn, lane);
    if (more) mixed_store_lds<S>(st, lds + (cur ^ 1) * S::STAGE_UNITS, tid);
    mixed_compute<S, FMT, kUnits / 4, kUnits / 2>(lds + cur * S::STAGE_UNITS, acc, wm, wn, lane);
    __syncthreads();
  }

  // Lane holds C[m][n .. n+3] for m = ... + lane % 32 and
  // n = ... + 8q + 4 (lane / 32), q = 0..3, in acc[.][.][4q .. 4q+3].
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < S::TM; ++i) {
    const int m = m0 + wm * S::WTM + 32 * i + r;
    if (m >= p.M) continue;
    float *crow = p.C + (long long)m * p.ldc;
#pragma unroll
    for (int j = 0; j < S::TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * S::WTN + 32 * j + 8 * q + 4 * h;
        const f32x4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
        if (n + 4 <= p.N) {
          *reinterpret_cast<f32x4u *>(crow + n) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) crow[n + e] = v[e];
        }
      }
    }
  }
}

using Mixed256 = MTile<256, 256, 2, 4>;     // 8 waves, 128 x 64 per wave
using Mixed128 = MTile<128, 128, 2, 2>;     // 4 waves, 64 x 64 per wave
using Mixed256w16 = MTile<256, 256, 4, 4, 4>;  // 16 waves, 64 x 64 per wave

const MixedConfig kMixedConfigs[] = {
    {Mixed256::BM, Mixed256::BN, kMixedBK, Mixed256::WGM, Mixed256::WGN, 1, "256x256x64 w2x4"},
    {Mixed128::BM, Mixed128::BN, kMixedBK, Mixed128::WGM, Mixed128::WGN, 2, "128x128x64 w2x2"},
    {Mixed256w16::BM, Mixed256w16::BN, kMixedBK, Mixed256w16::WGM, Mixed256w16::WGN, 1,
     "256x256x64 w4x4"},
    {256, 256, kMixedBK, 2, 2, 1, "256x256x64 w2x2 ldsdma mfma16x16x32"},
    {256, 256, kMixedBK, 2, 2, 1, "256x256x64 w2x2 ldsdma mfma32x32x16"},
};
constexpr int kMixedNumConfigs = sizeof(kMixedConfigs) / sizeof(kMixedConfigs[0]);

template <class S, int FMT>
hipError_t launch_one(const MixedProblem &p, hipStream_t s) {
  const long long tiles_m = ceil_div(p.M, S::BM), tiles_n = ceil_div(p.N, S::BN);
  const long long tiles = tiles_m * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  // Largest element offset from a tile origin: BM rows of A, kMixedBK rows of B.
  const bool off32 = (long long)S::BM * p.lda < (1LL << 31) &&
                     (long long)kMixedBK * p.ldb < (1LL << 31);
  if (off32)
    return launch_kernel(mixed_kernel<S, FMT, true>, dim3((unsigned)tiles), dim3(S::NT), s, p,
                         (int)tiles_m, (int)tiles_n);
  return launch_kernel(mixed_kernel<S, FMT, false>, dim3((unsigned)tiles), dim3(S::NT), s, p,
                       (int)tiles_m, (int)tiles_n);
}

}  // namespace

int mixed_num_configs() { return kMixedNumConfigs; }

const MixedConfig &mixed_config(int index) { return kMixedConfigs[index]; }

// Fewest rounds of resident workgroups, weighting a round by the tile area a
// CU covers in it; ties go to the larger tile (more reuse per LDS byte).
// Below four k steps a lone 256 x 256 workgroup per CU cannot hide its
// loads and stores behind matrix work, so short K takes the 128 x 128 entry
// (two workgroups per CU overlap each other's epilogues).
//
// Entry 3 (direct loads on 16x16x32 MFMAs, one wave per SIMD) takes every
// product whose K is a multiple of its 64-deep step and whose 256 x 256
// tiles fill the GPU, and any other 256 x 256 choice with such a K; its
// launcher falls back to entry 0 for rows that are not 16-byte aligned.
// With K = 64 (one step per tile, the time mostly the C stores) entry 4,
// the same kernel on 32x32x16 MFMAs, is faster (16384 x 16384 x 64: 200
// against 223 us); with more steps per tile the operand traffic through
// LDS bounds both and entry 3 is ahead (4096^3: 102 against 109 us;
// 4400 x 4352 x 128: 27.9 against 29.9).
int mixed_choose(int M, int N, int K) {
  const long long tiles256 = (long long)ceil_div(M, 256) * ceil_div(N, 256);
  if (K == kMixedBK && tiles256 >= 256) return 4;
  if (K % kMixedBK == 0 && tiles256 >= 256) return 3;
  if (K < 4 * kMixedBK) return 1;
  int best = 0;
  double best_cost = 0;
  for (int c = 0; c < 3; ++c) {
    const MixedConfig &cfg = kMixedConfigs[c];
    const double tiles = (double)ceil_div(M, cfg.BM) * (double)ceil_div(N, cfg.BN);
    const double slots = 256.0 * cfg.occupancy;
    const double rounds = (double)(long long)((tiles + slots - 1) / slots);
    const double cost = rounds * cfg.BM * cfg.BN * cfg.occupancy;
    if (c == 0 || cost < best_cost) best = c, best_cost = cost;
  }
  if (kMixedConfigs[best].BM == 256 && K % kMixedBK == 0) return 3;
  return best;
}

hipError_t launch_mixed(int format, int index, const MixedProblem &p, hipStream_t s) {
  const bool bf = format == kMixedBf16;
  switch (index) {
    case 0: return bf ? launch_one<Mixed256, kMixedBf16>(p, s) : launch_one<Mixed256, kMixedF16>(p, s);
    case 1: return bf ? launch_one<Mixed128, kMixedBf16>(p, s) : launch_one<Mixed128, kMixedF16>(p, s);
    case 2:
      return bf ? launch_one<Mixed256w16, kMixedBf16>(p, s) : launch_one<Mixed256w16, kMixedF16>(p, s);
    case 3:  // direct loads on 16x16x32 MFMAs where they fit, else entry 0
      if (mixed16_fits(p)) return launch_mixed16(format, p, s, false);
      return bf ? launch_one<Mixed256, kMixedBf16>(p, s) : launch_one<Mixed256, kMixedF16>(p, s);
    case 4:  // the same on 32x32x16 MFMAs
      if (mixed16_fits(p)) return launch_mixed16(format, p, s, true);
      return bf ? launch_one<Mixed256, kMixedBf16>(p, s) : launch_one<Mixed256, kMixedF16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gemm_f32_impl
