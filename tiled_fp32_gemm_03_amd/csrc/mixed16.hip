// 16-bit inputs on 16x16x32 MFMAs with direct-to-LDS loads, one wave per
// SIMD: the fp32 path's 128x128-wave recipe (big16_kernel) for bf16 and
// fp16 operands with fp32 accumulation.
//
// Tile 256x256 over 4 waves (2 x 2), each computing 128x128 as 8 x 8 blocks
// of v_mfma_f32_16x16x32_bf16 (or _f16): 64 chains, 256 accumulators per
// lane in the accumulation registers.  64-deep k steps, two LDS stages of
// 64 KB, both operands loaded by global_load_lds_dwordx4 in their own
// row-major layouts:
//   * A rows of 64 k (8 chunks of 16 bytes), chunk c of row r at
//     c ^ ((r >> 1) & 7); a lane's A operand (row m, k = 8 g .. 8 g + 7 of
//     a 32-deep group, g = lane / 16) is one 16-byte read;
//   * B rows of 256 n (16 slots of 32 bytes), slot s of k row k at
//     s ^ ((k & 3) | ((k >> 3) & 1) << 2); a lane's B operand (column n,
//     the same 8 k) comes from two ds_read_b64_tr_b16: in each 16-lane
//     group, lane L reads 4 elements of k row kbase + L / 4 at columns
//     4 (L % 4) .. + 3, and the read hands lane i the elements of column i
//     for k = kbase .. kbase + 3.  The slot permutation puts the 8 rows one
//     32-lane half reads on distinct banks.
// B is the MFMA's first operand and A its second, so a lane ends with four
// consecutive columns of one C row (16-byte stores).  Per step a wave
// issues 128 MFMAs against 16 direct loads, 16 A and 32 B reads and one
// barrier.  Each element is summed in 32-deep groups in ascending k, the
// MFMA adding a group's products; the bits can differ from the 32x32x16
// entries.
#include "gemm_internal.hpp"
#include "w16_tiles.hpp"
#include "addr_math16.hpp"

namespace gemm_f32_impl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct M16 {
  static constexpr int WTM = 128, WTN = 128, BK = 64;
  static constexpr int BM = 2 * WTM, BN = 2 * WTN;
  static constexpr int TBM = WTM / 16, TBN = WTN / 16;
  static constexpr int KG = BK / 32;             // 32-deep MFMA groups per step
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_DMA = A_BYTES / 1024 / 4;  // 1 KB instructions per wave and step
  static constexpr int B_DMA = B_BYTES / 1024 / 4;
  static constexpr int DMA = A_DMA + B_DMA;
  static constexpr int ACH = BK / 8;   // 16-byte chunks per A row
  static constexpr int BSL = BN / 16;  // 32-byte slots per B row
  static_assert(2 * STAGE <= kLdsBytes, "two stages fit in LDS");
  static_assert(ACH == 8, "the A permutation is written for 8 chunks per row");
  static_assert(DMA <= 2 * KG * TBM, "two direct loads per row of MFMAs cover a step's");
};

static_assert(M16::ACH == 8 && M16::BSL == 16, "layouts of addr_math16.hpp (m16_a_pos, m16_b_slot)");

template <int FMT>
__device__ inline f32x4 mfma32(i16x8 b, i16x8 a, f32x4 acc) {
  if constexpr (FMT == kMixedBf16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b),
                                                   __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b),
                                                  __builtin_bit_cast(f16x8, a), acc, 0, 0, 0);
}

// Fragment reads.  A: row block bm of the wave, 32-deep group kg.  B:
// column block bn, group kg, as two transposing reads.
__device__ inline i16x8 m16_read_a(const char *st, int wm, int bm, int kg, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  const int r = wm * M16::WTM + 16 * bm + l16;
  return *reinterpret_cast<const i16x8 *>(st + 16 * m16_a_pos(r, 4 * kg + g));
}
__device__ inline i16x8 m16_read_b(const char *st, int wn, int bn, int kg, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  const int s = wn * (M16::WTN / 16) + bn;  // 32-byte slot of this 16-column block
  const int q = l16 & 3;                    // which 8 bytes of the slot
  i16x4 h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int k = 32 * kg + 8 * g + 4 * half + (l16 >> 2);
    const char *addr = st + M16::A_BYTES + k * (M16::BN * 2) + 32 * m16_b_slot(k, s) + 8 * q;
    h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(addr));
  }
  return i16x8{h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
}

// The launcher guarantees M >= 256, N >= 256 (tiles moved inside C at the
// edges), K a positive multiple of 64, N % 8 == 0, 16-byte aligned rows of
// A and B, and 32-bit lane offsets (lane_offsets_fit over 256 rows of A and
// 64 rows of B).
template <int FMT>
__global__ void __launch_bounds__(256) mixed16_kernel(MixedProblem p, int tiles_m, int tiles_n) {
  using W = M16;
  __shared__ __attribute__((aligned(16))) char lds[2 * W::STAGE];
  const unsigned lds_u = (unsigned)(uintptr_t)(lds_void_t *)lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int ntiles = tiles_m * tiles_n;
  const int nk = p.K / W::BK;
  const int G = gridDim.x;
  const int lid = xcd_remap(blockIdx.x, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int my_tiles = (ntiles - lid + G - 1) / G;

  // Per-lane byte offsets of this wave's direct loads from a step's base
  // addresses: instruction q fills 1 KB of the stage in layout order.
  unsigned voff[W::DMA];
#pragma unroll
  for (int q = 0; q < W::A_DMA; ++q)
    voff[q] = (unsigned)(m16_dma_a_elem(64 * (wave * W::A_DMA + q) + lane, p.lda) * 2);
#pragma unroll
  for (int q = 0; q < W::B_DMA; ++q)
    voff[W::A_DMA + q] =
        (unsigned)(m16_dma_b_elem<false>(64 * (wave * W::B_DMA + q) + lane, p.ldb) * 2);
  const unsigned wave_a = (unsigned)(wave * W::A_DMA * 1024);
  const unsigned wave_b = (unsigned)(W::A_BYTES + wave * W::B_DMA * 1024);
  const long long b_step = (long long)W::BK * p.ldb;

  auto origin = [&](int t, int &m0, int &n0) __attribute__((always_inline)) {
    int tm, tn;
    tile_coords(lid + t * G, tiles_m, tiles_n, tm, tn);
    m0 = tm * W::BM;
    n0 = tn * W::BN;
    if (m0 + W::BM > p.M) m0 = p.M - W::BM;
    if (n0 + W::BN > p.N) n0 = p.N - W::BN;
  };
  auto tile_base = [&](int t, const uint16_t *&ab, const uint16_t *&bb)
      __attribute__((always_inline)) {
    int m0, n0;
    origin(t, m0, n0);
    ab = p.A + (long long)m0 * p.lda;
    bb = p.B + n0;
  };
  auto issue = [&](unsigned st, const uint16_t *ab, const uint16_t *bb, int q0, int q1)
      __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < W::DMA; ++q) {
      if (q < q0 || q >= q1) continue;
      if (q < W::A_DMA)
        ks_load_to_lds16(voff[q], reinterpret_cast<const float *>(ab), st + wave_a + q * 1024);
      else
        ks_load_to_lds16(voff[q], reinterpret_cast<const float *>(bb),
                         st + wave_b + (q - W::A_DMA) * 1024);
    }
  };

  const uint16_t *is_a, *is_b;  // operands of the step most recently issued
  tile_base(0, is_a, is_b);
  issue(lds_u, is_a, is_b, 0, W::DMA);
  int stage = 0;

  f32x4 acc[W::TBM][W::TBN];
  for (int t = 0; t < my_tiles; ++t) {
    const uint16_t *nt_a, *nt_b;  // the next tile's first step (this tile's on the last)
    tile_base(t + 1 < my_tiles ? t + 1 : t, nt_a, nt_b);
#pragma unroll
    for (int i = 0; i < W::TBM; ++i)
#pragma unroll
      for (int j = 0; j < W::TBN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kk = 0; kk < nk; ++kk) {
      const bool last = kk + 1 == nk;
      const uint16_t *ia = last ? nt_a : is_a + W::BK;
      const uint16_t *ib = last ? nt_b : is_b + b_step;
      __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));  // this step's loads (own)
      ks_lds_barrier();                                // everyone's; the other stage free
      const char *st = lds + stage * W::STAGE;
      const unsigned nst = lds_u + (stage ^ 1) * W::STAGE;

      // Group 0's operands in the order its first row of MFMAs uses them,
      // then each group's MFMAs row by row, the next group's fragments read
      // after the first half, two direct loads of the next step per row.
      i16x8 a0[W::TBM], a1[W::TBM], b0[W::TBN], b1[W::TBN];
      b0[0] = m16_read_b(st, wn, 0, 0, lane);
      __builtin_amdgcn_sched_barrier(0);
      a0[0] = m16_read_a(st, wm, 0, 0, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bn = 1; bn < W::TBN; ++bn) b0[bn] = m16_read_b(st, wn, bn, 0, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bm = 1; bm < W::TBM; ++bm) {
        a0[bm] = m16_read_a(st, wm, bm, 0, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int kg = 0; kg < W::KG; ++kg) {
        i16x8(&ac)[W::TBM] = (kg & 1) ? a1 : a0;
        i16x8(&an)[W::TBM] = (kg & 1) ? a0 : a1;
        i16x8(&bc)[W::TBN] = (kg & 1) ? b1 : b0;
        i16x8(&bnx)[W::TBN] = (kg & 1) ? b0 : b1;
#pragma unroll
        for (int bm = 0; bm < W::TBM; ++bm) {
#pragma unroll
          for (int bn = 0; bn < W::TBN; ++bn)
            acc[bm][bn] = mfma32<FMT>(bc[bn], ac[bm], acc[bm][bn]);
          constexpr int kLoadsPerRow = 2;
          const int row = kg * W::TBM + bm;
          if (row * kLoadsPerRow < W::DMA) {
            __builtin_amdgcn_sched_barrier(0);
            issue(nst, ia, ib, row * kLoadsPerRow, (row + 1) * kLoadsPerRow);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (kg + 1 < W::KG && bm == W::TBM / 2 - 1) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int bn = 0; bn < W::TBN; ++bn) bnx[bn] = m16_read_b(st, wn, bn, kg + 1, lane);
#pragma unroll
            for (int i = 0; i < W::TBM; ++i) an[i] = m16_read_a(st, wm, i, kg + 1, lane);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      is_a = ia;
      is_b = ib;
      stage ^= 1;
      // accumulators handed on in accumulation registers (see big16_kernel)
#pragma unroll
      for (int i = 0; i < W::TBM; ++i)
#pragma unroll
        for (int j = 0; j < W::TBN; ++j) asm volatile("" : "+a"(acc[i][j]));
    }

    int m0, n0;
    origin(t, m0, n0);
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

// The same tile, waves, steps and direct loads on 32x32x16 MFMAs.  One
// wave per SIMD issuing independent v_mfma_f32_16x16x32_bf16 reaches 1.3 to
// 1.5 PFLOP/s on the whole chip with no memory traffic at all, and
// v_mfma_f32_32x32x16_bf16 2.0 to 2.4 (each instruction is twice the work,
// so a lone wave keeps the matrix pipe full; gemm_f32_probe_mfma16).  The
// 16x16 form above runs at about 0.86 of its instruction's ceiling; this
// one needs 8% fewer cycles for a 4096^3 product, but under its load the
// engine clock settles about 14% lower (2.0 against 2.3 GHz), so it is
// faster only where the C stores dominate (K = 64).  A wave's 128 x 128 is 4 x 4
// blocks of 32 x 32 (16 accumulators each, 256 in all); a 64-deep step is
// 4 groups of 16 k, 16 MFMAs per group.  Fragments per lane (l32 = lane %
// 32, h = lane / 32): A row l32 of block bm, k = 16 kg + 8 h .. + 7, one
// 16-byte read in the layout above; B column l32 of block bn, the same 8 k,
// two transposing reads: 16-lane group q = lane / 16 reads the 16 columns
// 32 bn + 16 (q % 2) .. + 15 at k rows 16 kg + 8 (q / 2) + 4 half .. + 3.
// B rows of 256 n (16 slots of 32 bytes), slot s of k row k at
// m32_b_slot(k, s) (addr_math16.hpp): a 32-lane half reads two adjacent
// slots in four consecutive k rows, and the permutation puts those eight
// 32-byte pieces, and each 16-lane group's four, on distinct banks.
// Each element is summed in 16-deep groups in ascending k, as by the
// 32 x 32 x 16 entries that stage through registers, so the bits are
// theirs.
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct M32 {
  static constexpr int WTM = 128, WTN = 128, BK = 64;
  static constexpr int BM = 2 * WTM, BN = 2 * WTN;
  static constexpr int TBM = WTM / 32, TBN = WTN / 32;
  static constexpr int KG = BK / 16;             // 16-deep MFMA groups per step
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_DMA = A_BYTES / 1024 / 4;  // 1 KB instructions per wave and step
  static constexpr int B_DMA = B_BYTES / 1024 / 4;
  static constexpr int DMA = A_DMA + B_DMA;
  static constexpr int ACH = BK / 8;   // 16-byte chunks per A row
  static constexpr int BSL = BN / 16;  // 32-byte slots per B row
  static_assert(2 * STAGE <= kLdsBytes, "two stages fit in LDS");
  static_assert(ACH == 8, "the A permutation is written for 8 chunks per row");
  static_assert(DMA == 2 * 2 * TBM, "two direct loads per row of the first two groups");
};


template <int FMT>
__device__ inline f32x16 mfma32x32(i16x8 b, i16x8 a, f32x16 acc) {
  if constexpr (FMT == kMixedBf16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b),
                                                   __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, b),
                                                  __builtin_bit_cast(f16x8, a), acc, 0, 0, 0);
}

__device__ inline i16x8 m32_read_a(const char *st, int wm, int bm, int kg, int lane) {
  const int r = wm * M32::WTM + 32 * bm + (lane & 31);
  return *reinterpret_cast<const i16x8 *>(st + 16 * m16_a_pos(r, 2 * kg + (lane >> 5)));
}
__device__ inline i16x8 m32_read_b(const char *st, int wn, int bn, int kg, int lane) {
  const int l16 = lane & 15, q16 = lane >> 4;
  const int s = wn * (M32::WTN / 16) + 2 * bn + (q16 & 1);  // 32-byte slot (16 columns)
  i16x4 h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int k = 16 * kg + 8 * (q16 >> 1) + 4 * half + (l16 >> 2);
    const char *addr =
        st + M32::A_BYTES + k * (M32::BN * 2) + 32 * m32_b_slot(k, s) + 8 * (l16 & 3);
    h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(addr));
  }
  return i16x8{h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
}

template <int FMT>
__global__ void __launch_bounds__(256) mixed32_kernel(MixedProblem p, int tiles_m, int tiles_n) {
  using W = M32;
  __shared__ __attribute__((aligned(16))) char lds[2 * W::STAGE];
  const unsigned lds_u = (unsigned)(uintptr_t)(lds_void_t *)lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int ntiles = tiles_m * tiles_n;
  const int nk = p.K / W::BK;
  const int G = gridDim.x;
  const int lid = xcd_remap(blockIdx.x, G);
  if (lid >= ntiles) return;  // uniform per workgroup
  const int my_tiles = (ntiles - lid + G - 1) / G;

  unsigned voff[W::DMA];
#pragma unroll
  for (int q = 0; q < W::A_DMA; ++q)
    voff[q] = (unsigned)(m16_dma_a_elem(64 * (wave * W::A_DMA + q) + lane, p.lda) * 2);
#pragma unroll
  for (int q = 0; q < W::B_DMA; ++q)
    voff[W::A_DMA + q] =
        (unsigned)(m16_dma_b_elem<true>(64 * (wave * W::B_DMA + q) + lane, p.ldb) * 2);
  const unsigned wave_a = (unsigned)(wave * W::A_DMA * 1024);
  const unsigned wave_b = (unsigned)(W::A_BYTES + wave * W::B_DMA * 1024);
  const long long b_step = (long long)W::BK * p.ldb;

  auto origin = [&](int t, int &m0, int &n0) __attribute__((always_inline)) {
    int tm, tn;
    tile_coords(lid + t * G, tiles_m, tiles_n, tm, tn);
    m0 = tm * W::BM;
    n0 = tn * W::BN;
    if (m0 + W::BM > p.M) m0 = p.M - W::BM;
    if (n0 + W::BN > p.N) n0 = p.N - W::BN;
  };
  auto tile_base = [&](int t, const uint16_t *&ab, const uint16_t *&bb)
      __attribute__((always_inline)) {
    int m0, n0;
    origin(t, m0, n0);
    ab = p.A + (long long)m0 * p.lda;
    bb = p.B + n0;
  };
  auto issue = [&](unsigned st, const uint16_t *ab, const uint16_t *bb, int q0, int q1)
      __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < W::DMA; ++q) {
      if (q < q0 || q >= q1) continue;
      if (q < W::A_DMA)
        ks_load_to_lds16(voff[q], reinterpret_cast<const float *>(ab), st + wave_a + q * 1024);
      else
        ks_load_to_lds16(voff[q], reinterpret_cast<const float *>(bb),
                         st + wave_b + (q - W::A_DMA) * 1024);
    }
  };

  const uint16_t *is_a, *is_b;  // operands of the step most recently issued
  tile_base(0, is_a, is_b);
  issue(lds_u, is_a, is_b, 0, W::DMA);
  int stage = 0;

  f32x16 acc[W::TBM][W::TBN];
  for (int t = 0; t < my_tiles; ++t) {
    const uint16_t *nt_a, *nt_b;  // the next tile's first step (this tile's on the last)
    tile_base(t + 1 < my_tiles ? t + 1 : t, nt_a, nt_b);
#pragma unroll
    for (int i = 0; i < W::TBM; ++i)
#pragma unroll
      for (int j = 0; j < W::TBN; ++j) acc[i][j] = f32x16{};

    for (int kk = 0; kk < nk; ++kk) {
      const bool last = kk + 1 == nk;
      const uint16_t *ia = last ? nt_a : is_a + W::BK;
      const uint16_t *ib = last ? nt_b : is_b + b_step;
      __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));  // this step's loads (own)
      ks_lds_barrier();                                // everyone's; the other stage free
      const char *st = lds + stage * W::STAGE;
      const unsigned nst = lds_u + (stage ^ 1) * W::STAGE;

      i16x8 a0[W::TBM], a1[W::TBM], b0[W::TBN], b1[W::TBN];
#pragma unroll
      for (int bn = 0; bn < W::TBN; ++bn) b0[bn] = m32_read_b(st, wn, bn, 0, lane);
#pragma unroll
      for (int bm = 0; bm < W::TBM; ++bm) a0[bm] = m32_read_a(st, wm, bm, 0, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kg = 0; kg < W::KG; ++kg) {
        i16x8(&ac)[W::TBM] = (kg & 1) ? a1 : a0;
        i16x8(&an)[W::TBM] = (kg & 1) ? a0 : a1;
        i16x8(&bc)[W::TBN] = (kg & 1) ? b1 : b0;
        i16x8(&bnx)[W::TBN] = (kg & 1) ? b0 : b1;
#pragma unroll
        for (int bm = 0; bm < W::TBM; ++bm) {
#pragma unroll
          for (int bn = 0; bn < W::TBN; ++bn)
            acc[bm][bn] = mfma32x32<FMT>(bc[bn], ac[bm], acc[bm][bn]);
          const int row = kg * W::TBM + bm;
          if (row < 2 * W::TBM) {  // the next step's loads, two per row
            __builtin_amdgcn_sched_barrier(0);
            issue(nst, ia, ib, 2 * row, 2 * row + 2);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (kg + 1 < W::KG && bm == 0) {
            // the next group's fragments, a whole group ahead
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int bn = 0; bn < W::TBN; ++bn) bnx[bn] = m32_read_b(st, wn, bn, kg + 1, lane);
#pragma unroll
            for (int i = 0; i < W::TBM; ++i) an[i] = m32_read_a(st, wm, i, kg + 1, lane);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      is_a = ia;
      is_b = ib;
      stage ^= 1;
#pragma unroll
      for (int i = 0; i < W::TBM; ++i)
#pragma unroll
        for (int j = 0; j < W::TBN; ++j) asm volatile("" : "+a"(acc[i][j]));
    }

    // Lane (l32, h) holds row l32 of each 32 x 32 block and, in registers
    // 4 j .. 4 j + 3, its columns 8 j + 4 h .. + 3.
    int m0, n0;
    origin(t, m0, n0);
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int bm = 0; bm < W::TBM; ++bm) {
      float *crow = p.C + (long long)(m0 + wm * W::WTM + 32 * bm + l32) * p.ldc + n0 +
                    wn * W::WTN + 4 * h;
#pragma unroll
      for (int bn = 0; bn < W::TBN; ++bn)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4u *>(crow + 32 * bn + 8 * j) =
              f32x4{acc[bm][bn][4 * j], acc[bm][bn][4 * j + 1], acc[bm][bn][4 * j + 2],
                    acc[bm][bn][4 * j + 3]};
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait_imm(0));  // the redundant last reload
}

}  // namespace

bool mixed16_fits(const MixedProblem &p) {
  return (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && (p.lda & 7) == 0 && (p.ldb & 7) == 0 &&
         (p.N & 7) == 0 && p.M >= M16::BM && p.N >= M16::BN && p.K > 0 && p.K % M16::BK == 0 &&
         lane_offsets_fit(M16::BM, p.lda, 2) && lane_offsets_fit(M16::BK, p.ldb, 2);
}

hipError_t launch_mixed16(int format, const MixedProblem &p, hipStream_t s, bool mfma32) {
  if (!mixed16_fits(p)) return hipErrorInvalidValue;
  const long long tiles_m = ceil_div(p.M, M16::BM), tiles_n = ceil_div(p.N, M16::BN);
  const long long ntiles = tiles_m * tiles_n;
  if (ntiles > 0x7fffffffLL) return hipErrorInvalidValue;
  if (mfma32) {
    auto kern = format == kMixedBf16 ? mixed32_kernel<kMixedBf16> : mixed32_kernel<kMixedF16>;
    long long grid = format == kMixedBf16 ? resident_workgroups<mixed32_kernel<kMixedBf16>, 256>()
                                          : resident_workgroups<mixed32_kernel<kMixedF16>, 256>();
    if (grid > ntiles) grid = ntiles;
    return launch_kernel(kern, dim3((unsigned)grid), dim3(256), s, p, (int)tiles_m, (int)tiles_n);
  }
  if (format == kMixedBf16) {
    long long grid = resident_workgroups<mixed16_kernel<kMixedBf16>, 256>();
    if (grid > ntiles) grid = ntiles;
    return launch_kernel(mixed16_kernel<kMixedBf16>, dim3((unsigned)grid), dim3(256), s, p,
                         (int)tiles_m, (int)tiles_n);
  }
  long long grid = resident_workgroups<mixed16_kernel<kMixedF16>, 256>();
  if (grid > ntiles) grid = ntiles;
  return launch_kernel(mixed16_kernel<kMixedF16>, dim3((unsigned)grid), dim3(256), s, p,
                       (int)tiles_m, (int)tiles_n);
}

}  // namespace gemm_f32_impl
