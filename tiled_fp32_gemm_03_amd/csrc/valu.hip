// Register-blocked VALU rung: the pages' "one thread computes several
// outputs" step (geek-doc.cn "矩阵乘法 tiling", sections 三 and 五: raise the
// reuse of each staged element beyond BLOCK by giving each thread a small
// block of outputs) on the vector ALU, without matrix cores.
//
// Workgroup: 256 threads own a 128 x 128 tile of C.  Thread (ty, tx) of the
// 16 x 16 grid owns the four 4 x 4 blocks at rows {4ty, 64 + 4ty} and
// columns {4tx, 64 + 4tx}: 64 fp32 accumulators in registers.  Per k the
// thread reads 8 A values and 8 B values from LDS as four 128-bit reads and
// does 64 FMAs.  A is staged k-major (transposed on its way into LDS) so the
// 4 rows a thread needs are contiguous; B is staged as it lies in memory.
// Two LDS stages, one barrier per BK-deep step, register prefetch of the
// next step's tiles.  Out-of-range elements are loaded as 0 and out-of-range
// outputs are not stored (geek-doc.cn section 六; mayulu.co section 7).
//
// Roof: the fp32 vector peak, 157.3 TFLOP/s.  A gfx950 SIMD retires one
// wave64 v_fmac_f32 every two cycles, so the plain (non-packed) FMA reaches
// it; the vector-FMA probe measures it.  A single wave cannot issue that
// often, so the rate also depends on how many waves each SIMD holds, which
// is what the launch-table entries below trade against unrolling.
#include "gemm_internal.hpp"
#include "launch_util.hpp"

namespace gemm_f32_impl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kVT = kValuTile;      // tile edge
constexpr int kVPad = 4;            // floats after each LDS row
constexpr int kVS = kVT + kVPad;
constexpr int kVThreads = kValuThreads;
static_assert(kVT == 128 && kVThreads == 256,
              "thread-to-element maps below assume 128 x 128 tiles and 256 threads");

// One k step of BK (8 or 16) staged through registers: BK / 8 chunks of 4
// floats of A and of B per thread.  Chunk j of thread tid is A chunk
// tid + 256 j of the tile's 128 rows x BK / 4 chunks and B chunk tid + 256 j
// of its BK rows x 32 chunks.
template <int BK>
struct ValuStage {
  static constexpr int CH = BK / 8;
  f32x4 a[CH];  // A[m][k0 + 4c .. +3] for this thread's (m, c)
  f32x4 b[CH];  // B[k][n .. n+3] for this thread's (k, n)
};

template <int BK>
__device__ inline void valu_a_chunk(int j, int tid, int &am, int &ac) {
  const int c = tid + kVThreads * j;
  am = c / (BK / 4);
  ac = (c % (BK / 4)) * 4;
}
__device__ inline void valu_b_chunk(int j, int tid, int &bk, int &bn) {
  const int c = tid + kVThreads * j;
  bk = c >> 5;
  bn = (c & 31) * 4;
}

template <int BK, bool GUARD>
__device__ inline void valu_load(ValuStage<BK> &st, const Problem &p, int m0, int n0,
                                 int k0, int tid) {
#pragma unroll
  for (int j = 0; j < ValuStage<BK>::CH; ++j) {
    int am, ac, bk, bn;
    valu_a_chunk<BK>(j, tid, am, ac);
    valu_b_chunk(j, tid, bk, bn);
    const int gm = m0 + am, gka = k0 + ac;
    const int gkb = k0 + bk, gn = n0 + bn;
    const float *pa = p.A + (long long)gm * p.lda + gka;
    const float *pb = p.B + (long long)gkb * p.ldb + gn;
    if (!GUARD) {
      st.a[j] = *reinterpret_cast<const f32x4u *>(pa);
      st.b[j] = *reinterpret_cast<const f32x4u *>(pb);
    } else {
      f32x4 a{0.f, 0.f, 0.f, 0.f}, b{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (gm < p.M && gka + e < p.K) a[e] = pa[e];
        if (gkb < p.K && gn + e < p.N) b[e] = pb[e];
      }
      st.a[j] = a;
      st.b[j] = b;
    }
  }
}

template <int BK>
__device__ inline void valu_store_lds(const ValuStage<BK> &st, float *as, float *bs, int tid) {
#pragma unroll
  for (int j = 0; j < ValuStage<BK>::CH; ++j) {
    int am, ac, bk, bn;
    valu_a_chunk<BK>(j, tid, am, ac);
    valu_b_chunk(j, tid, bk, bn);
#pragma unroll
    for (int e = 0; e < 4; ++e) as[(ac + e) * kVS + am] = st.a[j][e];  // transposed
    *reinterpret_cast<f32x4 *>(bs + bk * kVS + bn) = st.b[j];
  }
}

// KUNROLL: how many of the BK k values the compiler may unroll, i.e. how far
// LDS reads run ahead of the FMAs; fewer live fragments means fewer VGPRs.
// WAVES: waves per SIMD the register allocation must allow.  BK: the k
// step, i.e. how many k share one barrier and one round of staging.
template <int KUNROLL, int WAVES, int kVBK>
__global__ void __launch_bounds__(kVThreads) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES)))
    valu_kernel(Problem p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) float as[2][kVBK * kVS];
  __shared__ __attribute__((aligned(16))) float bs[2][kVBK * kVS];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const long long ntiles = (long long)tiles_m * tiles_n;
  const int nk = (p.K + kVBK - 1) / kVBK;

  for (long long t = blockIdx.x; t < ntiles; t += gridDim.x) {
    // An overhanging last tile row or column is moved back to end at C's
    // edge (when C is at least one tile wide); the overlap with its
    // neighbour is stored twice with identical values (every element is one
    // FMA chain in ascending k), and the tile needs no guarded loads.
    int m0 = (int)(t / tiles_n) * kVT, n0 = (int)(t % tiles_n) * kVT;
    if (m0 + kVT > p.M && p.M >= kVT) m0 = p.M - kVT;
    if (n0 + kVT > p.N && p.N >= kVT) n0 = p.N - kVT;
    const bool interior = m0 + kVT <= p.M && n0 + kVT <= p.N;
    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    ValuStage<kVBK> st;
    if (interior && kVBK <= p.K) valu_load<kVBK, false>(st, p, m0, n0, 0, tid);
    else valu_load<kVBK, true>(st, p, m0, n0, 0, tid);
    valu_store_lds(st, as[0], bs[0], tid);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        const int k1 = (kt + 1) * kVBK;
        if (interior && k1 + kVBK <= p.K) valu_load<kVBK, false>(st, p, m0, n0, k1, tid);
        else valu_load<kVBK, true>(st, p, m0, n0, k1, tid);
      }
      const float *a_s = as[cur];
      const float *b_s = bs[cur];
#pragma unroll KUNROLL
      for (int k = 0; k < kVBK; ++k) {
        const f32x4 a0 = *reinterpret_cast<const f32x4 *>(a_s + k * kVS + 4 * ty);
        const f32x4 a1 = *reinterpret_cast<const f32x4 *>(a_s + k * kVS + 64 + 4 * ty);
        const f32x4 b0 = *reinterpret_cast<const f32x4 *>(b_s + k * kVS + 4 * tx);
        const f32x4 b1 = *reinterpret_cast<const f32x4 *>(b_s + k * kVS + 64 + 4 * tx);
        const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
      }
      if (more) valu_store_lds(st, as[cur ^ 1], bs[cur ^ 1], tid);
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
      if (row >= p.M) continue;
      float *crow = p.C + (long long)row * p.ldc;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = n0 + 64 * h + 4 * tx;
        const f32x4 v{acc[i][4 * h], acc[i][4 * h + 1], acc[i][4 * h + 2], acc[i][4 * h + 3]};
        if (col + 4 <= p.N) {
          *reinterpret_cast<f32x4u *>(crow + col) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < p.N) crow[col + e] = v[e];
        }
      }
    }
  }
}

// Launch table: the same tile and thread map, compiled for different
// register budgets.  Waves per SIMD is what decides this kernel's speed: a
// single wave issues a vector instruction only every few cycles, so the
// vector ALU needs several resident waves per SIMD to stay busy.
struct ValuEntry {
  int kunroll, waves, bk;
};
constexpr ValuEntry kValuEntries[] = {
    {8, 2, 8},   // 0: fully unrolled k step, ~232 VGPRs, 2 waves per SIMD
    {1, 4, 8},   // 1: rolled k loop, 118 VGPRs, 4 waves per SIMD
    {2, 3, 8},   // 2: k loop unrolled by 2, 3 waves per SIMD
    {4, 4, 8},   // 3: k loop unrolled by 4 under a 4-wave budget
    {4, 4, 16},  // 4: entry 3 with 16-deep steps (half the barriers)
    {2, 4, 16},  // 5: 16-deep steps, k loop unrolled by 2
};
constexpr int kValuNumEntries = sizeof(kValuEntries) / sizeof(kValuEntries[0]);

template <int E>
hipError_t launch_valu_entry(dim3 grid, const Problem &p, int tiles_m, int tiles_n,
                             hipStream_t s) {
  constexpr ValuEntry e = kValuEntries[E];
  return launch_kernel(valu_kernel<e.kunroll, e.waves, e.bk>, grid, dim3(kVThreads), s, p,
                       tiles_m, tiles_n);
}

}  // namespace

int valu_num_configs() { return kValuNumEntries; }

int valu_config_bk(int index) { return kValuEntries[index].bk; }
// Entry 5: best or within run-to-run spread of the best on the measured
// workloads (4096^3 87.7 TFLOP/s against 86.1 for entry 3 and 88.6 for
// entry 0; 4097 x 4095 x 2049 71.8; 16384 x 16384 x 64 76.4).
int valu_choose(int M, int N, int K) { return 5; }

hipError_t launch_valu(int index, const Problem &p, hipStream_t s) {
  const long long tiles_m = ceil_div(p.M, kVT), tiles_n = ceil_div(p.N, kVT);
  if (tiles_m > 0x7fffffffLL || tiles_n > 0x7fffffffLL) return hipErrorInvalidValue;
  long long grid = tiles_m * tiles_n;
  const long long cap = 1LL << 20;  // the kernel loops over tiles beyond this
  if (grid > cap) grid = cap;
  const dim3 g((unsigned)grid);
  switch (index) {
    case 0: return launch_valu_entry<0>(g, p, (int)tiles_m, (int)tiles_n, s);
    case 1: return launch_valu_entry<1>(g, p, (int)tiles_m, (int)tiles_n, s);
    case 2: return launch_valu_entry<2>(g, p, (int)tiles_m, (int)tiles_n, s);
    case 3: return launch_valu_entry<3>(g, p, (int)tiles_m, (int)tiles_n, s);
    case 4: return launch_valu_entry<4>(g, p, (int)tiles_m, (int)tiles_n, s);
    case 5: return launch_valu_entry<5>(g, p, (int)tiles_m, (int)tiles_n, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gemm_f32_impl
