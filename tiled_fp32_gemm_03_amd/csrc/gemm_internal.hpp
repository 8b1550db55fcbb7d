// Internal declarations shared by the kernel translation units and the C-ABI
// front end of the gemm_f32 library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "host_plan.hpp"

namespace gemm_f32_impl {

// One product C = A x B, row-major with leading dimensions (elements).
struct Problem {
  int M, N, K;
  const float *A;
  long long lda;
  const float *B;
  long long ldb;
  float *C;
  long long ldc;
};

hipError_t launch_zero(const Problem &p, hipStream_t s);
hipError_t launch_naive(const Problem &p, hipStream_t s);
hipError_t launch_tiled(int T, bool padded, const Problem &p, hipStream_t s);

// Register-blocked VALU kernel: 128 x 128 tiles, 256 threads, k step 8; its
// launch-table entries differ only in register budget.
constexpr int kValuTile = 128, kValuThreads = 256;
int valu_num_configs();
int valu_config_bk(int index);  // the k step of launch-table entry `index`
int valu_choose(int M, int N, int K);
hipError_t launch_valu(int index, const Problem &p, hipStream_t s);

// One product with 16-bit inputs (codes of kMixedBf16 or kMixedF16) and an
// fp32 result, row-major with leading dimensions (elements).
struct MixedProblem {
  int M, N, K;
  const uint16_t *A;
  long long lda;
  const uint16_t *B;
  long long ldb;
  float *C;
  long long ldc;
};

constexpr int kMixedBf16 = 0, kMixedF16 = 1;

struct MixedConfig {
  int BM, BN, BK;
  int WGM, WGN;   // waves along M and N (threads = 64 * WGM * WGN)
  int occupancy;  // workgroups per CU that fit in LDS
  const char *name;
};

// The 16x16x32-MFMA kernel with direct loads (mixed16.hip): whether it
// takes the product (16-byte aligned rows of A and B, N % 8 == 0, C at least
// 256 x 256, K a positive multiple of 64, 32-bit lane offsets: lane_offsets_fit),
// and its launch.
bool mixed16_fits(const MixedProblem &p);
hipError_t launch_mixed16(int format, const MixedProblem &p, hipStream_t s, bool mfma32);

int mixed_num_configs();
const MixedConfig &mixed_config(int index);
int mixed_choose(int M, int N, int K);
hipError_t launch_mixed(int format, int index, const MixedProblem &p, hipStream_t s);
hipError_t launch_zero_f32(float *C, int M, int N, long long ldc, hipStream_t s);

// The 192x192, 192x256 and 128x128 direct-load kernels (w16_vgpr.hip): whether each
// takes the product (16-byte aligned rows of A and B, N % 4 == 0, C at
// least one tile each way, K a positive multiple of 32, 32-bit lane offsets:
// lane_offsets_fit), and its launch.
bool big16_192_fits(const Problem &p);
hipError_t launch_big16_192(const Problem &p, hipStream_t s);
bool big16_192x256_fits(const Problem &p);
hipError_t launch_big16_192x256(const Problem &p, hipStream_t s);
bool big16_128_fits(const Problem &p);
hipError_t launch_big16_128(const Problem &p, hipStream_t s);
// Split-K form of the 128x128 kernel: grid row y computes k in
// [y kc, (y + 1) kc) into slab y of ws (M x N, row pitch N); kc must be a
// multiple of 32 and the product must fit as above.  The slabs are summed
// by the caller.
bool big16_128_split_fits(const Problem &p, int kc);
hipError_t launch_big16_128_split(const Problem &p, int splits, int kc, float *ws,
                                  hipStream_t s);

// One product on production launch-table entry `index` (host_plan.hpp holds
// the table, the automatic choice and the split-K plan), and the split-K
// form of a plan: each chunk's partial product into its own M x N slab of
// `ws`, then the slabs summed in chunk order into C.
hipError_t launch_prod(int index, const Problem &p, hipStream_t s);
hipError_t launch_prod_split(const SplitPlan &plan, const Problem &p, float *ws, hipStream_t s);

}  // namespace gemm_f32_impl
