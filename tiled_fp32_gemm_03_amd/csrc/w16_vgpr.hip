// Members of the 16x16-MFMA direct-load kernel family (big16_kernel) whose
// accumulators fit in VGPRs beside their fragments:
//   192x192 tiles on 96x96 waves, 32-deep steps (144 accumulators per lane),
//     for products whose tile count leaves 256x256 tiles a partial last
//     round (3072^3 is exactly one round of 192x192 tiles, 6144^3 four);
//   128x128 tiles on 64x64 waves, 32-deep steps (64 accumulators, 64 KB of
//     LDS, two workgroups per CU), for mid-size products, and in split-K
//     form for products with few output tiles;
//   192x256 tiles on 96x128 waves, 32-deep steps (192 accumulators, 112 KB
//     of LDS), for products whose 256x256 tiles leave a partial last round
//     and whose 192x256 tiles do not (3072x4096 is one round, 6144^2 three).
//
// This translation unit is built with the MFMAs in their VGPR form
// (-mllvm -amdgpu-mfma-vgpr-form=1, for this file only): with fewer than
// 256 accumulators per lane the accumulation-register form lets the
// register allocator move accumulators between the register files every
// step.  The 256x256 members (256 accumulators) stay in prod.hip in the
// accumulation-register form.
#include "w16_tiles.hpp"

namespace gemm_f32_impl {
namespace {

using W192 = W16<96, 96, 32, 2>;
using W128 = W16<64, 64, 32, 2>;
using W192x256 = W16<96, 128, 32, 2>;

// Direct loads need 16-byte aligned rows of A and B and N % 4 == 0; the
// kernel needs C at least one tile each way, K a positive multiple of the
// step and 32-bit lane offsets for its A tile and B step (lane_offsets_fit).
template <class W>
bool direct_fits(const Problem &p) {
  return (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && (p.lda & 3) == 0 && (p.ldb & 3) == 0 &&
         (p.N & 3) == 0 && p.M >= W::BM && p.N >= W::BN && p.K > 0 && p.K % W::BK == 0 &&
         lane_offsets_fit(W::BM, p.lda, 4) && lane_offsets_fit(W::BK, p.ldb, 4);
}

}  // namespace

bool big16_192_fits(const Problem &p) { return direct_fits<W192>(p); }

hipError_t launch_big16_192(const Problem &p, hipStream_t s) {
  if (!direct_fits<W192>(p)) return hipErrorInvalidValue;
  return launch_big16_grid<W192, big16_kernel<W192>>(p, s);
}

bool big16_192x256_fits(const Problem &p) { return direct_fits<W192x256>(p); }

hipError_t launch_big16_192x256(const Problem &p, hipStream_t s) {
  if (!direct_fits<W192x256>(p)) return hipErrorInvalidValue;
  return launch_big16_grid<W192x256, big16_kernel<W192x256>>(p, s);
}

bool big16_128_fits(const Problem &p) { return direct_fits<W128>(p); }

hipError_t launch_big16_128(const Problem &p, hipStream_t s) {
  if (!direct_fits<W128>(p)) return hipErrorInvalidValue;
  return launch_big16_grid<W128, big16_kernel<W128>>(p, s);
}

bool big16_128_split_fits(const Problem &p, int kc) {
  return direct_fits<W128>(p) && kc > 0 && kc % W128::BK == 0;
}

hipError_t launch_big16_128_split(const Problem &p, int splits, int kc, float *ws,
                                  hipStream_t s) {
  if (!big16_128_split_fits(p, kc)) return hipErrorInvalidValue;
  const long long tiles_m = ceil_div(p.M, W128::BM), tiles_n = ceil_div(p.N, W128::BN);
  const long long ntiles = tiles_m * tiles_n;
  if (ntiles > 0x7fffffffLL || splits < 1 || splits > kMaxGridY) return hipErrorInvalidValue;
  return launch_kernel(big16_split_kernel<W128>, dim3((unsigned)ntiles, (unsigned)splits),
                       dim3(256), s, p, (int)tiles_m, (int)tiles_n, kc, ws);
}

}  // namespace gemm_f32_impl
