// The 192x192 member of the 128x128-wave kernel family (big16_kernel with
// 96x96 wave tiles): 4 waves, one per SIMD, each computing 6 x 6 blocks of
// v_mfma_f32_16x16x4_f32 over 32-deep steps of direct loads.  It covers
// products whose tile count leaves 256x256 tiles a partial last round
// (3072^3 is exactly one round of 192x192 tiles, 6144^3 four).
//
// This translation unit is built with the MFMAs in their VGPR form
// (accumulators in ordinary VGPRs; the build passes
// -mllvm -amdgpu-mfma-vgpr-form=1 for this file only): with 144
// accumulators per lane, the accumulation-register form makes the register
// allocator move accumulators between register files every step, while all
// of them fit in VGPRs beside the fragments.  The 256x256 members stay in
// prod.hip, in the accumulation-register form.
#include "w16_tiles.hpp"

namespace gemm_f32_impl {

using W192 = W16<96, 96, 32, 2>;

bool big16_192_fits(const Problem &p) {
  return (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && (p.lda & 3) == 0 && (p.ldb & 3) == 0 &&
         (p.N & 3) == 0 && p.M >= W192::BM && p.N >= W192::BN && p.K > 0 &&
         p.K % W192::BK == 0 && p.lda < (1 << 24) && p.ldb < (1 << 24);
}

hipError_t launch_big16_192(const Problem &p, hipStream_t s) {
  if (!big16_192_fits(p)) return hipErrorInvalidValue;
  return launch_big16_grid<W192, big16_kernel<W192>>(p, s);
}

}  // namespace gemm_f32_impl
