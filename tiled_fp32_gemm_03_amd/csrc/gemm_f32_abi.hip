// C-ABI front end of the gemm_f32 library: argument validation, the variant
// ladder and the launch tables.  Validation touches no GPU state, so every
// error is returned before anything is enqueued.
#include "gemm_f32.h"
#include "gemm_internal.hpp"
#include "gemm_mixed.h"

#include <cstdint>
#include <cstdio>
#include <mutex>

using namespace gemm_f32_impl;

// host_plan.hpp repeats the status codes it returns; they must be the ABI's.
static_assert(kOk == GEMM_F32_OK && kInvalidDim == GEMM_F32_INVALID_DIM &&
                  kInvalidLd == GEMM_F32_INVALID_LD && kNullPtr == GEMM_F32_NULL_PTR &&
                  kBadVariant == GEMM_F32_BAD_VARIANT && kMisaligned == GEMM_F32_MISALIGNED &&
                  kBadConfig == GEMM_F32_BAD_CONFIG && kBadArg == GEMM_F32_BAD_ARG,
              "status codes of host_plan.hpp and gemm_f32.h differ");

namespace {

constexpr int kTiledT[GEMM_F32_NUM_VARIANTS] = {0, 16, 0, 32, 4, 32, 0};

thread_local char t_last_error[256] = "";

int launch_status(hipError_t err, const char *what) {
  if (err == hipSuccess) return GEMM_F32_OK;
  std::snprintf(t_last_error, sizeof(t_last_error), "%s: %s (%s)", what,
                hipGetErrorName(err), hipGetErrorString(err));
  return GEMM_F32_LAUNCH_FAILED;
}

int num_configs(int variant) {
  if (variant < 0 || variant >= GEMM_F32_NUM_VARIANTS) return 0;
  if (variant == GEMM_F32_PROD) return prod_num_configs();
  if (variant == GEMM_F32_VALU) return valu_num_configs();
  return 1;
}

int resolve_config(int variant, int config, int M, int N, int K, int *out) {
  if (variant < 0 || variant >= GEMM_F32_NUM_VARIANTS)
    return GEMM_F32_BAD_VARIANT;
  if (config < -1 || config >= num_configs(variant)) return GEMM_F32_BAD_CONFIG;
  if (config == -1) {
    if (variant == GEMM_F32_PROD) config = prod_choose(M, N, K);
    else if (variant == GEMM_F32_VALU) config = valu_choose(M, N, K);
    else config = 0;
  }
  if (variant == GEMM_F32_PROD && !prod_supports(config, M, N, K))
    return GEMM_F32_BAD_CONFIG;
  *out = config;
  return GEMM_F32_OK;
}

int validate(int M, int N, int K, const float *A, int lda, const float *B,
             int ldb, float *C, int ldc, int variant, int config,
             int *chosen) {
  int rc = check_shape(M, N, K);
  if (rc != GEMM_F32_OK) return rc;
  rc = check_ld(N, K, lda, ldb, ldc);
  if (rc != GEMM_F32_OK) return rc;
  rc = resolve_config(variant, config, M, N, K, chosen);
  if (rc != GEMM_F32_OK) return rc;
  return check_pointers(M, N, K, A, B, C, 4);
}

// The checks of the split-K entries, in order, and their plan.
int splitk_validate(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                    float *C, int ldc, int config, int splits, SplitPlan *plan) {
  int rc = check_shape(M, N, K);
  if (rc != GEMM_F32_OK) return rc;
  rc = check_ld(N, K, lda, ldb, ldc);
  if (rc != GEMM_F32_OK) return rc;
  if (splits < 0) return GEMM_F32_BAD_ARG;
  if (!splitk_plan(M, N, K, config, splits, plan)) return GEMM_F32_BAD_CONFIG;
  return GEMM_F32_OK;
}

}  // namespace

extern "C" int gemm_f32_ex(int M, int N, int K, const float *A, int lda,
                           const float *B, int ldb, float *C, int ldc,
                           int variant, int config, void *stream) {
  int chosen = 0;
  int rc = validate(M, N, K, A, lda, B, ldb, C, ldc, variant, config, &chosen);
  if (rc != GEMM_F32_OK) return rc;
  if (M == 0 || N == 0) return GEMM_F32_OK;

  const Problem p{M, N, K, A, lda, B, ldb, C, ldc};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return launch_status(launch_zero(p, s), "zero fill");  // the empty sum
  if (variant == GEMM_F32_NAIVE) return launch_status(launch_naive(p, s), "naive");
  if (variant == GEMM_F32_PROD) return launch_status(launch_prod(chosen, p, s), "prod");
  if (variant == GEMM_F32_VALU) return launch_status(launch_valu(chosen, p, s), "valu");
  return launch_status(
      launch_tiled(kTiledT[variant], variant == GEMM_F32_TILED32_PAD, p, s), "tiled");
}

extern "C" int gemm_f32(int M, int N, int K, const float *A, int lda,
                        const float *B, int ldb, float *C, int ldc,
                        int variant, void *stream) {
  return gemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, variant, -1, stream);
}

extern "C" int gemm_f32_num_configs(int variant) { return num_configs(variant); }

extern "C" int gemm_f32_tile(int variant, int config, int M, int N, int K,
                             int *BM, int *BN, int *BK, int *threads,
                             int *chosen_config) {
  int rc = check_shape(M, N, K);
  if (rc != GEMM_F32_OK) return rc;
  int chosen = 0;
  rc = resolve_config(variant, config, M, N, K, &chosen);
  if (rc != GEMM_F32_OK) return rc;
  int bm, bn, bk, nt;
  if (variant == GEMM_F32_NAIVE) {
    bm = 4, bn = 64, bk = 1, nt = 256;
  } else if (variant == GEMM_F32_PROD) {
    const ProdConfig &c = prod_config(chosen);
    bm = prod_kind(chosen) == kStrip ? strip_rows(M) : c.BM;
    bn = prod_kind(chosen) == kStripN ? strip_cols(N) : c.BN;
    bk = c.BK, nt = 64 * c.WGM * c.WGN;
  } else if (variant == GEMM_F32_VALU) {
    bm = bn = kValuTile, bk = valu_config_bk(chosen), nt = kValuThreads;
  } else {
    const int t = kTiledT[variant];
    bm = bn = bk = t, nt = t * t;
  }
  if (BM) *BM = bm;
  if (BN) *BN = bn;
  if (BK) *BK = bk;
  if (threads) *threads = nt;
  if (chosen_config) *chosen_config = chosen;
  return GEMM_F32_OK;
}

// ---- split-K ---------------------------------------------------------------

extern "C" int gemm_f32_splitk_plan(int M, int N, int K, int config, int splits,
                                    int *config_out, int *splits_out, int *kc_out,
                                    long long *workspace_bytes) {
  int rc = check_shape(M, N, K);
  if (rc != GEMM_F32_OK) return rc;
  if (splits < 0) return GEMM_F32_BAD_ARG;
  SplitPlan plan;
  if (!splitk_plan(M, N, K, config, splits, &plan)) return GEMM_F32_BAD_CONFIG;
  if (config_out) *config_out = plan.config;
  if (splits_out) *splits_out = plan.splits;
  if (kc_out) *kc_out = plan.kc;
  if (workspace_bytes) *workspace_bytes = plan.workspace_bytes;
  return GEMM_F32_OK;
}

extern "C" int gemm_f32_splitk(int M, int N, int K, const float *A, int lda, const float *B,
                               int ldb, float *C, int ldc, int config, int splits,
                               void *workspace, long long workspace_bytes, void *stream) {
  SplitPlan plan;
  int rc = splitk_validate(M, N, K, A, lda, B, ldb, C, ldc, config, splits, &plan);
  if (rc != GEMM_F32_OK) return rc;
  if (M == 0 || N == 0) return GEMM_F32_OK;
  rc = check_pointers(M, N, K, A, B, C, 4);
  if (rc != GEMM_F32_OK) return rc;
  if (plan.workspace_bytes > 0 &&
      (bad_buffer(workspace) || workspace_bytes < plan.workspace_bytes))
    return GEMM_F32_BAD_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Problem p{M, N, K, A, lda, B, ldb, C, ldc};
  if (K == 0) return launch_status(launch_zero(p, s), "zero fill");
  return launch_status(launch_prod_split(plan, p, static_cast<float *>(workspace), s), "splitk");
}

// ---- split-K without allocation ---------------------------------------------
//
// The slabs of the split-K path live in `scratch`, a file-scope device array
// of GEMM_F32_NOALLOC_SCRATCH_BYTES on every GPU the library runs on (each
// device holds its own copy until the process ends).  In host code the
// array's name is not a device address: the address is taken once per
// device with hipGetSymbolAddress, with that device current, and only that
// pointer is handed to kernels.  Every call on one device shares its array;
// the split kernels overwrite each slab element they later sum, so nothing
// has to be cleared between calls, but calls that overlap in time on one
// device race on it.

namespace {

constexpr long long kScratchBytes = GEMM_F32_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) float scratch[kScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch[kMaxDevices];  // per device, set once under g_scratch_mu

// This device's copy of `scratch`, looked up on the device's first call.
int scratch_for_device(int dev, float **out) {
  if (dev < 0 || dev >= kMaxDevices) return GEMM_F32_BAD_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return launch_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch address");
    g_scratch[dev] = static_cast<float *>(ptr);
  }
  *out = g_scratch[dev];
  return GEMM_F32_OK;
}

}  // namespace

extern "C" int gemm_f32_splitk_noalloc(int M, int N, int K, const float *A, int lda,
                                       const float *B, int ldb, float *C, int ldc, int config,
                                       int splits, void *stream) {
  SplitPlan plan;
  int rc = splitk_validate(M, N, K, A, lda, B, ldb, C, ldc, config, splits, &plan);
  if (rc != GEMM_F32_OK) return rc;
  if (plan.workspace_bytes > kScratchBytes) return GEMM_F32_SCRATCH_TOO_SMALL;
  if (M == 0 || N == 0) return GEMM_F32_OK;
  rc = check_pointers(M, N, K, A, B, C, 4);
  if (rc != GEMM_F32_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The stream's device must be the current one: the scratch address is
  // looked up with that device current.
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_F32_BAD_ARG;
  if (s != nullptr) {
    if (hipStreamGetDevice(s, &sdev) != hipSuccess || sdev != dev) return GEMM_F32_BAD_ARG;
  }
  const Problem p{M, N, K, A, lda, B, ldb, C, ldc};
  if (K == 0) return launch_status(launch_zero(p, s), "zero fill");
  float *ws = nullptr;
  if (plan.workspace_bytes > 0) {
    rc = scratch_for_device(dev, &ws);
    if (rc != GEMM_F32_OK) return rc;
  }
  return launch_status(launch_prod_split(plan, p, ws, s), "splitk noalloc");
}

// ---- 16-bit inputs ---------------------------------------------------------

namespace {

int mixed_resolve(int config, int M, int N, int K, int *out) {
  if (config < -1 || config >= mixed_num_configs()) return GEMM_F32_BAD_CONFIG;
  *out = config == -1 ? mixed_choose(M, N, K) : config;
  return GEMM_F32_OK;
}

}  // namespace

extern "C" int gemm_mixed(int M, int N, int K, const void *A, int lda, const void *B,
                          int ldb, float *C, int ldc, int format, int config,
                          void *stream) {
  int rc = check_shape(M, N, K);
  if (rc != GEMM_F32_OK) return rc;
  rc = check_ld(N, K, lda, ldb, ldc);
  if (rc != GEMM_F32_OK) return rc;
  if (format != GEMM_MIXED_BF16 && format != GEMM_MIXED_F16) return GEMM_F32_BAD_ARG;
  int chosen = 0;
  rc = mixed_resolve(config, M, N, K, &chosen);
  if (rc != GEMM_F32_OK) return rc;
  if (M == 0 || N == 0) return GEMM_F32_OK;
  rc = check_pointers(M, N, K, A, B, C, 2);
  if (rc != GEMM_F32_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return launch_status(launch_zero_f32(C, M, N, ldc, s), "zero fill");
  const MixedProblem p{M, N, K, static_cast<const uint16_t *>(A), lda,
                       static_cast<const uint16_t *>(B), ldb, C, ldc};
  return launch_status(
      launch_mixed(format == GEMM_MIXED_BF16 ? kMixedBf16 : kMixedF16, chosen, p, s),
      "mixed");
}

extern "C" int gemm_mixed_num_configs(void) { return mixed_num_configs(); }

extern "C" int gemm_mixed_tile(int config, int M, int N, int K, int *BM, int *BN, int *BK,
                               int *threads, int *chosen_config) {
  int rc = check_shape(M, N, K);
  if (rc != GEMM_F32_OK) return rc;
  int chosen = 0;
  rc = mixed_resolve(config, M, N, K, &chosen);
  if (rc != GEMM_F32_OK) return rc;
  const MixedConfig &c = mixed_config(chosen);
  if (BM) *BM = c.BM;
  if (BN) *BN = c.BN;
  if (BK) *BK = c.BK;
  if (threads) *threads = 64 * c.WGM * c.WGN;
  if (chosen_config) *chosen_config = chosen;
  return GEMM_F32_OK;
}

extern "C" const char *gemm_f32_last_error(void) { return t_last_error; }

extern "C" const char *gemm_f32_status_string(int status) {
  switch (status) {
    case GEMM_F32_OK: return "ok";
    case GEMM_F32_INVALID_DIM: return "invalid dimension: M, N and K must be >= 0";
    case GEMM_F32_INVALID_LD:
      return "invalid leading dimension: need lda >= max(1,K), ldb >= max(1,N), ldc >= max(1,N)";
    case GEMM_F32_NULL_PTR: return "null pointer for a non-empty matrix";
    case GEMM_F32_BAD_VARIANT: return "unknown variant";
    case GEMM_F32_LAUNCH_FAILED: return "kernel launch failed";
    case GEMM_F32_MISALIGNED: return "pointer not aligned to its element size";
    case GEMM_F32_BAD_CONFIG:
      return "launch-table index out of range or not valid for this shape";
    case GEMM_F32_BAD_ARG: return "invalid argument";
    case GEMM_F32_BAD_WORKSPACE:
      return "split-K workspace missing, smaller than the plan needs, or not 4-byte aligned";
    case GEMM_F32_SCRATCH_TOO_SMALL:
      return "the split-K plan needs more than the library's fixed scratch array holds";
    default: return "unknown status";
  }
}

extern "C" const char *gemm_f32_version(void) { return "gemm_f32 0.1.0 gfx950"; }
