// Measurement probes: HBM streaming passes (copy, fill and the pages' vector
// add, mayulu.co "CUDA 编程系列之三", section 4) and fp32 MFMA and vector-ALU
// FMA throughput loops.  They give the roofline's measured denominators and a copy kernel of
// known traffic for counter calibration; they are not part of C = A x B.
#include "gemm_f32.h"
#include "gemm_f32_probes.h"
#include "launch_util.hpp"

#include <cstdint>

using namespace gemm_f32_impl;

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kStreamThreads = 256;

template <int KIND>
__global__ void __launch_bounds__(kStreamThreads)
    stream_kernel(long long n4, const f32x4 *__restrict__ x,
                  const f32x4 *__restrict__ y, f32x4 *__restrict__ z) {
  const long long stride = (long long)gridDim.x * kStreamThreads;
  for (long long i = (long long)blockIdx.x * kStreamThreads + threadIdx.x;
       i < n4; i += stride) {
    if constexpr (KIND == GEMM_F32_PROBE_COPY) {
      z[i] = x[i];
    } else if constexpr (KIND == GEMM_F32_PROBE_FILL) {
      z[i] = f32x4{1.f, 1.f, 1.f, 1.f};
    } else {
      z[i] = x[i] + y[i];
    }
  }
}

// Tail (n % 4 elements) handled by one small scalar launch.
template <int KIND>
__global__ void stream_tail(long long start, long long n, const float *x,
                            const float *y, float *z) {
  const long long i = start + threadIdx.x;
  if (i >= n) return;
  if constexpr (KIND == GEMM_F32_PROBE_COPY) {
    z[i] = x[i];
  } else if constexpr (KIND == GEMM_F32_PROBE_FILL) {
    z[i] = 1.f;
  } else {
    z[i] = x[i] + y[i];
  }
}

constexpr int kMfmaChains = 8;
constexpr int kMfmaThreads = 256;

__global__ void __launch_bounds__(kMfmaThreads)
    mfma_probe_kernel(int iters, float *out) {
  const int lane = threadIdx.x & 63;
  float a = 1.0f + lane * 1e-3f;
  float b = 1.0f - lane * 1e-3f;
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (lane == 0) out[blockIdx.x * (kMfmaThreads / 64) + (threadIdx.x >> 6)] = s;
}

// bf16 matrix-core throughput at one wave per SIMD (256 threads per
// workgroup), the occupancy of the 16-bit rung's direct-load kernels: each
// wave runs `iters` rounds of CH16 independent v_mfma_f32_16x16x32_bf16
// chains (SHAPE 16) or CH32 independent v_mfma_f32_32x32x16_bf16 chains
// (SHAPE 32) on register operands.  The operands are small positive
// values, so the accumulators grow by a bounded amount per round and stay
// finite for any iteration count.
constexpr int kMfma16Threads = 256;
constexpr int kMfma16Chains16 = 32, kMfma16Chains32 = 8;
typedef __bf16 bf16x8p __attribute__((ext_vector_type(8)));
typedef float f32x4p __attribute__((ext_vector_type(4)));

template <int SHAPE>
__global__ void __launch_bounds__(kMfma16Threads) mfma16_probe_kernel(int iters, float *out) {
  const int lane = threadIdx.x & 63;
  bf16x8p a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(1e-3f * (1 + ((lane + j) & 7)));
    b[j] = (__bf16)(1e-3f * (1 + ((lane + 3 * j) & 7)));
  }
  float s = 0.f;
  if constexpr (SHAPE == 16) {
    f32x4p acc[kMfma16Chains16];
#pragma unroll
    for (int c = 0; c < kMfma16Chains16; ++c) acc[c] = f32x4p{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kMfma16Chains16; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kMfma16Chains16; ++c) s += acc[c][0] + acc[c][3];
  } else {
    f32x16 acc[kMfma16Chains32];
#pragma unroll
    for (int c = 0; c < kMfma16Chains32; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kMfma16Chains32; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kMfma16Chains32; ++c) s += acc[c][0] + acc[c][15];
  }
  if (lane == 0) out[blockIdx.x * (kMfma16Threads / 64) + (threadIdx.x >> 6)] = s;
}

constexpr int kValuChains = 16;
constexpr int kValuRounds = 8;  // rounds per loop trip, so the branch is rare
constexpr int kValuThreads = 256;

// Independent scalar FMA chains per lane, acc = x * y + acc with x and y in
// registers: the v_fmac_f32 form a register-blocked GEMM issues (never the
// packed form: the library is built with packed fp32 disabled).  The chains
// grow by about 1e-6 per round, so values stay finite for any iteration count.
__global__ void __launch_bounds__(kValuThreads)
    valu_probe_kernel(int iters, float *out) {
  const int lane = threadIdx.x & 63;
  const float x = 1e-3f + lane * 1e-7f;
  const float y = 1e-3f - lane * 1e-7f;
  float acc[kValuChains];
#pragma unroll
  for (int c = 0; c < kValuChains; ++c) acc[c] = (float)c;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < kValuRounds; ++r)
#pragma unroll
      for (int c = 0; c < kValuChains; ++c) acc[c] = __builtin_fmaf(x, y, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kValuChains; ++c) s += acc[c];
  if (lane == 0) out[blockIdx.x * (kValuThreads / 64) + (threadIdx.x >> 6)] = s;
}

constexpr int kLdsThreads = 256;
constexpr int kLdsVecs = 4096;  // 64 KiB of float4 per workgroup
constexpr int kLdsReadsPerTrip = 8;

// 128-bit LDS reads, conflict-free (consecutive lanes read consecutive
// 16-byte words).  Each trip issues 8 independent reads 4 KiB apart and
// folds them into a running sum; the window slides by one word per trip so
// no read repeats an address of the trip before.
__global__ void __launch_bounds__(kLdsThreads) lds_probe_kernel(int iters, float *out) {
  __shared__ f32x4 buf[kLdsVecs];
  const int tid = threadIdx.x;
  for (int i = tid; i < kLdsVecs; i += kLdsThreads) buf[i] = f32x4{1.f, 0.f, 0.f, 0.f} * (float)(i & 7);
  __syncthreads();
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  int base = 0;
  for (int it = 0; it < iters; ++it) {
    const f32x4 *p = buf + tid + base;  // highest index 255 + 255 + 7 * 256 < kLdsVecs
#pragma unroll
    for (int r = 0; r < kLdsReadsPerTrip; ++r) acc += p[r * kLdsThreads];
    base = (base + 1) & (kLdsThreads - 1);
  }
  const float s = acc[0] + acc[1] + acc[2] + acc[3];
  if ((tid & 63) == 0) out[blockIdx.x * (kLdsThreads / 64) + (tid >> 6)] = s;
}

// Matrix-core work and C-sized stores at the ratio of a K = 64 product:
// each wave runs `trips` rounds of 16 independent v_mfma_f32_16x16x4_f32
// (16 x 2048 FLOP) followed by one 128-bit store per lane (1 KB per wave),
// i.e. 32 FLOP per stored byte, the intensity K / 2 of a product whose time
// is its output.  The stores of round t from all waves fill one contiguous
// run of waves KB, so the output is written once, front to back.  MODE 1
// drops the stores (the matrix work alone), MODE 2 drops the MFMAs (the
// stores alone).  Each wave also reports its shader-clock cycles
// (s_memtime) and its constant 100 MHz real-time ticks (s_memrealtime) over
// the loop: their ratio is the engine clock while the probe ran.
// The MFMA operands are 16 + 16 registers of random values in +-[1, 2),
// drawn once per lane and rotated at compile-time indices, so consecutive
// MFMAs see different operands as a product's do: with constant operands
// the matrix cores draw less power, and with the stores running the part
// then holds a higher clock than a real product gets (2.37 against 2.32 GHz,
// 0.249 against 0.257 ms per 16384 x 16384 x 64 on one MI355X).
constexpr int kFusedThreads = 256;
constexpr int kFusedChains = 16;  // MFMAs per store

template <int MODE>
__global__ void __launch_bounds__(kFusedThreads)
    fused_probe_kernel(int trips, f32x4 *__restrict__ out, unsigned long long *__restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const long long wave = (long long)blockIdx.x * (kFusedThreads / 64) + (threadIdx.x >> 6);
  const long long waves = (long long)gridDim.x * (kFusedThreads / 64);
  float av[kFusedChains], bv[kFusedChains];
  unsigned xs = 0x9E3779B9u ^ (unsigned)(wave * 64 + lane) * 2654435761u;
#pragma unroll
  for (int q = 0; q < kFusedChains; ++q) {  // xorshift32; sign bit and 23 mantissa bits random
    xs ^= xs << 13;
    xs ^= xs >> 17;
    xs ^= xs << 5;
    av[q] = __uint_as_float(0x3F800000u | (xs >> 9) | (xs << 31));
    xs ^= xs << 13;
    xs ^= xs >> 17;
    xs ^= xs << 5;
    bv[q] = __uint_as_float(0x3F800000u | (xs >> 9) | (xs << 31));
  }
  f32x4 acc[kFusedChains];
#pragma unroll
  for (int c = 0; c < kFusedChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  // Rounds in groups of kFusedChains: round j of a group first stores chain
  // j (its last MFMA is 16 MFMAs back, so the store does not wait for it),
  // then issues one MFMA per chain; every chain's result is used
  // (trips % kFusedChains == 0).  The scheduling barriers keep one store
  // per 16 MFMAs instead of letting the compiler gather the stores.
  for (int t0r = 0; t0r < trips; t0r += kFusedChains) {
#pragma unroll
    for (int j = 0; j < kFusedChains; ++j) {
      const long long t = t0r + j;
      if constexpr (MODE == 0) {
        out[(t * waves + wave) * 64 + lane] = acc[j];
      } else if constexpr (MODE == 2) {
        out[(t * waves + wave) * 64 + lane] = f32x4{1.f, 1.f, 1.f, (float)t};
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE != 2) {
#pragma unroll
        for (int c = 0; c < kFusedChains; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[(c + j) % kFusedChains],
                                                        bv[(3 * c + 5 * j) % kFusedChains],
                                                        acc[c], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if constexpr (MODE != 2) {  // keep the last round's matrix work live
    f32x4 s = acc[0];
#pragma unroll
    for (int c = 1; c < kFusedChains; ++c) s += acc[c];
    out[wave * 64 + lane] = s;
  }
  if (clocks != nullptr && lane == 0) {
    clocks[2 * wave] = t1 - t0;
    clocks[2 * wave + 1] = r1 - r0;
  }
}

bool misaligned16(const void *p) {
  return (reinterpret_cast<std::uintptr_t>(p) & 15u) != 0;
}

template <int KIND>
hipError_t launch_stream(long long n, const float *x, const float *y, float *z,
                         hipStream_t s) {
  const long long n4 = n / 4;
  if (n4 > 0) {
    long long blocks = ceil_div(n4, kStreamThreads);
    const long long cap = 256LL * 64;  // 64 workgroups per CU, grid-stride beyond
    if (blocks > cap) blocks = cap;
    hipError_t e = launch_kernel(
        stream_kernel<KIND>, dim3((unsigned)blocks), dim3(kStreamThreads), s, n4,
        reinterpret_cast<const f32x4 *>(x), reinterpret_cast<const f32x4 *>(y),
        reinterpret_cast<f32x4 *>(z));
    if (e != hipSuccess) return e;
  }
  if (n % 4) {
    return launch_kernel(stream_tail<KIND>, dim3(1), dim3(4), s, n4 * 4, n, x,
                         y, z);
  }
  return hipSuccess;
}

}  // namespace

extern "C" int gemm_f32_probe_stream(int kind, long long n, const float *x,
                                     const float *y, float *z, void *stream) {
  if (n < 0 || kind < GEMM_F32_PROBE_COPY || kind > GEMM_F32_PROBE_VADD)
    return GEMM_F32_BAD_ARG;
  if (n == 0) return GEMM_F32_OK;
  if (z == nullptr) return GEMM_F32_NULL_PTR;
  if (kind != GEMM_F32_PROBE_FILL && x == nullptr) return GEMM_F32_NULL_PTR;
  if (kind == GEMM_F32_PROBE_VADD && y == nullptr) return GEMM_F32_NULL_PTR;
  if (misaligned16(z) || (x && misaligned16(x)) || (y && misaligned16(y)))
    return GEMM_F32_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (kind) {
    case GEMM_F32_PROBE_COPY: e = launch_stream<GEMM_F32_PROBE_COPY>(n, x, y, z, s); break;
    case GEMM_F32_PROBE_FILL: e = launch_stream<GEMM_F32_PROBE_FILL>(n, x, y, z, s); break;
    default: e = launch_stream<GEMM_F32_PROBE_VADD>(n, x, y, z, s); break;
  }
  return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_LAUNCH_FAILED;
}

extern "C" long long gemm_f32_probe_mfma_flops(int workgroups, int iters) {
  if (workgroups < 1 || iters < 1) return -1;
  const long long per_mfma = 2LL * 32 * 32 * 2;
  return (long long)workgroups * (kMfmaThreads / 64) * (long long)iters *
         kMfmaChains * per_mfma;
}

extern "C" int gemm_f32_probe_mfma(int workgroups, int iters, float *out,
                                   void *stream) {
  if (workgroups < 1 || iters < 1) return GEMM_F32_BAD_ARG;
  if (out == nullptr) return GEMM_F32_NULL_PTR;
  if (reinterpret_cast<std::uintptr_t>(out) & 3u) return GEMM_F32_MISALIGNED;
  hipError_t e = launch_kernel(mfma_probe_kernel, dim3(workgroups),
                               dim3(kMfmaThreads), static_cast<hipStream_t>(stream),
                               iters, out);
  return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_LAUNCH_FAILED;
}

extern "C" long long gemm_f32_probe_mfma16_flops(int shape, int workgroups, int iters) {
  if ((shape != 16 && shape != 32) || workgroups < 1 || iters < 1) return -1;
  const long long per_wave_round =
      shape == 16 ? kMfma16Chains16 * (2LL * 16 * 16 * 32) : kMfma16Chains32 * (2LL * 32 * 32 * 16);
  return (long long)workgroups * (kMfma16Threads / 64) * (long long)iters * per_wave_round;
}

extern "C" int gemm_f32_probe_mfma16(int shape, int workgroups, int iters, float *out,
                                     void *stream) {
  if ((shape != 16 && shape != 32) || workgroups < 1 || iters < 1) return GEMM_F32_BAD_ARG;
  if (out == nullptr) return GEMM_F32_NULL_PTR;
  if (reinterpret_cast<std::uintptr_t>(out) & 3u) return GEMM_F32_MISALIGNED;
  hipError_t e = shape == 16
                     ? launch_kernel(mfma16_probe_kernel<16>, dim3(workgroups),
                                     dim3(kMfma16Threads), static_cast<hipStream_t>(stream),
                                     iters, out)
                     : launch_kernel(mfma16_probe_kernel<32>, dim3(workgroups),
                                     dim3(kMfma16Threads), static_cast<hipStream_t>(stream),
                                     iters, out);
  return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_LAUNCH_FAILED;
}

extern "C" long long gemm_f32_probe_valu_flops(int workgroups, int iters) {
  if (workgroups < 1 || iters < 1) return -1;
  return (long long)workgroups * kValuThreads * (long long)iters * kValuRounds *
         kValuChains * 2;
}

extern "C" int gemm_f32_probe_valu(int workgroups, int iters, float *out,
                                   void *stream) {
  if (workgroups < 1 || iters < 1) return GEMM_F32_BAD_ARG;
  if (out == nullptr) return GEMM_F32_NULL_PTR;
  if (reinterpret_cast<std::uintptr_t>(out) & 3u) return GEMM_F32_MISALIGNED;
  hipError_t e = launch_kernel(valu_probe_kernel, dim3(workgroups),
                               dim3(kValuThreads), static_cast<hipStream_t>(stream),
                               iters, out);
  return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_LAUNCH_FAILED;
}

extern "C" long long gemm_f32_probe_lds_bytes(int workgroups, int iters) {
  if (workgroups < 1 || iters < 1) return -1;
  return (long long)workgroups * kLdsThreads * (long long)iters * kLdsReadsPerTrip * 16;
}

extern "C" int gemm_f32_probe_lds(int workgroups, int iters, float *out, void *stream) {
  if (workgroups < 1 || iters < 1) return GEMM_F32_BAD_ARG;
  if (out == nullptr) return GEMM_F32_NULL_PTR;
  if (reinterpret_cast<std::uintptr_t>(out) & 3u) return GEMM_F32_MISALIGNED;
  hipError_t e = launch_kernel(lds_probe_kernel, dim3(workgroups), dim3(kLdsThreads),
                               static_cast<hipStream_t>(stream), iters, out);
  return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_LAUNCH_FAILED;
}

extern "C" long long gemm_f32_probe_fused_flops(int mode, int workgroups, int trips) {
  if (mode < GEMM_F32_FUSED_BOTH || mode > GEMM_F32_FUSED_STORE || workgroups < 1 || trips < 1 ||
      trips % kFusedChains != 0)
    return -1;
  if (mode == GEMM_F32_FUSED_STORE) return 0;
  return (long long)workgroups * (kFusedThreads / 64) * (long long)trips * kFusedChains *
         (2LL * 16 * 16 * 4);
}

extern "C" long long gemm_f32_probe_fused_bytes(int mode, int workgroups, int trips) {
  if (mode < GEMM_F32_FUSED_BOTH || mode > GEMM_F32_FUSED_STORE || workgroups < 1 || trips < 1 ||
      trips % kFusedChains != 0)
    return -1;
  const long long per_round = (long long)workgroups * (kFusedThreads / 64) * 1024;
  // MFMA-only mode stores one KB per wave at the end; the fused mode stores
  // that last KB into round 0's run again (after its loop)
  return mode == GEMM_F32_FUSED_MFMA ? per_round : per_round * trips;
}

extern "C" int gemm_f32_probe_fused(int mode, int workgroups, int trips, float *out,
                                    long long out_bytes, unsigned long long *clocks,
                                    void *stream) {
  const long long need = gemm_f32_probe_fused_bytes(mode, workgroups, trips);
  if (need < 0) return GEMM_F32_BAD_ARG;
  if (out == nullptr) return GEMM_F32_NULL_PTR;
  if (misaligned16(out) || (reinterpret_cast<std::uintptr_t>(clocks) & 7u))
    return GEMM_F32_MISALIGNED;
  if (out_bytes < need) return GEMM_F32_BAD_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  f32x4 *o = reinterpret_cast<f32x4 *>(out);
  hipError_t e;
  switch (mode) {
    case GEMM_F32_FUSED_BOTH:
      e = launch_kernel(fused_probe_kernel<0>, dim3(workgroups), dim3(kFusedThreads), s, trips, o,
                        clocks);
      break;
    case GEMM_F32_FUSED_MFMA:
      e = launch_kernel(fused_probe_kernel<1>, dim3(workgroups), dim3(kFusedThreads), s, trips, o,
                        clocks);
      break;
    default:
      e = launch_kernel(fused_probe_kernel<2>, dim3(workgroups), dim3(kFusedThreads), s, trips, o,
                        clocks);
      break;
  }
  return e == hipSuccess ? GEMM_F32_OK : GEMM_F32_LAUNCH_FAILED;
}

extern "C" int gemm_f32_device_props(int device, int *cus, int *clock_khz, int *lds_per_cu,
                                     int *wave_size, int *l2_bytes) {
  struct Q {
    int *out;
    hipDeviceAttribute_t attr;
  };
  const Q qs[] = {{cus, hipDeviceAttributeMultiprocessorCount},
                  {clock_khz, hipDeviceAttributeClockRate},
                  {lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor},
                  {wave_size, hipDeviceAttributeWarpSize},
                  {l2_bytes, hipDeviceAttributeL2CacheSize}};
  for (const Q &q : qs) {
    if (q.out == nullptr) continue;
    if (hipDeviceGetAttribute(q.out, q.attr, device) != hipSuccess) return GEMM_F32_BAD_ARG;
  }
  return GEMM_F32_OK;
}
