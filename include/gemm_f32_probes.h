/*
 * gemm_f32_probes.h -- measurement probes shipped with the gemm_f32 library.
 *
 * They supply the denominators of the roofline report (page 4, mayulu.co
 * "CUDA 编程系列之三", sections 1-3: a kernel is bounded by the lower of the
 * compute roof and intensity x bandwidth) and a copy kernel of known size to
 * calibrate memory counters.  They are not part of the product C = A x B.
 *
 * All pointers are device pointers owned by the caller; nothing is allocated.
 * Calls are asynchronous on `stream` (hipStream_t as void*, NULL = null
 * stream).  Status codes are those of gemm_f32.h.
 */
#ifndef GEMM_F32_PROBES_H
#define GEMM_F32_PROBES_H

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming kinds.  Bytes moved per element: copy 8, fill 4, vector add 12.
 * Vector add C[i] = A[i] + B[i] is the pages' memory yardstick: one FLOP per
 * twelve bytes (mayulu.co section 4). */
#define GEMM_F32_PROBE_COPY 0 /* z[i] = x[i]          */
#define GEMM_F32_PROBE_FILL 1 /* z[i] = 1.0f          */
#define GEMM_F32_PROBE_VADD 2 /* z[i] = x[i] + y[i]   */

/*
 * gemm_f32_probe_stream -- one streaming pass over n floats with 128-bit
 * accesses.  x (and y for VADD) are read, z is written; for FILL, x and y
 * may be NULL; for COPY, y may be NULL.  n >= 0.  All pointers must be
 * 16-byte aligned.  Returns GEMM_F32_BAD_ARG for an unknown kind or a
 * negative n, GEMM_F32_NULL_PTR / GEMM_F32_MISALIGNED for bad pointers.
 */
int gemm_f32_probe_stream(int kind, long long n, const float *x,
                          const float *y, float *z, void *stream);

/*
 * gemm_f32_probe_mfma -- fp32 matrix-core throughput probe with no memory
 * traffic in its loop: `workgroups` workgroups of 256 threads, each wave
 * running `iters` rounds of 8 independent v_mfma_f32_32x32x2_f32 chains.
 * One float per wave is written to out (out must hold workgroups * 4
 * floats) so the work stays live.  workgroups >= 1, iters >= 1.
 * gemm_f32_probe_mfma_flops returns the FLOPs such a call performs
 * (-1 for invalid arguments).
 */
int gemm_f32_probe_mfma(int workgroups, int iters, float *out, void *stream);
long long gemm_f32_probe_mfma_flops(int workgroups, int iters);

/*
 * gemm_f32_probe_mfma16 -- bf16 matrix-core throughput probe, the measured
 * compute roof of the 16-bit rung (geek-doc.cn, "矩阵乘法 tiling", §五
 * names 16-bit matrix-core GEMM as the next step; mayulu.co, "CUDA 编程系列之三",
 * §2-§3: a kernel is bounded by the compute roof it can reach).  No memory
 * traffic in its loop: `workgroups` workgroups of 256 threads (one wave per
 * SIMD when workgroups <= the CU count), each wave running `iters` rounds
 * of 32 independent v_mfma_f32_16x16x32_bf16 chains (shape 16) or 8
 * independent v_mfma_f32_32x32x16_bf16 chains (shape 32).  One float per
 * wave is written to out (out must hold workgroups * 4 floats, 4-byte
 * aligned).  shape is 16 or 32, workgroups >= 1, iters >= 1, else
 * GEMM_F32_BAD_ARG.  gemm_f32_probe_mfma16_flops returns the FLOPs such a
 * call performs (-1 for invalid arguments).
 */
int gemm_f32_probe_mfma16(int shape, int workgroups, int iters, float *out, void *stream);
long long gemm_f32_probe_mfma16_flops(int shape, int workgroups, int iters);

/*
 * gemm_f32_probe_valu -- fp32 vector-ALU throughput probe, the compute roof
 * of kernels that multiply-add on the vector ALU rather than on matrix cores:
 * `workgroups` workgroups of 256 threads, each lane running `iters` loop
 * trips of 8 rounds over 16 independent scalar fused multiply-add chains
 * (v_fmac_f32, 128 per trip).  One float
 * per wave is written to out (out must hold workgroups * 4 floats).
 * workgroups >= 1, iters >= 1.  gemm_f32_probe_valu_flops returns the FLOPs
 * such a call performs (2 per FMA per lane; -1 for invalid arguments).
 */
int gemm_f32_probe_valu(int workgroups, int iters, float *out, void *stream);
long long gemm_f32_probe_valu_flops(int workgroups, int iters);

/*
 * gemm_f32_probe_lds -- LDS read-bandwidth probe, the on-chip roof of the
 * tiled kernels (their inner products read operands from LDS):
 * `workgroups` workgroups of 256 threads, each holding 64 KiB of LDS and
 * running `iters` trips of 8 conflict-free 128-bit reads per lane.  One
 * float per wave is written to out (out must hold workgroups * 4 floats).
 * workgroups >= 1, iters >= 1.  gemm_f32_probe_lds_bytes returns the bytes
 * such a call reads from LDS (-1 for invalid arguments).
 */
int gemm_f32_probe_lds(int workgroups, int iters, float *out, void *stream);
long long gemm_f32_probe_lds_bytes(int workgroups, int iters);

/*
 * gemm_f32_probe_fused -- the hardware's rate at the intensity of the skinny
 * K = 64 product, where the output is most of the traffic.  The pages bound
 * a kernel by the lower of its compute roof and intensity x bandwidth
 * (mayulu.co "CUDA 编程系列之三", sections 2-3); this probe measures what the
 * part sustains when both kinds of work run together at one fixed ratio:
 * `workgroups` workgroups of 256 threads (4 waves), each wave running `trips`
 * rounds of 16 independent v_mfma_f32_16x16x4_f32 (32768 FLOP) followed by
 * one 128-bit store per lane (1 KB), i.e. 32 FLOP per stored byte, which is
 * K / 2 for K = 64.  The MFMA operands are random values rotated through
 * registers, so the matrix cores draw the power a product's operands make
 * them draw (the clock under this load depends on it).  With 256 workgroups and 1024 trips it does the FLOPs of
 * a 16384 x 16384 x 64 product and writes its 1 GiB of output.
 *   mode     GEMM_F32_FUSED_BOTH, _MFMA (no stores in the loop) or _STORE
 *            (no MFMAs).
 *   out      device buffer of at least gemm_f32_probe_fused_bytes(mode,
 *            workgroups, trips) bytes, 16-byte aligned; out_bytes its size.
 *            Round t of all waves writes one contiguous run of
 *            workgroups * 4 KB.  After its loop each wave writes one more
 *            KB, the sum of its chains, into round 0's run (all the
 *            MFMA-only mode writes), so no MFMA result goes unused.
 *   clocks   NULL, or 8-byte aligned device memory for 2 * workgroups * 4
 *            values: per wave, shader-clock cycles (s_memtime) and constant
 *            100 MHz real-time ticks (s_memrealtime) over its loop; cycles x
 *            100 MHz / ticks is the engine clock under that load.
 * workgroups >= 1, trips a positive multiple of 16 (round j of each group of
 * 16 stores chain j, so every chain's result is used).  Returns
 * GEMM_F32_BAD_ARG for an unknown mode,
 * bad counts or a short buffer, GEMM_F32_NULL_PTR / GEMM_F32_MISALIGNED for
 * bad pointers.  gemm_f32_probe_fused_flops and _bytes give the FLOPs and the
 * bytes stored by such a call (-1 for invalid arguments).
 */
#define GEMM_F32_FUSED_BOTH 0
#define GEMM_F32_FUSED_MFMA 1
#define GEMM_F32_FUSED_STORE 2
int gemm_f32_probe_fused(int mode, int workgroups, int trips, float *out, long long out_bytes,
                         unsigned long long *clocks, void *stream);
long long gemm_f32_probe_fused_flops(int mode, int workgroups, int trips);
long long gemm_f32_probe_fused_bytes(int mode, int workgroups, int trips);

/*
 * gemm_f32_device_props -- properties of HIP device `device` that the
 * roofline report quotes: compute units, peak engine clock (kHz), LDS bytes
 * per compute unit, wave size and L2 bytes.  Any output pointer may be NULL.
 * Returns GEMM_F32_BAD_ARG if the runtime cannot answer (no such device).
 */
int gemm_f32_device_props(int device, int *cus, int *clock_khz, int *lds_per_cu,
                          int *wave_size, int *l2_bytes);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F32_PROBES_H */
