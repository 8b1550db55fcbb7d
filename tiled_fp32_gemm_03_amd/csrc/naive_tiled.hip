// Rungs 1 and 2 of the kernel ladder (gfx950), plus the K = 0 fill.
//
// Rung 1, naive: one thread owns one element of C and reads its operands
// straight from global memory every step, accumulating in an fp32 register
// (geek-doc.cn "矩阵乘法 tiling", section 一; csh0101.cc "CUDA 深入浅出（二）",
// section "naive kernel 怎么读数据").  A wave of 64 lanes takes 64 consecutive
// columns of one row: the B reads of a wave are contiguous and the A read is
// one address broadcast to the wave.
//
// Rung 2, textbook tiling: one T x T workgroup owns one T x T tile of C; per
// k step every thread copies one A element and one B element into LDS, a
// barrier makes the tiles visible, each thread does T multiply-adds out of
// LDS, and a second barrier keeps the next step from overwriting tiles still
// being read (geek-doc.cn section 四 and its pitfall list in section 六;
// csh0101.cc section "代码里的样子"; ijyty.com steps ①-⑧; mayulu.co
// "CUDA 编程系列之三", section 6).  x indices pick the column and y indices the
// row (ijyty.com step ②).  Elements outside A or B are loaded as 0 rather
// than skipped (geek-doc.cn section 六; mayulu.co section 7), and threads
// whose output lies outside C still take part in loads and barriers.
#include "gemm_internal.hpp"
#include "launch_util.hpp"

namespace gemm_f32_impl {
namespace {

__global__ void __launch_bounds__(256) zero_kernel(Problem p) {
  const long long total = (long long)p.M * p.N;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
       e < total; e += stride) {
    const long long i = e / p.N, j = e - i * p.N;
    p.C[i * p.ldc + j] = 0.0f;
  }
}

constexpr int kNaiveX = 64, kNaiveY = 4;

__global__ void __launch_bounds__(kNaiveX *kNaiveY)
    naive_kernel(Problem p, int row_blocks) {
  const long long col = (long long)blockIdx.x * kNaiveX + threadIdx.x;
  for (long long rb = blockIdx.y; rb < row_blocks; rb += gridDim.y) {
    const long long row = rb * kNaiveY + threadIdx.y;
    if (row >= p.M || col >= p.N) continue;
    const float *a = p.A + row * p.lda;
    const float *b = p.B + col;
    float acc = 0.0f;
    for (int k = 0; k < p.K; ++k) acc += a[k] * b[(long long)k * p.ldb];
    p.C[row * p.ldc + col] = acc;
  }
}

// PAD floats after each LDS row: the padded form the pages point to for
// shared-memory bank conflicts (geek-doc.cn section 五).  With this access
// pattern (As[ty][k] is one address per row of threads, Bs[k][tx] walks
// consecutive words) the unpadded tiles are already conflict-free on CDNA4's
// LDS; the padded rung exists to measure that claim.
template <int T, int PAD = 0>
__global__ void __launch_bounds__(T *T) tiled_kernel(Problem p, int tiles_m) {
  __shared__ float As[T][T + PAD];
  __shared__ float Bs[T][T + PAD];
  const int tx = threadIdx.x, ty = threadIdx.y;
  const long long col = (long long)blockIdx.x * T + tx;
  const int phases = (p.K + T - 1) / T;
  for (long long by = blockIdx.y; by < tiles_m; by += gridDim.y) {
    const long long row = by * T + ty;
    float acc = 0.0f;
    for (int ph = 0; ph < phases; ++ph) {
      const int ka = ph * T + tx;  // k of the A element this thread copies
      const int kb = ph * T + ty;  // k of the B element this thread copies
      As[ty][tx] = (row < p.M && ka < p.K) ? p.A[row * p.lda + ka] : 0.0f;
      Bs[ty][tx] = (kb < p.K && col < p.N) ? p.B[(long long)kb * p.ldb + col] : 0.0f;
      __syncthreads();  // tiles complete before anyone reads them
#pragma unroll
      for (int k = 0; k < T; ++k) acc += As[ty][k] * Bs[k][tx];
      __syncthreads();  // everyone done reading before the next overwrite
    }
    if (row < p.M && col < p.N) p.C[row * p.ldc + col] = acc;
  }
}

int clamp_grid_y(long long blocks) {
  return (int)(blocks < kMaxGridY ? blocks : kMaxGridY);
}

}  // namespace

hipError_t launch_zero(const Problem &p, hipStream_t s) {
  const long long total = (long long)p.M * p.N;
  long long blocks = ceil_div(total, 256);
  if (blocks > 65536) blocks = 65536;
  return launch_kernel(zero_kernel, dim3((unsigned)blocks), dim3(256), s, p);
}

hipError_t launch_zero_f32(float *C, int M, int N, long long ldc, hipStream_t s) {
  const Problem p{M, N, 0, nullptr, 1, nullptr, 1, C, ldc};
  return launch_zero(p, s);
}

hipError_t launch_naive(const Problem &p, hipStream_t s) {
  const long long gx = ceil_div(p.N, kNaiveX);
  const long long rows = ceil_div(p.M, kNaiveY);
  return launch_kernel(naive_kernel, dim3((unsigned)gx, clamp_grid_y(rows)),
                       dim3(kNaiveX, kNaiveY), s, p, (int)rows);
}

hipError_t launch_tiled(int T, bool padded, const Problem &p, hipStream_t s) {
  const long long gx = ceil_div(p.N, T);
  const long long tiles_m = ceil_div(p.M, T);
  const dim3 grid((unsigned)gx, clamp_grid_y(tiles_m));
  if (padded) {
    if (T != 32) return hipErrorInvalidValue;
    return launch_kernel(tiled_kernel<32, 1>, grid, dim3(32, 32), s, p, (int)tiles_m);
  }
  switch (T) {
    case 4: return launch_kernel(tiled_kernel<4>, grid, dim3(4, 4), s, p, (int)tiles_m);
    case 16: return launch_kernel(tiled_kernel<16>, grid, dim3(16, 16), s, p, (int)tiles_m);
    case 32: return launch_kernel(tiled_kernel<32>, grid, dim3(32, 32), s, p, (int)tiles_m);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gemm_f32_impl
