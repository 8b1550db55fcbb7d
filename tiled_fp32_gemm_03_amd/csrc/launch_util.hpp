// Small launch helper: hipLaunchKernel returns the status of this launch
// itself, so no sticky runtime error of an earlier call is picked up.
#pragma once

#include <hip/hip_runtime.h>

namespace gemm_f32_impl {

template <typename... KArgs>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block,
                         hipStream_t stream, KArgs... args) {
  void *ptrs[] = {static_cast<void *>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block,
                         ptrs, 0, stream);
}

inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// The direct-to-LDS loads address each lane's 16 bytes as a 64-bit base in
// scalar registers plus a 32-bit unsigned byte offset, computed per lane as
// (r * ld + chunk) * elem_bytes for row r of a tile of `rows` rows.  A row's
// chunks lie within its ld elements, so every offset of such a tile is below
// rows * ld * elem_bytes; when that product fits in 32 bits no offset wraps.
// Each launcher of a direct-load kernel checks this for its A tile (BM rows)
// and its B step (BK rows) and otherwise runs a kernel with 64-bit addresses.
inline bool lane_offsets_fit(long long rows, long long ld, long long elem_bytes) {
  return rows > 0 && ld >= 0 && rows * ld * elem_bytes <= (1LL << 32);
}

}  // namespace gemm_f32_impl
