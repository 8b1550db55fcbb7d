// Small launch helper: hipLaunchKernel returns the status of this launch
// itself, so no sticky runtime error of an earlier call is picked up.
#pragma once

#include <hip/hip_runtime.h>

#include "host_plan.hpp"  // ceil_div, lane_offsets_fit

namespace gemm_f32_impl {

template <typename... KArgs>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block,
                         hipStream_t stream, KArgs... args) {
  void *ptrs[] = {static_cast<void *>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block,
                         ptrs, 0, stream);
}

}  // namespace gemm_f32_impl
