// Workgroup-to-tile order shared by the matrix-core kernels (gfx950).
//
// The dispatcher deals consecutive workgroups of a launch to the 8 XCDs
// round robin, and each XCD has its own L2.  xcd_remap renumbers launch
// indices so every XCD works on a contiguous run of logical ids, and
// tile_coords walks those ids in groups of kGroupRows tile rows, column by
// column, so the workgroups resident on one XCD share rows of A and columns
// of B in its L2.
#pragma once

#include <hip/hip_runtime.h>

namespace gemm_f32_impl {

constexpr int kXcds = 8;
constexpr int kGroupRows = 8;

// Launch index b of G -> logical id: each XCD gets a contiguous run of ids.
__device__ inline int xcd_remap(int b, int G) {
  const int per = G / kXcds, rem = G % kXcds, x = b % kXcds;
  return x * per + (x < rem ? x : rem) + b / kXcds;
}

// Logical id -> (tile row, tile column), in groups of kGroupRows tile rows
// walked column by column.
__device__ inline void tile_coords(int lid, int tiles_m, int tiles_n, int &tm,
                                   int &tn) {
  const int per_group = kGroupRows * tiles_n;
  const int g = lid / per_group;
  const int first = g * kGroupRows;
  const int rows = tiles_m - first < kGroupRows ? tiles_m - first : kGroupRows;
  const int r = lid - g * per_group;
  tm = first + r % rows;
  tn = r / rows;
}

}  // namespace gemm_f32_impl
