// LDS layouts and direct-load positions of the 16-bit-input kernels with
// direct-to-LDS loads (mixed16.hip), as constexpr functions shared by the
// kernels and the host replay (tests/host_replay.cpp), apart from
// addr_math.hpp so that the fp32 kernels' sources are unchanged by them.
#pragma once

namespace gemm_f32_impl {

// A stage: 256 rows of 64 bf16/fp16 codes (8 chunks of 16 bytes), chunk c
// of row r at position 8 r + (c ^ ((r >> 1) & 7)).  A fragment read takes
// one chunk of 16 consecutive rows; the 128-byte rows put even and odd
// rows in different halves of a 256-byte bank window and the swizzle
// separates the pairs, so the 16 reads land on distinct 16-byte bank groups.
constexpr int m16_a_pos(int r, int c) { return 8 * r + (c ^ ((r >> 1) & 7)); }
// B stage: 64 k rows of 256 codes (16 slots of 32 bytes).  Slot s of k row
// k sits at slot position m16_b_slot (the 16x16x32 kernel) or m32_b_slot
// (the 32x32x16 kernel).  A transposing read takes 8 bytes per lane: a
// 16-lane group reads one slot in 4 consecutive k rows, and a 32-lane half
// two groups.  The 16x16x32 kernel's halves read one slot in k rows kb ..
// kb + 3 and kb + 8 .. kb + 11; the 32x32x16 kernel's read two adjacent
// slots (2j, 2j + 1) in k rows kb .. kb + 3 (kb a multiple of 4).  Both
// permutations put each 16-lane group's four pieces on distinct 32-byte
// positions of a 128-byte window and each half's eight on distinct
// positions of a 256-byte window (rows are 512 bytes, whole windows,
// apart).  For the 32x32x16 kernel that needs f(k mod 4) = 0, 2, 5, 7:
// distinct modulo 4 and in distinct pairs {2i, 2i + 1}.
constexpr int m16_b_slot(int k, int s) { return s ^ ((k & 3) | (((k >> 3) & 1) << 2)); }
constexpr int m32_b_slot(int k, int s) { return s ^ ((2 * (k & 3)) ^ ((k >> 1) & 1)); }
// Direct loads: lane position j of a stage (16-byte chunks in layout order)
// is filled from this element offset of the step's origin.  Both slot
// permutations are XORs, so they are their own inverses.
constexpr long long m16_dma_a_elem(int j, long long lda) {
  const int r = j / 8;
  const int c = (j % 8) ^ ((r >> 1) & 7);
  return (long long)r * lda + 8 * c;
}
template <bool M32>
constexpr long long m16_dma_b_elem(int j, long long ldb) {
  const int k = j / 32, pos = j % 32;
  const int slot = M32 ? m32_b_slot(k, pos >> 1) : m16_b_slot(k, pos >> 1);
  return (long long)k * ldb + 8 * (2 * slot + (pos & 1));
}

}  // namespace gemm_f32_impl
