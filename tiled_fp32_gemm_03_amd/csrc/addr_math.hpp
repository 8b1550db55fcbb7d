// The index arithmetic that decides which memory each lane of the
// matrix-core kernels touches: the workgroup-to-tile order, edge tiles moved
// back inside C, the per-lane offsets of the direct-to-LDS loads, the LDS
// chunk layouts they fill, and the windows of guarded and partial k-step
// loads.  Every function is constexpr (so callable from device code as well
// as from host code) and free of HIP types: the kernels and the host replay
// that checks every address of the benchmark's workloads against its
// matrix run the very same functions.
#pragma once

namespace gemm_f32_impl {

// ---- workgroup -> tile ---------------------------------------------------

// The dispatcher deals consecutive workgroups of a launch to the 8 XCDs
// round robin, and each XCD has its own L2.  xcd_remap renumbers launch
// indices so every XCD works on a contiguous run of logical ids, and
// tile_coords walks those ids in groups of kGroupRows tile rows, column by
// column, so the workgroups resident on one XCD share rows of A and columns
// of B in its L2.
constexpr int kXcds = 8;
constexpr int kGroupRows = 8;

// Launch index b of G -> logical id: each XCD gets a contiguous run of ids.
constexpr int xcd_remap(int b, int G) {
  const int per = G / kXcds, rem = G % kXcds, x = b % kXcds;
  return x * per + (x < rem ? x : rem) + b / kXcds;
}

// Logical id -> (tile row, tile column), in groups of kGroupRows tile rows
// walked column by column.
constexpr void tile_coords(int lid, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int per_group = kGroupRows * tiles_n;
  const int g = lid / per_group;
  const int first = g * kGroupRows;
  const int rows = tiles_m - first < kGroupRows ? tiles_m - first : kGroupRows;
  const int r = lid - g * per_group;
  tm = first + r % rows;
  tn = r / rows;
}

// Tile t's origin for BM x BN tiles over an M x N product.  A last tile row
// or column that would overhang C is moved back to end at C's edge (when C
// is at least one tile wide): it then overlaps its neighbour, and both
// compute the shared elements in the same k order, so they store identical
// values -- while the tile needs no guarded loads.
constexpr void edge_tile_origin(int t, int tiles_m, int tiles_n, int BM, int BN, int M, int N,
                                int &m0, int &n0) {
  int tm = 0, tn = 0;
  tile_coords(t, tiles_m, tiles_n, tm, tn);
  m0 = tm * BM;
  n0 = tn * BN;
  if (m0 + BM > M && M >= BM) m0 = M - BM;
  if (n0 + BN > N && N >= BN) n0 = N - BN;
}

// ---- LDS layouts of the 16x16-MFMA kernels (16-byte chunks) --------------

// A rows of ACH chunks (ACH = BK / 4): chunk c of row r sits at position
// c ^ perm(r), so that 16 consecutive rows land on distinct banks (rows of
// 128 B pair up in a 256-byte bank window; rows of 256 B fill it).
template <int ACH>
constexpr int w16_a_perm(int r) {
  return ACH == 16 ? (r & 15) : ((r >> 1) & 7);
}
template <int ACH>
constexpr int w16_a_pos(int r, int c) {
  return r * ACH + (c ^ w16_a_perm<ACH>(r));
}
// B k rows of BCH chunks (BCH = BN / 4): chunk c of k row k sits at
// c ^ (4 ((k >> 2) & 3)), so the four lane groups of a fragment read, which
// take k rows 4 apart, fall on distinct banks.
template <int BCH>
constexpr int w16_b_pos(int k, int c) {
  return k * BCH + (c ^ (4 * ((k >> 2) & 3)));
}

// ---- direct-to-LDS loads ---------------------------------------------------

// One 16-byte direct load per lane fills 1 KB of LDS in lane order, so lane
// l of instruction `blk` fills chunk position 64 blk + l of its tile's
// layout; it loads the global chunk that belongs there.  Offsets are in
// elements from the k step's base (the tile's first row, first k column).
// A: position 64 blk + l is row (64 / ACH) blk + l / ACH, position l % ACH.
template <int ACH>
constexpr long long dma_a_elem(int blk, int lane, long long lda) {
  const int r = (64 / ACH) * blk + lane / ACH;
  const int c = (lane % ACH) ^ w16_a_perm<ACH>(r);
  return (long long)r * lda + 4 * c;
}
// B: position j = 64 blk + l is k row j / BCH, position j % BCH.
template <int BCH>
constexpr long long dma_b_elem(int j, long long ldb) {
  const int k = j / BCH;
  const int c = (j % BCH) ^ (4 * ((k >> 2) & 3));
  return (long long)k * ldb + 4 * c;
}

// K-split 64x64 kernel: wave w reads only k in [16 w, 16 w + 16) of each
// 64-deep step, so it loads that quarter of the tile's 64 A rows itself,
// into an LDS region no other wave reads (its B k rows, 16 w .. 16 w + 15
// of dma_b_elem<16>'s layout, are likewise its own).  The A quarter holds
// 64 rows of 4 chunks, chunk c of row r at position 4 r + (c ^ ks_a_swz(r)):
// a fragment read takes one chunk of 16 consecutive rows, and the swizzle
// puts any 8 (or 16) consecutive rows' chunks on distinct 16-byte bank
// groups of a 128-byte (or 256-byte) bank window.
constexpr int ks_a_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
constexpr int ks_a_pos(int r, int c) { return 4 * r + (c ^ ks_a_swz(r)); }
// Direct load q (0..3) of wave w: lane l fills position 64 q + l, which is
// row 16 q + l / 4.  Element offset from the k step's base (the tile's
// first row, the step's first k column).
constexpr long long ks_dma_a_elem(int q, int lane, int wave, long long lda) {
  const int r = 16 * q + lane / 4;
  const int c = (lane & 3) ^ ks_a_swz(r);
  return (long long)r * lda + 16 * wave + 4 * c;
}
// How many of the 4 elements of a chunk starting at column kc lie inside K.
constexpr int chunk_valid(int kc, int K) { return kc + 4 <= K ? 4 : (kc < K ? K - kc : 0); }

// ---- guarded and partial windows -------------------------------------------

// Branch-free guarded chunk load of the register-staged kernels: the chunk
// of 4 elements at (row, col) of a rows x cols matrix with leading
// dimension ld.  A chunk wholly inside its row is loaded in place; one that
// straddles the row end loads the 4-element window ending at the row end
// (so no byte past the row is touched) and records the shift; a chunk
// outside the matrix loads from the matrix origin and is marked empty.
// Returns the element offset of the window; meta = (valid << 2) | shift.
// Needs cols >= 4.
constexpr long long guarded_window(int row, int rows, int col, int cols, long long ld,
                                   int &meta) {
  int valid = 0, shift = 0;
  long long off = 0;
  if (row < rows && col < cols) {
    if (col + 4 <= cols) {
      valid = 4;
      off = (long long)row * ld + col;
    } else {
      valid = cols - col;
      shift = col - (cols - 4);
      off = (long long)row * ld + (cols - 4);
    }
  }
  meta = (valid << 2) | shift;
  return off;
}

// A k chunk starting at column kc of a row of K elements in a partial k
// step: the first column of the 4-element window it is read from (the
// chunk itself when it lies inside K, else the last window of the row),
// how many of its elements lie inside K, and where they sit in the window.
// Needs K >= 4.
constexpr int tail_window(int kc, int K, int &valid, int &shift) {
  valid = kc + 4 <= K ? 4 : (kc < K ? K - kc : 0);
  const int col = valid == 4 ? kc : K - 4;
  shift = valid > 0 && valid < 4 ? kc - col : 0;
  return col;
}

}  // namespace gemm_f32_impl
