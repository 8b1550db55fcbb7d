// Host-only planning of the gemm_f32 library: argument checks, the
// production kernel's launch table and automatic choice, the thin-strip
// rule, the row cut and the split-K plan.  Plain C++17 with no HIP types, so
// the same source is linked into the library and built on its own with the
// address and undefined-behaviour sanitizers by the host tests.  Nothing
// here touches a GPU.
#pragma once

#include <cstdint>

namespace gemm_f32_impl {

// Status codes of include/gemm_f32.h (repeated so this unit stands alone).
constexpr int kOk = 0, kInvalidDim = 1, kInvalidLd = 2, kNullPtr = 3, kBadVariant = 4,
              kMisaligned = 6, kBadConfig = 7, kBadArg = 8;

constexpr long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// The direct-to-LDS loads address each lane's 16 bytes as a 64-bit base in
// scalar registers plus a 32-bit unsigned byte offset, computed per lane as
// (r * ld + chunk) * elem_bytes for row r of a tile of `rows` rows.  A row's
// chunks lie within its ld elements, so every offset of such a tile is below
// rows * ld * elem_bytes; when that product fits in 32 bits no offset wraps.
// Each launcher of a direct-load kernel checks this for its A tile (BM rows)
// and its B step (BK rows) and otherwise runs a kernel with 64-bit addresses.
constexpr bool lane_offsets_fit(long long rows, long long ld, long long elem_bytes) {
  return rows > 0 && ld >= 0 && rows * ld * elem_bytes <= (1LL << 32);
}

// Largest grid.y the runtime accepts; kernels loop when a dimension exceeds it.
constexpr int kMaxGridY = 65535;

// ---- argument checks ---------------------------------------------------

// M, N and K must be >= 0.
int check_shape(int M, int N, int K);

// Leading dimensions: lda >= max(1, K), ldb >= max(1, N), ldc >= max(1, N).
int check_ld(int N, int K, int lda, int ldb, int ldc);

// Pointers of a product whose shape passed check_shape: for a non-empty C,
// non-null C and (when K > 0) A and B, then alignment of C to 4 bytes and
// of A and B to `in_align` bytes (4 for fp32 operands, 2 for 16-bit codes).
int check_pointers(int M, int N, int K, const void *A, const void *B, const void *C,
                   int in_align);

// check_ld, then check_pointers: the checks every product entry makes, in
// that order, before launching anything.
int check_operands(int M, int N, int K, const void *A, int lda, const void *B, int ldb,
                   const void *C, int ldc, int in_align);

// A caller-provided buffer (the split-K workspace): NULL or not 4-byte
// aligned is refused.
bool bad_buffer(const void *p);

// ---- the production kernel's launch table ------------------------------

// Launch-table entry of the production kernel.
struct ProdConfig {
  int BM, BN, BK;  // workgroup tile and k step
  int WGM, WGN;    // waves along M and N (threads = 64 * WGM * WGN)
  int occupancy;   // intended workgroups per CU (documentation, grid sizing)
  const char *name;
};

// kKloop: any K, k loop over steps of BK.  kPanel: all of K in one LDS
// stage, K <= BK, whole tiles only (remainders become strips).  kKsplit: the
// 16x16-MFMA families, any K.  kStrip: the thin-M strip kernel on the whole
// product, M <= kStripMaxRows.  kStripN: the thin-N kernel on the whole
// product, N <= kStripMaxCols.
enum ProdKind { kKloop, kPanel, kKsplit, kStrip, kStripN };

int prod_num_configs();
const ProdConfig &prod_config(int index);
ProdKind prod_kind(int index);
bool prod_supports(int index, int M, int N, int K);

// The entry that computes thin remainder strips, and the most rows a bottom
// strip may have to go to the thin-M strip kernel.
constexpr int kRemainderConfig = 3;
constexpr int kStripMaxRows = 32;
// The launch-table entry that runs the thin-M strip kernel on a whole
// product of at most kStripMaxRows rows (one launch; it reads B once), and
// the rows one of its workgroups holds for an M-row product (the kernel is
// instantiated for 1, 2, 4, 8, 16 and 32).  Two launches of 32 rows lose to
// the tile entries where those fill the chip (64 x 16384 x 4096: 303 us).
constexpr int kStripConfig = 26;
constexpr int strip_rows(int M) {
  return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : M <= 16 ? 16 : 32;
}
// Quads of k whose loads a strip lane issues before using any (its batch),
// per row count: measured kernel durations on N = 1024-32768, K = 2049-8192
// (1 x 4095 x 2049: 10.7, 11.4, 13.0 us for 1, 2, 4 quads; 8 x 8191 x 4096:
// 36.0 us for 1, 38.8 for 2; 4 x 16384 x 4096: 49.6 for 1, 44.9 for 2).
constexpr int strip_batch_quads(int rows) { return rows == 2 || rows == 4 ? 2 : 1; }
// The launch-table entry that runs the thin-N kernel on a whole product of
// at most kStripMaxCols columns, the columns it is instantiated for, and
// the k of B it stages in LDS at a time for that many columns.
constexpr int kStripMaxCols = 16;
constexpr int kColStripConfig = 27;
constexpr int strip_cols(int N) { return N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : 16; }
constexpr int col_chunk(int cols) { return cols <= 8 ? 1024 : 512; }

// Rows (or columns) of a thin remainder strip worth a separate launch: an
// overhanging tile row that is at most 1/8 full.
int thin_remainder(int extent, int tile);

// The automatic choice's model of the k-loop entries: the best entry, its
// modelled TFLOP/s, and that rate again if its tiles fill every workgroup
// slot (else 0).
struct KloopModel {
  int entry;
  double score, full_rate;
};
KloopModel model_kloop(int M, int N, int K);

// Entry 25's row cut: the number of 256-row tile rows computed by entry 19
// in whole rounds, or 0 when no cut models faster than the best single entry.
int region_rows(int M, int N, int K);

// The plain product's automatic entry; through `full_rate` (if given) its
// modelled TFLOP/s when its tiles fill every workgroup slot, else 0.
int prod_choose(int M, int N, int K, double *full_rate = nullptr);

// Split-K form of the production kernel: K is cut into `splits` chunks of
// kc (a multiple of the entry's BK); each chunk's partial product goes to its
// own M x N slab of a workspace, and a second kernel sums the slabs in chunk
// order into C.
struct SplitPlan {
  int config;                 // launch-table entry
  int splits;                 // chunks actually used (1 = plain product)
  int kc;                     // k values per chunk
  long long workspace_bytes;  // splits * M * N * 4, or 0 when splits == 1
};
bool splitk_plan(int M, int N, int K, int config, int splits, SplitPlan *out);

// ---- measured rates behind the automatic choice -------------------------

// One candidate of the k-loop model: its tile, the TFLOP/s it sustains on
// one MI355X when every compute unit is busy (separately for K a multiple
// of 32, where it loads directly to LDS, and otherwise), and how many of its
// workgroups fit on the chip at once.
struct KloopRate {
  int entry, bm, bn;
  double tflops_whole_steps, tflops_partial_steps;
  int slots;
};
int kloop_rate_count();
const KloopRate &kloop_rate(int i);

}  // namespace gemm_f32_impl
