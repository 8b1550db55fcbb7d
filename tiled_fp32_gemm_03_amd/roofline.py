"""Roofline bookkeeping for the benchmark: algorithmic work, the tiled load
model per launch-table entry, and MI355X peak figures.

Algorithmic work of C = A x B (beta = 0): 2*M*N*K FLOP; compulsory bytes
4*(M*K + K*N + M*N) -- A and B read once, C written once and never read.
Intensity is their ratio and the binding roof is the lower of the compute
peak and intensity x bandwidth (mayulu.co "CUDA 编程系列之三", sections 2-3).

Issued global loads of a workgroup-tiled kernel: every tile of C walks all
k steps and loads a BM x BK block of A plus a BK x BN block of B per step;
with ceilings for ragged edges that is (BM*BK + BK*BN) * ceil(K/BK) *
ceil(M/BM) * ceil(N/BN) elements (the T x T case is geek-doc.cn "矩阵乘法
tiling", section 三: 2N^3/T).  The naive kernel issues 2*M*N*K loads
(csh0101.cc "CUDA 深入浅出（二）", naive section).
"""
from __future__ import annotations

# MI355X published peaks (dense, no sparsity).
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_BF16_MFMA_TFLOPS = 2500.0  # also fp16
PEAK_HBM_GBPS = 8000.0
CUS = 256
CLOCK_GHZ = 2.4


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def compulsory_bytes(M: int, N: int, K: int, in_bytes: int = 4) -> int:
    """A and B read once (``in_bytes`` per element), fp32 C written once."""
    return in_bytes * (M * K + K * N) + 4 * M * N


def intensity(M: int, N: int, K: int) -> float:
    b = compulsory_bytes(M, N, K)
    return flops(M, N, K) / b if b else 0.0


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def issued_load_elements(variant: str, M: int, N: int, K: int, tile: dict) -> int:
    """Model element loads for the launch-table entry ``tile`` (from gemm_f32_tile)."""
    if variant == "naive":
        return 2 * M * N * K
    bm, bn, bk = tile["BM"], tile["BN"], tile["BK"]
    return (bm * bk + bk * bn) * _cdiv(K, bk) * _cdiv(M, bm) * _cdiv(N, bn)


def binding_roof_tflops(M: int, N: int, K: int, peak_tflops: float, bw_gbps: float) -> float:
    return min(peak_tflops, intensity(M, N, K) * bw_gbps / 1000.0)


# ---- the floor that eight separate L2s set on a persistent tiled product ----
# The dispatcher deals consecutive workgroups to the 8 XCDs round robin; the
# persistent kernels renumber them so each XCD's workgroups walk a block of
# tiles (8 tile rows at a time, column by column), and each XCD's L2 then
# has to fetch every A row panel and B column panel its tiles touch at least
# once.  This mirrors that mapping (xcd_remap and tile_coords of the kernels)
# to count those panels: a measured L2-to-fabric read volume at this floor
# means no panel is fetched twice into one L2.

def _xcd_remap(b: int, grid: int, xcds: int) -> int:
    per, rem, x = grid // xcds, grid % xcds, b % xcds
    return x * per + min(x, rem) + b // xcds


def _tile_coords(lid: int, tiles_m: int, tiles_n: int, group_rows: int) -> tuple[int, int]:
    per_group = group_rows * tiles_n
    g = lid // per_group
    first = g * group_rows
    rows = min(tiles_m - first, group_rows)
    r = lid - g * per_group
    return first + r % rows, r // rows


def xcd_panel_bytes(M: int, N: int, K: int, BM: int, BN: int, grid: int, in_bytes: int = 4,
                    xcds: int = 8, group_rows: int = 8) -> dict:
    """Bytes each XCD's L2 must fetch (every A row panel and B column panel
    its workgroups' tiles touch, once) plus C written once, for a persistent
    grid of ``grid`` workgroups over BM x BN tiles with full-K panels."""
    tiles_m, tiles_n = _cdiv(M, BM), _cdiv(N, BN)
    ntiles = tiles_m * tiles_n
    rows = [set() for _ in range(xcds)]
    cols = [set() for _ in range(xcds)]
    for b in range(grid):
        t = _xcd_remap(b, grid, xcds)
        while t < ntiles:
            tm, tn = _tile_coords(t, tiles_m, tiles_n, group_rows)
            rows[b % xcds].add(tm)
            cols[b % xcds].add(tn)
            t += grid
    a = sum(len(r) for r in rows) * min(BM, M) * K * in_bytes
    b = sum(len(c) for c in cols) * min(BN, N) * K * in_bytes
    return {"read_bytes": a + b, "write_bytes": 4 * M * N, "bytes": a + b + 4 * M * N,
            "a_panel_fetches": sum(len(r) for r in rows), "b_panel_fetches": sum(len(c) for c in cols)}
