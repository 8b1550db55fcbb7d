"""The pages' counting model for the matrix multiply -- TEST INFRASTRUCTURE ONLY.

Operation counts, global-load counts, arithmetic intensity and the roofline,
written from the pages' own derivations so that tests can check the GPU
package's reporting against them.  Independent of the GPU package.

Counting conventions (all quantities are model counts, not measurements):

* One loop-body step of the product does one multiply and one add: 2 FLOP;
  the whole product is 2*M*N*K FLOP (page 1, "矩阵乘法 tiling", section 一:
  2N^3 for N x N; page 1 section 一 also: about 137 GFLOP at N = 4096).
* The naive kernel loads one A element and one B element from global memory
  per step: 2 loads per output per k, 2*M*N*K loads in total; the C write-back
  is left out (page 2, "CUDA 深入浅出（二）", section "naive kernel 怎么读数据":
  2N per output element times N^2 outputs = 2N^3).
* The T x T tiled kernel loads a T x T block of A and a T x T block of B per
  tile step, 2*T^2 elements, where the naive kernel would have issued 2*T^3
  (page 2, section "对一个 C_tile 数数"); over (N/T)^2 tiles of N/T steps each
  that is 2N^3/T (page 1 section 三, first display equation; page 2 section
  "推广到整个 N×N 矩阵").  The pages assume T divides N (page 2, same
  section).  Reading taken here for other shapes: a tile that overhangs an
  edge still counts its whole blocks (the zero-filled slots are issued loads
  too), so the count uses ceilings.  A rectangular BM x BN tile with a BK-deep
  k step generalises the same count to (BM*BK + BK*BN) per step.
* Arithmetic intensity is FLOP per byte of global traffic (page 4, "CUDA 编程
  系列之三", section 2); with 4-byte floats the naive kernel has
  2 FLOP / 8 B = 0.25 FLOP/B (page 1 section 一) and the tiled kernel T/4
  FLOP/B (page 1 section 三, second display equation).
* The ridge point is peak FLOP/s over peak B/s; attainable throughput is the
  lower of the compute roof and intensity x bandwidth (page 4, sections 2 and
  3).  Vector add does 1 FLOP per 12 bytes (page 4 section 4).
"""
from __future__ import annotations

import math

FLOAT_BYTES = 4


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def flops(M: int, N: int, K: int) -> int:
    """Floating-point operations of C = A x B: two per (i, j, k) term."""
    return 2 * M * N * K


def naive_loads(M: int, N: int, K: int) -> int:
    """Global element loads of the one-thread-per-output kernel (C write excluded)."""
    per_output = 2 * K          # one A and one B element per k
    outputs = M * N
    return outputs * per_output


def tile_step_loads(T: int) -> tuple[int, int]:
    """(tiled, naive) global element loads of one T x T tile over one T-deep step."""
    tiled = T * T + T * T       # one A block and one B block
    naive = (T * T) * (2 * T)   # T^2 outputs, 2T loads each
    return tiled, naive


def tiled_loads(M: int, N: int, K: int, T: int) -> int:
    """Global element loads of the T x T tiled kernel (ceil over ragged edges)."""
    return blocked_loads(M, N, K, T, T, T)


def blocked_loads(M: int, N: int, K: int, BM: int, BN: int, BK: int) -> int:
    """Element loads when one workgroup owns a BM x BN tile and steps BK along k."""
    if min(BM, BN, BK) <= 0:
        raise ValueError("tile sizes must be positive")
    tiles = _ceil_div(M, BM) * _ceil_div(N, BN)
    steps = _ceil_div(K, BK)
    per_step = BM * BK + BK * BN
    return tiles * steps * per_step


def reuse_factor(T: int) -> int:
    """How many outputs use each element brought on chip: T (not T^2)."""
    tiled, naive = tile_step_loads(T)
    return naive // tiled


def intensity_naive() -> float:
    """FLOP per byte of the naive kernel: 2 FLOP per 2 float loads."""
    return 2.0 / (2 * FLOAT_BYTES)


def intensity_tiled(T: int) -> float:
    """FLOP per byte of the T x T tiled kernel on a divisible square problem."""
    n = T * 8  # any multiple of T gives the same ratio
    return flops(n, n, n) / (tiled_loads(n, n, n, T) * FLOAT_BYTES)


def intensity_vector_add() -> float:
    """C[i] = A[i] + B[i]: one add against two 4-byte reads and one 4-byte write."""
    return 1.0 / (3 * FLOAT_BYTES)


def input_bytes_square(N: int) -> int:
    """Bytes of the two N x N float inputs."""
    return 2 * N * N * FLOAT_BYTES


def ridge(peak_flops: float, peak_bytes_per_s: float) -> float:
    """Arithmetic intensity where the bandwidth slope meets the compute roof."""
    return peak_flops / peak_bytes_per_s


def attainable(intensity: float, peak_flops: float, peak_bytes_per_s: float) -> float:
    """Roofline: the lower of the compute roof and intensity x bandwidth."""
    return min(peak_flops, intensity * peak_bytes_per_s)


def higham_gamma(n: int, unit_roundoff: float = 2.0 ** -24) -> float:
    """gamma_n = n u / (1 - n u), the classical bound factor for an n-term dot
    product in floating point with unit roundoff u (Higham, Accuracy and
    Stability of Numerical Algorithms, 2nd ed., section 3.1)."""
    nu = n * unit_roundoff
    if nu >= 1.0:
        return math.inf
    return nu / (1.0 - nu)


def textbook_owner(T: int, block_xy: tuple[int, int], thread_xy: tuple[int, int]) -> tuple[int, int]:
    """(row, col) of the C element owned by a thread of the T x T tiled kernel:
    x indices pick the column, y indices the row (page 3, step ②; page 1
    section 四: one block per C tile, one thread per element)."""
    bx, by = block_xy
    tx, ty = thread_xy
    return by * T + ty, bx * T + tx
