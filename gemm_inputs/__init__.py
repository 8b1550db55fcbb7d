"""Seeded synthetic inputs for the dense fp32 matrix multiply C = A x B.

This module is shared by the oracle side (tests, the CPU baseline) and the
GPU side (tests, bench, smoke).  It only draws random matrices; it holds no
part of the product's arithmetic, so neither side can borrow the other's.

Workloads.  The pages work on square N x N row-major float matrices (page 1,
"矩阵乘法 tiling", section 一 and the N = 4096 worked size in sections 一
and 三; page 4, "CUDA 编程系列之三", section 6).  The five named workloads
below generalise that to M x K times K x N with the value distributions and
seeds fixed for this project:

  square_256      256^3, uniform[-1, 1], seed 0
  square_1024_int 1024^3, integers uniform in {-4..4} stored as fp32, seed 1
                  (every partial sum is an integer below 2^24, so exact)
  square_4096     4096^3, uniform[-1, 1], seed 2 (the pages' worked size)
  ragged          M=4097, N=4095, K=2049, standard normal, seed 3
  skinny_k64      M=N=16384, K=64, uniform[-1, 1], seed 4
  deep_k          M=N=256, K=16384, uniform[-1, 1], seed 5 -- not one of the
                  benchmark's configurations: a deep-K product with fewer
                  output tiles than compute units, the case K-splitting is for

Generator.  numpy's PCG64 via ``numpy.random.default_rng(seed)``; A is drawn
first and B second from the same generator.  Matrices are returned as
C-contiguous float32 arrays (row-major, leading dimension = column count).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "draw", "make", "make_workload", "sha256",
           "to_code16", "make_mixed", "make_mixed_workload"]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str  # "uniform" | "int4" | "normal"
    seed: int
    description: str

    @property
    def flops(self) -> int:
        # Counting convention only (one multiply and one add per term);
        # used for reporting, never for computing C.
        return 2 * self.M * self.N * self.K


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("square_256", 256, 256, 256, "uniform", 0,
                 "square 256^3, A,B ~ U[-1,1], seed 0"),
        Workload("square_1024_int", 1024, 1024, 1024, "int4", 1,
                 "square 1024^3, A,B integers uniform in {-4..4}, seed 1"),
        Workload("square_4096", 4096, 4096, 4096, "uniform", 2,
                 "square 4096^3, A,B ~ U[-1,1], seed 2"),
        Workload("ragged", 4097, 4095, 2049, "normal", 3,
                 "ragged M=4097 N=4095 K=2049, A,B ~ N(0,1), seed 3"),
        Workload("skinny_k64", 16384, 16384, 64, "uniform", 4,
                 "skinny M=N=16384 K=64, A,B ~ U[-1,1], seed 4"),
        Workload("deep_k", 256, 256, 16384, "uniform", 5,
                 "deep-K M=N=256 K=16384, A,B ~ U[-1,1], seed 5"),
    )
}


def draw(rng: np.random.Generator, shape: tuple[int, int], dist: str) -> np.ndarray:
    """One float32 matrix of ``shape`` from ``rng`` with distribution ``dist``.

    ``dist``: "uniform" -> U[-1, 1); "int4" -> integers uniform in {-4..4};
    "normal" -> N(0, 1); "ones" -> all 1.0; "small_int" -> integers in {-3..3}.
    """
    if dist == "uniform":
        out = rng.uniform(-1.0, 1.0, shape).astype(np.float32)
    elif dist == "int4":
        out = rng.integers(-4, 5, shape).astype(np.float32)
    elif dist == "small_int":
        out = rng.integers(-3, 4, shape).astype(np.float32)
    elif dist == "normal":
        out = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "ones":
        out = np.ones(shape, dtype=np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return np.ascontiguousarray(out)


def make(M: int, N: int, K: int, dist: str, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """A (M x K) then B (K x N), both float32 row-major, from one seeded PCG64."""
    if min(M, N, K) < 0:
        raise ValueError("dimensions must be non-negative")
    rng = np.random.default_rng(seed)
    a = draw(rng, (M, K), dist)
    b = draw(rng, (K, N), dist)
    return a, b


def make_workload(name: str) -> tuple[Workload, np.ndarray, np.ndarray]:
    w = WORKLOADS[name]
    a, b = make(w.M, w.N, w.K, w.dist, w.seed)
    return w, a, b


def to_code16(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round float32 values to 16-bit codes (uint16), nearest-even.

    Input preparation for the 16-bit-input product, the step a caller takes
    before handing matrices over; the product itself only reads the codes.
    "f16": numpy's float32 -> float16 conversion.  "bf16": the upper half of
    the binary32 word after adding half an ulp of the 16-bit result (ties to
    even); inputs here are finite.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if fmt == "f16":
        return x.astype(np.float16).view(np.uint16)
    if fmt == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    raise ValueError(f"unknown 16-bit format {fmt!r}")


def make_mixed(M: int, N: int, K: int, dist: str, seed: int,
               fmt: str) -> tuple[np.ndarray, np.ndarray]:
    """The float32 pair of ``make`` rounded to 16-bit codes of ``fmt``."""
    a, b = make(M, N, K, dist, seed)
    return to_code16(a, fmt), to_code16(b, fmt)


def make_mixed_workload(name: str, fmt: str) -> tuple[Workload, np.ndarray, np.ndarray]:
    w = WORKLOADS[name]
    a, b = make_mixed(w.M, w.N, w.K, w.dist, w.seed, fmt)
    return w, a, b


def sha256(x: np.ndarray) -> str:
    """Hex digest of the raw bytes of a C-contiguous array (reproducibility log)."""
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()
