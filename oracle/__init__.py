"""CPU oracle for the fp32 matrix multiply -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the GPU library and
never imports it; the product path must never route through it.

Contents
  gemm(A, B)            C = A x B by the plain definition, fp64 accumulation
                        in ascending k, one rounding to fp32 (C library
                        ``liboracle.so``, see gemm_oracle.c for the citation).
  gemm_elems(A, B, i, j) selected elements of the same product.
  gemm_ld(...)          the raw leading-dimension form over flat buffers.
  decode16(bits, fmt)   values of bf16 / fp16 codes ("bf16" | "f16"), fp64.
  gemm_mixed(A, B, fmt) C = A x B over 16-bit codes (uint16 arrays), same
                        fp64 accumulation, fp32 result.
  gemm_mixed_elems(...) selected elements of that product.
  model                 the pages' operation and load counting model.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(brute force against exact integers, identity, all-ones, the 8x8 / T=4 block
decomposition of page 3, integer exactness, an fp64 BLAS witness and the
Higham error bound), ``tests/test_oracle_mixed_pins.py`` (both 16-bit
decoders against numpy's and torch's conversions over all 65536 codes and
the formats' printed constants; the product against exact rational
arithmetic) and ``tests/test_model_pins.py`` (numbers the pages print).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import model  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int64)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_dp = ctypes.POINTER(ctypes.c_double)

FORMATS = {"bf16": 0, "f16": 1}


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build_oracle import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_gemm_f32.argtypes = [_i64, _i64, _i64, _fp, _i64, _fp, _i64, _fp, _i64]
    lib.oracle_gemm_f32.restype = ctypes.c_int
    lib.oracle_gemm_f32_elems.argtypes = [_i64, _i64, _i64, _fp, _i64, _fp, _i64,
                                          _i64, _ip, _ip, _fp]
    lib.oracle_gemm_f32_elems.restype = ctypes.c_int
    lib.oracle_decode16.argtypes = [_i64, _u16p, ctypes.c_int, _dp]
    lib.oracle_decode16.restype = ctypes.c_int
    lib.oracle_gemm_mixed.argtypes = [_i64, _i64, _i64, _u16p, _i64, _u16p, _i64, ctypes.c_int,
                                      _fp, _i64]
    lib.oracle_gemm_mixed.restype = ctypes.c_int
    lib.oracle_gemm_mixed_elems.argtypes = [_i64, _i64, _i64, _u16p, _i64, _u16p, _i64,
                                            ctypes.c_int, _i64, _ip, _ip, _fp]
    lib.oracle_gemm_mixed_elems.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _fptr(x: np.ndarray):
    return x.ctypes.data_as(_fp)


def _as_f32_2d(x: np.ndarray, name: str) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.strides[1] != 4 or (x.shape[0] > 1 and x.strides[0] % 4):
        x = np.ascontiguousarray(x)
    return x


def _ld(x: np.ndarray) -> int:
    return max(1, x.strides[0] // 4) if x.shape[0] > 1 else max(1, x.shape[1])


def gemm_ld(M, N, K, a_buf, lda, b_buf, ldb, c_buf, ldc) -> None:
    """Raw form over flat float32 buffers: C[i*ldc+j] = sum_k A[i*lda+k]*B[k*ldb+j]."""
    for buf in (a_buf, b_buf, c_buf):
        if buf.dtype != np.float32 or not buf.flags.c_contiguous:
            raise TypeError("buffers must be C-contiguous float32")
    if M > 0 and N > 0:
        need_c = (M - 1) * ldc + N
        if c_buf.size < need_c:
            raise ValueError("C buffer too small")
    if M > 0 and K > 0 and a_buf.size < (M - 1) * lda + K:
        raise ValueError("A buffer too small")
    if K > 0 and N > 0 and b_buf.size < (K - 1) * ldb + N:
        raise ValueError("B buffer too small")
    rc = _load().oracle_gemm_f32(M, N, K, _fptr(a_buf), lda, _fptr(b_buf), ldb,
                                 _fptr(c_buf), ldc)
    if rc != 0:
        raise ValueError(f"oracle_gemm_f32 rejected its arguments (rc={rc})")


def gemm(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """C = A x B (float32 in, float32 out) by the plain definition."""
    a = _as_f32_2d(a, "A")
    b = _as_f32_2d(b, "B")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {a.shape} x {b.shape}")
    c = np.empty((M, N), dtype=np.float32)
    if M == 0 or N == 0:
        return c
    a_flat = a.reshape(-1) if a.flags.c_contiguous else np.ascontiguousarray(a).reshape(-1)
    b_flat = b.reshape(-1) if b.flags.c_contiguous else np.ascontiguousarray(b).reshape(-1)
    if a_flat.size == 0:
        a_flat = np.zeros(1, np.float32)
    if b_flat.size == 0:
        b_flat = np.zeros(1, np.float32)
    gemm_ld(M, N, K, a_flat, max(1, K), b_flat, max(1, N), c.reshape(-1), max(1, N))
    return c


def gemm_elems(a: np.ndarray, b: np.ndarray, ii, jj) -> np.ndarray:
    """out[t] = (A x B)[ii[t], jj[t]], each by the plain definition."""
    a = np.ascontiguousarray(_as_f32_2d(a, "A"))
    b = np.ascontiguousarray(_as_f32_2d(b, "B"))
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {a.shape} x {b.shape}")
    ii = np.ascontiguousarray(np.asarray(ii, dtype=np.int64).reshape(-1))
    jj = np.ascontiguousarray(np.asarray(jj, dtype=np.int64).reshape(-1))
    if ii.shape != jj.shape:
        raise ValueError("index arrays differ in length")
    out = np.empty(ii.size, dtype=np.float32)
    if ii.size == 0:
        return out
    a_flat = a.reshape(-1) if a.size else np.zeros(1, np.float32)
    b_flat = b.reshape(-1) if b.size else np.zeros(1, np.float32)
    rc = _load().oracle_gemm_f32_elems(
        M, N, K, _fptr(a_flat), max(1, K), _fptr(b_flat), max(1, N), ii.size,
        ii.ctypes.data_as(_ip), jj.ctypes.data_as(_ip), _fptr(out))
    if rc != 0:
        raise ValueError(f"oracle_gemm_f32_elems rejected its arguments (rc={rc})")
    return out


def _fmt(fmt: str) -> int:
    try:
        return FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown 16-bit format {fmt!r}; one of {sorted(FORMATS)}") from None


def _as_u16_2d(x: np.ndarray, name: str) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint16 array of 16-bit codes")
    return np.ascontiguousarray(x)


def decode16(bits: np.ndarray, fmt: str) -> np.ndarray:
    """fp64 values of bf16 or fp16 codes (any shape of uint16)."""
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    out = np.empty(bits.shape, dtype=np.float64)
    if bits.size:
        rc = _load().oracle_decode16(bits.size, bits.ctypes.data_as(_u16p), _fmt(fmt),
                                     out.ctypes.data_as(_dp))
        if rc != 0:
            raise ValueError(f"oracle_decode16 rejected its arguments (rc={rc})")
    return out


def gemm_mixed(a: np.ndarray, b: np.ndarray, fmt: str) -> np.ndarray:
    """C = A x B over 16-bit codes (uint16, row-major), fp32 result."""
    a = _as_u16_2d(a, "A")
    b = _as_u16_2d(b, "B")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {a.shape} x {b.shape}")
    c = np.empty((M, N), dtype=np.float32)
    if M == 0 or N == 0:
        return c
    a_flat = a.reshape(-1) if a.size else np.zeros(1, np.uint16)
    b_flat = b.reshape(-1) if b.size else np.zeros(1, np.uint16)
    rc = _load().oracle_gemm_mixed(M, N, K, a_flat.ctypes.data_as(_u16p), max(1, K),
                                   b_flat.ctypes.data_as(_u16p), max(1, N), _fmt(fmt),
                                   _fptr(c.reshape(-1)), max(1, N))
    if rc != 0:
        raise ValueError(f"oracle_gemm_mixed rejected its arguments (rc={rc})")
    return c


def gemm_mixed_elems(a: np.ndarray, b: np.ndarray, fmt: str, ii, jj) -> np.ndarray:
    """out[t] = (A x B)[ii[t], jj[t]] over 16-bit codes, each by the definition."""
    a = _as_u16_2d(a, "A")
    b = _as_u16_2d(b, "B")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {a.shape} x {b.shape}")
    ii = np.ascontiguousarray(np.asarray(ii, dtype=np.int64).reshape(-1))
    jj = np.ascontiguousarray(np.asarray(jj, dtype=np.int64).reshape(-1))
    if ii.shape != jj.shape:
        raise ValueError("index arrays differ in length")
    out = np.empty(ii.size, dtype=np.float32)
    if ii.size == 0:
        return out
    a_flat = a.reshape(-1) if a.size else np.zeros(1, np.uint16)
    b_flat = b.reshape(-1) if b.size else np.zeros(1, np.uint16)
    rc = _load().oracle_gemm_mixed_elems(
        M, N, K, a_flat.ctypes.data_as(_u16p), max(1, K), b_flat.ctypes.data_as(_u16p),
        max(1, N), _fmt(fmt), ii.size, ii.ctypes.data_as(_ip), jj.ctypes.data_as(_ip),
        _fptr(out))
    if rc != 0:
        raise ValueError(f"oracle_gemm_mixed_elems rejected its arguments (rc={rc})")
    return out


def num_threads() -> int:
    """Threads the oracle's OpenMP regions use (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_num_threads())
