"""Helpers shared by the GPU parity tests (not a test module).

tol_check is the floating-point bar of the parity tests, derived from fp32
accumulation: max |C - C_ref| <= 1e-4 * sqrt(K) and
||C - C_ref||_F / ||C_ref||_F <= 1e-5, computed in fp64 on the host.
sample_indices picks the elements a full-size product is checked on: random
ones plus whole first and last rows and columns (every edge tile).
"""
import numpy as np


def tol_check(got: np.ndarray, ref: np.ndarray, K: int, what: str):
    got64 = got.astype(np.float64)
    ref64 = ref.astype(np.float64)
    assert np.all(np.isfinite(got64)), f"{what}: non-finite output"
    err = np.abs(got64 - ref64)
    max_err = float(err.max()) if err.size else 0.0
    denom = float(np.sqrt((ref64 ** 2).sum()))
    fro = float(np.sqrt((err ** 2).sum())) / denom if denom > 0 else float(np.sqrt((err ** 2).sum()))
    assert max_err <= 1e-4 * np.sqrt(max(K, 1)), f"{what}: max err {max_err:.3g} (K={K})"
    assert fro <= 1e-5, f"{what}: relative Frobenius error {fro:.3g}"


def sample_indices(M, N, n, seed):
    rng = np.random.default_rng(seed)
    ii = [rng.integers(0, M, n)]
    jj = [rng.integers(0, N, n)]
    # whole first/last row and column (every edge tile), and the corners
    for r in (0, M - 1):
        cols = np.arange(N)
        ii.append(np.full(N, r))
        jj.append(cols)
    for c in (0, N - 1):
        rows = np.arange(M)
        ii.append(rows)
        jj.append(np.full(M, c))
    return np.concatenate(ii).astype(np.int64), np.concatenate(jj).astype(np.int64)
