"""Helpers shared by the GPU parity tests (not a test module).

tol_check is the floating-point bar of the parity tests, derived from fp32
accumulation: max |C - C_ref| <= 1e-4 * sqrt(K) and
||C - C_ref||_F / ||C_ref||_F <= 1e-5, computed in fp64 on the host.
full_tol_check applies the same bar to a whole matrix, a band of rows at a
time so that a 1 GiB product needs no 2 GiB fp64 temporaries, and
full_exact_check compares whole matrices bit for bit.
sample_indices picks the elements a full-size product is checked on where
the oracle has to compute them one by one: random ones plus whole first and
last rows and columns (every edge tile).
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


def _band_errors(got, ref, r0, r1):
    g = got[r0:r1].astype(np.float64)
    r = ref[r0:r1].astype(np.float64)
    d = np.abs(g - r)
    k = int(d.argmax()) if d.size else 0
    return (float(d.flat[k]) if d.size else 0.0, r0 + k // got.shape[1], k % got.shape[1],
            float(np.dot(d.ravel(), d.ravel())), float(np.dot(r.ravel(), r.ravel())),
            bool(np.isfinite(g).all()))


def full_errors(got: np.ndarray, ref: np.ndarray, band_elems: int = 1 << 22) -> dict:
    """Max |got - ref|, where it sits, and the relative Frobenius error over
    every element of two equally shaped 2-D float32 matrices, in fp64.  Bands
    of rows run on a few host threads (numpy releases the GIL); the sums are
    added in band order, so the result does not depend on the thread count."""
    from concurrent.futures import ThreadPoolExecutor
    assert got.shape == ref.shape and got.ndim == 2, (got.shape, ref.shape)
    M, N = got.shape
    rows = max(1, band_elems // max(N, 1))
    bands = [(r0, min(M, r0 + rows)) for r0 in range(0, M, rows)]
    with ThreadPoolExecutor(max_workers=min(8, max(1, len(bands)))) as ex:
        parts = list(ex.map(lambda b: _band_errors(got, ref, *b), bands))
    max_err, where, err2, ref2, finite = 0.0, (0, 0), 0.0, 0.0, True
    for (m, i, j, e2, r2, fin) in parts:
        if m > max_err:
            max_err, where = m, (i, j)
        err2 += e2
        ref2 += r2
        finite = finite and fin
    fro = np.sqrt(err2) / np.sqrt(ref2) if ref2 > 0 else np.sqrt(err2)
    return {"max_err": max_err, "where": where, "rel_fro": float(fro), "finite": finite}


def full_tol_check(got: np.ndarray, ref: np.ndarray, K: int, what: str) -> dict:
    """tol_check over every element of C (not a sample)."""
    e = full_errors(got, ref)
    assert e["finite"], f"{what}: non-finite output"
    assert e["max_err"] <= 1e-4 * np.sqrt(max(K, 1)), \
        f"{what}: max err {e['max_err']:.3g} at {e['where']} (K={K})"
    assert e["rel_fro"] <= 1e-5, f"{what}: relative Frobenius error {e['rel_fro']:.3g}"
    return e


def full_exact_check(got: np.ndarray, ref: np.ndarray, what: str):
    """Bit-exact equality of every element (-0 and +0 counted equal)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    bad = np.flatnonzero(got.ravel() != ref.ravel())
    assert bad.size == 0, (f"{what}: {bad.size} elements differ, first at "
                           f"{divmod(int(bad[0]), got.shape[1])}")


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
