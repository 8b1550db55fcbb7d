"""Leading dimensions past the reach of 32-bit lane offsets.

The direct-to-LDS kernels address their operands as a scalar base plus a
32-bit byte offset per lane, so each launcher takes them only while every
offset of a tile's rows stays below 2^32 (lane_offsets_fit over the tile's A
rows and one k step of B rows); otherwise it runs a kernel with 64-bit
addresses.  These products put rows of A, B or C 4 to 9 GB apart (MI355X
holds 288 GB): at the largest leading dimension the guard admits (direct
loads whose offsets reach past 2^31, so an offset taken as signed would
fail) and just beyond it (the 64-bit kernels), and compare every entry of
the launch tables with the oracle.  Only the used part of each operand is written; the
oracle sees the dense matrices.  A wrong guard would read wrapped rows inside
the same buffer (wrong values, no fault), which the comparison catches.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gemm_inputs import make, make_mixed  # noqa: E402
from parity_util import tol_check  # noqa: E402

# fp32: 256-row A tiles fit while 256 ld 4 <= 2^32; 32-row B steps while 32 ld 4 <= 2^32.
LD_A_EDGE, LD_A = 4_194_304, 4_210_752
LD_B_EDGE, LD_B = 33_554_432, 34_636_834
LD_C = 4_210_752
# 16-bit codes: 256-row A tiles fit while 256 ld 2 <= 2^32.
LD_A16_EDGE, LD_A16 = 8_388_608, 8_421_504


@pytest.fixture(scope="module")
def g():
    import tiled_fp32_gemm_03_amd as lib
    return lib


def _strided(rows, cols, ld, dtype, dev):
    buf = torch.zeros(((rows - 1) * ld + cols,), dtype=dtype, device=dev)
    return buf, buf.as_strided((rows, cols), (ld, 1))


def _entries(g, M, N, K):
    out = [("naive", -1), ("tiled", -1), ("tiled32", -1), ("valu", -1)]
    for cfg in range(g.gemm_f32_num_configs("prod")):
        try:
            g.gemm_f32_tile("prod", cfg, M, N, K)
        except g.GemmError:
            continue
        out.append(("prod", cfg))
    return out + [("prod", -1)]


_LDS = {"A_edge": (LD_A_EDGE, 0, 0), "A": (LD_A, 0, 0), "B_edge": (0, LD_B_EDGE, 0),
        "B": (0, LD_B, 0), "C": (0, 0, LD_C)}


@pytest.mark.parametrize("which", list(_LDS))
@pytest.mark.parametrize("shape", [(256, 256, 64), (300, 260, 65), (5, 300, 65), (300, 5, 65)])
def test_f32_leading_dimension_beyond_32bit_offsets(g, which, shape):
    """Every entry that takes the shape; the thin ones (5 rows: the thin-M
    strip; 5 columns: the thin-N kernel) address with 64-bit offsets
    throughout."""
    M, N, K = shape
    dev = torch.device("cuda:0")
    a, b = make(M, N, K, "normal", seed=M + N + K)
    ref = oracle.gemm(a, b)
    la, lb, lc = _LDS[which]
    lda, ldb, ldc = la or K, lb or N, lc or N
    print(f"case: {which} ld {max(lda, ldb, ldc)} shape {M}x{N}x{K}", flush=True)
    abuf, av = _strided(M, K, lda, torch.float32, dev)
    bbuf, bv = _strided(K, N, ldb, torch.float32, dev)
    cbuf, cv = _strided(M, N, ldc, torch.float32, dev)
    av.copy_(torch.from_numpy(a))
    bv.copy_(torch.from_numpy(b))
    s = torch.cuda.current_stream().cuda_stream
    for variant, cfg in _entries(g, M, N, K):
        cv.fill_(float("nan"))
        g.gemm_f32_ex(M, N, K, abuf.data_ptr(), lda, bbuf.data_ptr(), ldb, cbuf.data_ptr(), ldc,
                      variant, cfg, s)
        torch.cuda.synchronize()
        tol_check(cv.cpu().numpy(), ref, K, f"{variant}#{cfg} {which} ld {shape}")
    del abuf, bbuf, cbuf
    torch.cuda.empty_cache()


def test_splitk_leading_dimension_beyond_32bit_offsets(g):
    M, N, K = 256, 256, 4096
    dev = torch.device("cuda:0")
    a, b = make(M, N, K, "normal", seed=11)
    ref = oracle.gemm(a, b)
    print(f"case: split-K, A ld {LD_A} shape {M}x{N}x{K}", flush=True)
    abuf, av = _strided(M, K, LD_A, torch.float32, dev)
    av.copy_(torch.from_numpy(a))
    tb = torch.from_numpy(b).to(dev)
    c = g.matmul_splitk(av, tb, splits=8)
    torch.cuda.synchronize()
    tol_check(c.cpu().numpy(), ref, K, "split-K, A ld beyond 32-bit offsets")
    del abuf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("lda", [LD_A16_EDGE, LD_A16])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_mixed_leading_dimension_beyond_32bit_offsets(g, fmt, lda):
    M, N, K = 256, 256, 128
    dev = torch.device("cuda:0")
    a16, b16 = make_mixed(M, N, K, "small_int", seed=5, fmt=fmt)
    ref = oracle.gemm_mixed(a16, b16, fmt)
    print(f"case: {fmt}, A ld {lda} shape {M}x{N}x{K}", flush=True)
    abuf, av = _strided(M, K, lda, torch.int16, dev)
    av.copy_(torch.from_numpy(a16.view(np.int16)))
    tb = torch.from_numpy(b16.view(np.int16)).to(dev)
    c = torch.empty((M, N), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    for cfg in list(range(g.gemm_mixed_num_configs())) + [-1]:
        try:
            g.gemm_mixed_tile(cfg, M, N, K)
        except g.GemmError:
            continue
        c.fill_(float("nan"))
        g.gemm_mixed(M, N, K, abuf.data_ptr(), lda, tb.data_ptr(), N, c.data_ptr(), N, fmt, cfg, s)
        torch.cuda.synchronize()
        assert np.array_equal(c.cpu().numpy(), ref), f"{fmt}#{cfg}"
    del abuf
    torch.cuda.empty_cache()
