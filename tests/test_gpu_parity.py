"""GPU parity: every rung of the kernel ladder against the CPU oracle, element
by element on the same seeded inputs, through the C ABI.

Bars (from the arithmetic):
  * integer-valued inputs whose partial sums stay below 2^24: bit-exact;
  * other inputs: max |C - C_ref| <= 1e-4 * sqrt(K) and
    ||C - C_ref||_F / ||C_ref||_F <= 1e-5 (fp64 on the host).
Full-size workloads are checked on sampled elements (the oracle computes them
one by one) plus properties that hold at any size.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gemm_inputs import WORKLOADS, make, make_workload  # noqa: E402
from parity_util import sample_indices as _sample_indices  # noqa: E402
from parity_util import tol_check as _tol_check  # noqa: E402

LADDER = ("naive", "tiled", "tiled32", "tiled32_pad", "valu", "prod")


@pytest.fixture(scope="module")
def g():
    import tiled_fp32_gemm_03_amd as lib
    return lib


def _dev():
    return torch.device("cuda:0")


def _run(g, a, b, variant, config=-1):
    ta = torch.from_numpy(a).to(_dev())
    tb = torch.from_numpy(b).to(_dev())
    c = g.matmul(ta, tb, variant=variant, config=config)
    torch.cuda.synchronize()
    return c.cpu().numpy()


def _prod_configs(g):
    return list(range(g.gemm_f32_num_configs("prod")))


# ---- small and ragged shapes, every rung ---------------------------------

SMALL_SHAPES = [(1, 1, 1), (3, 5, 7), (33, 65, 17), (64, 64, 64), (127, 129, 131),
                (257, 383, 129), (300, 200, 700), (130, 520, 33)]


@pytest.mark.parametrize("variant", LADDER)
@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_small_integer_bit_exact(g, variant, shape):
    M, N, K = shape
    print(f"case: int {variant} {shape}", flush=True)
    a, b = make(M, N, K, "small_int", seed=M * 7 + N * 3 + K)
    assert np.array_equal(_run(g, a, b, variant), oracle.gemm(a, b))


@pytest.mark.parametrize("variant", LADDER)
@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_small_uniform_tolerance(g, variant, shape):
    M, N, K = shape
    print(f"case: uniform {variant} {shape}", flush=True)
    a, b = make(M, N, K, "uniform", seed=M + N + K)
    _tol_check(_run(g, a, b, variant), oracle.gemm(a, b), K, f"{variant} {shape}")


def _supported(g, cfg, M, N, K):
    try:
        g.gemm_f32_tile("prod", cfg, M, N, K)
        return True
    except g.GemmError:
        return False


def test_valu_entries_agree_bitwise_on_ragged_floats(g):
    """Each element is one FMA chain in ascending k in every entry and tile
    position, edge tiles moved inside C included: identical bits."""
    for (M, N, K) in [(1000, 1003, 515), (700, 300, 129)]:
        a, b = make(M, N, K, "normal", seed=M * N)
        ref = _run(g, a, b, "valu", 0)
        for cfg in range(1, g.gemm_f32_num_configs("valu")):
            print(f"case: valu bitwise agreement config {cfg} {M}x{N}x{K}", flush=True)
            assert np.array_equal(_run(g, a, b, "valu", cfg), ref), (cfg, M, N, K)


def test_every_valu_config(g):
    """Every register-budget entry of the VALU rung: the k loop rolled and
    unrolled, K below, at and past one 8-deep step, ragged tiles."""
    for cfg in range(g.gemm_f32_num_configs("valu")):
        for (M, N, K) in [(257, 383, 129), (128, 128, 8), (1, 300, 7), (200, 1, 33),
                          (300, 260, 17), (129, 131, 1)]:
            print(f"case: valu config {cfg} {M}x{N}x{K}", flush=True)
            a, b = make(M, N, K, "small_int", seed=cfg + M + K)
            assert np.array_equal(_run(g, a, b, "valu", cfg), oracle.gemm(a, b)), (cfg, M, N, K)
            a, b = make(M, N, K, "normal", seed=cfg + N + K)
            _tol_check(_run(g, a, b, "valu", cfg), oracle.gemm(a, b), K, f"valu cfg {cfg}")


def test_every_prod_config(g):
    for cfg in _prod_configs(g):
        for (M, N, K) in [(257, 383, 129), (512, 256, 64), (1, 300, 40), (200, 1, 33),
                          (300, 260, 17)]:
            if not _supported(g, cfg, M, N, K):
                continue
            print(f"case: prod config {cfg} {M}x{N}x{K}", flush=True)
            a, b = make(M, N, K, "small_int", seed=cfg + M)
            assert np.array_equal(_run(g, a, b, "prod", cfg), oracle.gemm(a, b)), (cfg, M, N, K)
            a, b = make(M, N, K, "normal", seed=cfg + N)
            _tol_check(_run(g, a, b, "prod", cfg), oracle.gemm(a, b), K, f"prod cfg {cfg}")


def _small_k_configs(g):
    return [c for c in _prod_configs(g) if g.gemm_f32_tile("prod", c, 1, 1, 1)["BK"] == 64
            and not _supported(g, c, 1, 1, 65)]


def test_small_k_panel_configs(g):
    """The small-K entries: whole-tile shapes (several tiles per workgroup on
    the persistent grid), K below and at the limit, and ragged shapes whose
    remainders go to the strip launches."""
    cfgs = _small_k_configs(g)
    assert cfgs, "expected small-K launch-table entries"
    shapes = [(2048, 2048, 64), (1024, 4096, 64), (512, 512, 63), (1024, 1024, 17),
              (768, 640, 3), (256, 256, 1), (300, 520, 64), (129, 4100, 40), (5000, 129, 64),
              (100, 100, 64)]
    for cfg in cfgs:
        for (M, N, K) in shapes:
            print(f"case: small-K config {cfg} {M}x{N}x{K}", flush=True)
            a, b = make(M, N, K, "small_int", seed=cfg * 31 + M + K)
            assert np.array_equal(_run(g, a, b, "prod", cfg), oracle.gemm(a, b)), (cfg, M, N, K)
            a, b = make(M, N, K, "uniform", seed=cfg * 17 + N + K)
            _tol_check(_run(g, a, b, "prod", cfg), oracle.gemm(a, b), K, f"small-K cfg {cfg}")


def test_kloop_entries_agree_bitwise_on_ragged_floats(g):
    """Every k-loop entry sums each element in the same k order, whatever
    the tile size, the tile's position or whether its edge tile was moved
    back inside C (overlapping a neighbour) -- so on float inputs they must
    agree bit for bit.  The shapes leave no thin remainder for any tile size
    (a thin strip goes to the strip kernel, which sums K in another order)."""
    kloop = [c for c in _prod_configs(g)
             if _supported(g, c, 1, 1, 65) and c not in OWN_ORDER_ENTRIES + STRIP_ENTRIES]
    for (M, N, K) in [(1000, 1003, 515), (3000, 300, 129), (700, 4000, 64)]:
        for cfg in kloop:
            t = g.gemm_f32_tile("prod", cfg, M, N, K)
            assert M % t["BM"] * 8 > t["BM"] and N % t["BN"] * 8 > t["BN"], (cfg, M, N)
        a, b = make(M, N, K, "normal", seed=M + N)
        ref = _run(g, a, b, "prod", kloop[0])
        for cfg in kloop[1:]:
            print(f"case: bitwise agreement config {cfg} {M}x{N}x{K}", flush=True)
            assert np.array_equal(_run(g, a, b, "prod", cfg), ref), (cfg, M, N, K)


KSPLIT_ENTRY = 16  # 64x64x64, K split over the waves (its own summation order)
# 16x16 MFMAs: one wave per SIMD on 64x64 (17, 23), 128x128 (19) and 96x96
# (22) wave tiles; 256x256 direct-to-LDS on 16 waves (18); 128x128 wave
# tiles staged through registers (20)
W16_ENTRIES = (17, 18, 19, 20, 22, 23, 24)
# rows in whole rounds of entry 19's tiles plus a remainder on its own entry,
# or the whole product on the model's entry: the order of whichever runs
ROW_REGION_ENTRY = 25
OWN_ORDER_ENTRIES = (KSPLIT_ENTRY,) + W16_ENTRIES + (ROW_REGION_ENTRY,)
# the thin-M and thin-N kernels on whole products of at most 8 rows or
# columns (k-slices summed at the end, their own order;
# test_strip_entry_whole_product, test_colstrip_entry_whole_product)
STRIP_ENTRY = 26
COLSTRIP_ENTRY = 27
STRIP_ENTRIES = (STRIP_ENTRY, COLSTRIP_ENTRY)
LDS_DMA_ENTRY = 15  # 256x256x32 with direct-to-LDS loads
REG_STAGED_ENTRY = 12  # the same tiles through registers


def test_lds_dma_entry_matches_register_staged(g):
    """The direct-to-LDS entry takes its direct path only when A and B rows
    are 16-byte aligned and N % 4 == 0, and the register path for the K tail
    and for tiles of products narrower than one tile.  It sums every element
    in the same k order as the register-staged kernel with the same tiles,
    so on float inputs the two agree bit for bit: K tails, tiles moved
    inside C, products narrower than a tile, K below one step, workgroups
    that walk two tiles, padded leading dimensions, and unaligned rows (the
    fallback)."""
    assert g.gemm_f32_tile("prod", LDS_DMA_ENTRY, 1, 1, 1) == {
        **g.gemm_f32_tile("prod", REG_STAGED_ENTRY, 1, 1, 1), "config": LDS_DMA_ENTRY}
    dev = _dev()
    cases = [  # (M, N, K, pad_a, pad_b)
        (1024, 1024, 1000, 0, 0), (1300, 1028, 512, 0, 0), (200, 512, 300, 0, 0),
        (512, 200, 96, 0, 0), (4352, 4352, 256, 0, 0), (1024, 1024, 4, 0, 0),
        (600, 1024, 2048, 0, 0), (777, 1028, 515, 4, 8), (1024, 1024, 1024, 1, 0),
        (1024, 1020, 640, 0, 3)]
    for (M, N, K, pa, pb) in cases:
        print(f"case: lds-dma vs register-staged {M}x{N}x{K} pad {pa},{pb}", flush=True)
        a, b = make(M, N, K, "normal", seed=M + 3 * N + 7 * K)
        abuf = torch.zeros((M, K + pa), device=dev)
        bbuf = torch.zeros((K, N + pb), device=dev)
        abuf[:, :K] = torch.from_numpy(a).to(dev)
        bbuf[:, :N] = torch.from_numpy(b).to(dev)
        outs = []
        for cfg in (REG_STAGED_ENTRY, LDS_DMA_ENTRY):
            c = g.matmul(abuf[:, :K], bbuf[:, :N], variant="prod", config=cfg)
            torch.cuda.synchronize()
            outs.append(c.cpu().numpy())
        assert np.array_equal(outs[0], outs[1]), (M, N, K, pa, pb)
        ii, jj = _sample_indices(M, N, 4000, seed=M + K)
        _tol_check(outs[1][ii, jj], oracle.gemm_elems(a, b, ii, jj), K, f"lds-dma {M}x{N}x{K}")


BIG16_DIRECT_ENTRY = 19  # 128x128-wave tiles with direct loads (tail form for K % 32 != 0)
BIG16_STAGED_ENTRY = 20  # the same tiles, LDS layout and k order, staged through registers


def test_direct_tail_form_matches_register_staged(g):
    """The direct-load 128x128-wave kernel takes rows that are only 4-byte
    aligned and K that is not a multiple of its 32-deep step (the partial
    last step filled through registers, zero past K).  It sums every element
    in the register-staged kernel's k order, so the two agree bit for bit on
    float inputs: tails of 1..31, odd leading dimensions, operands one float
    into their buffers, two tiles per workgroup, K between one and two
    steps, and the ragged workload's own shape."""
    dev = _dev()
    cases = [  # (M, N, K, pad_a, pad_b, shift)
        (4097, 4095, 2049, 0, 0, 0), (512, 512, 33, 0, 0, 0), (520, 300, 63, 1, 3, 1),
        (256, 256, 47, 0, 0, 1), (1000, 1028, 1000, 0, 0, 0), (4352, 4096, 40, 0, 0, 0),
        (777, 516, 95, 4, 8, 0), (300, 260, 2049, 1, 1, 1), (4352, 4096, 65, 0, 0, 0),
        (4352, 4096, 34, 1, 1, 1)]
    # Every tail length: r = 1 and 2 run one and two MFMA groups of the
    # partial step, 3..16 four, 17..31 the whole step.
    cases += [(256, 256, 64 + r, r % 3, (r * 5) % 7, r % 2) for r in range(1, 32)]
    for (M, N, K, pa, pb, sh) in cases:
        print(f"case: direct tail vs staged {M}x{N}x{K} pad {pa},{pb} shift {sh}", flush=True)
        a, b = make(M, N, K, "normal", seed=M + 7 * N + 13 * K)
        abuf = torch.zeros((M * (K + pa) + sh,), device=dev)
        bbuf = torch.zeros((K * (N + pb) + sh,), device=dev)
        av = abuf[sh:].view(M, K + pa)
        bv = bbuf[sh:].view(K, N + pb)
        av[:, :K] = torch.from_numpy(a).to(dev)
        bv[:, :N] = torch.from_numpy(b).to(dev)
        outs = []
        for cfg in (BIG16_STAGED_ENTRY, BIG16_DIRECT_ENTRY):
            c = g.matmul(av[:, :K], bv[:, :N], variant="prod", config=cfg)
            torch.cuda.synchronize()
            outs.append(c.cpu().numpy())
        assert np.array_equal(outs[0], outs[1]), (M, N, K, pa, pb, sh)
        ii, jj = _sample_indices(M, N, 4000, seed=M + K)
        _tol_check(outs[1][ii, jj], oracle.gemm_elems(a, b, ii, jj), K, f"direct tail {M}x{N}x{K}")


@pytest.mark.parametrize("entry", OWN_ORDER_ENTRIES)
def test_own_order_entries(g, entry):
    """Entries that sum each element in their own order: the 64x64 K-split
    entry (each wave sums its quarter of every 64-deep k step; the four
    partial tiles are added in wave order) and the one-wave-per-SIMD 16x16
    MFMA entries.  They are held to the fp32 bar (exact on integers), not to
    bit agreement with the other entries.  Shapes: one tile per CU, K tails
    (register path), K below one step, tiles moved inside C, several tiles
    per workgroup (also with one k step each, and unevenly dealt), an odd
    number of k steps, a single tile, padded leading dimensions, unaligned
    rows and products narrower than a tile (the register-staged fallbacks)."""
    dev = _dev()
    cases = [  # (M, N, K, pad_a, pad_b, pad_c)
        (1024, 1024, 1024, 0, 0, 0), (1000, 1028, 1000, 0, 0, 0), (100, 68, 4, 0, 0, 0),
        (130, 1000, 2048, 0, 0, 0), (2048, 2048, 512, 0, 0, 0), (64, 64, 64, 0, 0, 0),
        (777, 516, 700, 4, 8, 5), (300, 300, 257, 1, 0, 0), (512, 260, 96, 0, 3, 0),
        (2304, 1280, 320, 0, 0, 0), (260, 132, 100, 0, 0, 0), (4352, 4100, 32, 0, 0, 0),
        (600, 520, 96, 4, 8, 5), (2048, 1024, 64, 0, 0, 0), (1088, 1024, 128, 0, 4, 0),
        # register-staged 128x128-wave path: K below one step, a tail of 1
        # after one full step, the 4-element minimum, rows not 16-byte
        # aligned, and workgroups that walk two tiles with a K tail
        (256, 256, 31, 0, 0, 0), (512, 300, 33, 1, 0, 0), (300, 260, 4, 0, 1, 0),
        (4352, 4096, 40, 0, 0, 0)]
    for (M, N, K, pa, pb, pc) in cases:
        for dist in ("small_int", "normal"):
            print(f"case: entry {entry} {M}x{N}x{K} pad {pa},{pb},{pc} {dist}", flush=True)
            a, b = make(M, N, K, dist, seed=M + 5 * N + 11 * K)
            abuf = torch.zeros((M, K + pa), device=dev)
            bbuf = torch.zeros((K, N + pb), device=dev)
            cbuf = torch.full((M, N + pc), -3.0, device=dev)
            abuf[:, :K] = torch.from_numpy(a).to(dev)
            bbuf[:, :N] = torch.from_numpy(b).to(dev)
            g.matmul(abuf[:, :K], bbuf[:, :N], out=cbuf[:, :N], variant="prod", config=entry)
            torch.cuda.synchronize()
            c = cbuf.cpu().numpy()
            assert np.all(c[:, N:] == -3.0)
            got, ref = c[:, :N], oracle.gemm(a, b)
            if dist == "small_int":
                assert np.array_equal(got, ref), (M, N, K, pa, pb, pc)
            else:
                _tol_check(got, ref, K, f"entry {entry} {M}x{N}x{K}")
                again = g.matmul(abuf[:, :K], bbuf[:, :N], variant="prod", config=entry)
                torch.cuda.synchronize()
                assert np.array_equal(again.cpu().numpy(), got), "not deterministic"


def test_lds_dma_entry_integer_exact(g):
    for (M, N, K) in [(1024, 1024, 1000), (520, 516, 260), (256, 256, 32)]:
        print(f"case: lds-dma integer {M}x{N}x{K}", flush=True)
        a, b = make(M, N, K, "small_int", seed=M * 5 + K)
        assert np.array_equal(_run(g, a, b, "prod", LDS_DMA_ENTRY), oracle.gemm(a, b)), (M, N, K)


def test_small_k_many_tiles_per_workgroup(g):
    """Tall products where every small-K workgroup walks several output tiles
    (both parities of the tile count, K at and below the limit), checked on
    sampled elements plus whole edge rows and columns."""
    for cfg in _small_k_configs(g):
        for (M, N, K) in [(16384, 2560, 64), (16384, 1536, 40), (8192, 3968, 64)]:
            print(f"case: small-K many tiles config {cfg} {M}x{N}x{K}", flush=True)
            a, b = make(M, N, K, "small_int", seed=cfg + M + N + K)
            dev = _dev()
            c = g.matmul(torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev), variant="prod",
                         config=cfg)
            torch.cuda.synchronize()
            ii, jj = _sample_indices(M, N, 20000, seed=cfg + K)
            got = c[torch.from_numpy(ii).to(dev), torch.from_numpy(jj).to(dev)].cpu().numpy()
            assert np.array_equal(got, oracle.gemm_elems(a, b, ii, jj)), (cfg, M, N, K)


def test_small_k_padded_leading_dimensions(g):
    dev = _dev()
    M, N, K = 1024, 768, 64
    lda, ldb, ldc = 68, 772, 777  # ldc odd: dword-aligned rows of C
    a, b = make(M, N, K, "small_int", seed=3)
    for cfg in _small_k_configs(g):
        abuf = torch.zeros((M, lda), device=dev)
        bbuf = torch.zeros((K, ldb), device=dev)
        cbuf = torch.full((M, ldc), -1.0, device=dev)
        abuf[:, :K] = torch.from_numpy(a).to(dev)
        bbuf[:, :N] = torch.from_numpy(b).to(dev)
        g.matmul(abuf[:, :K], bbuf[:, :N], out=cbuf[:, :N], variant="prod", config=cfg)
        torch.cuda.synchronize()
        c = cbuf.cpu().numpy()
        assert np.array_equal(c[:, :N], oracle.gemm(a, b))
        assert np.all(c[:, N:] == -1.0)


def test_thin_remainder_strips(g):
    """Main block plus thin remainder strips: a bottom strip of up to BM/8
    rows (at most 32) goes to the thin-M strip kernel in one launch; a
    right strip of up to BN/8 columns to small tiles."""
    for cfg in (0, 2, 7):
        t = g.gemm_f32_tile("prod", cfg, 1, 1, 1)
        bm, bn = t["BM"], t["BN"]
        for r in sorted({1, 2, 5, 8, 9, 16, 17, bm // 8}):
            for (N, K) in [(200, 130), (2 * bn + max(1, bn // 8), 33)]:
                M = 2 * bm + r
                print(f"case: strips cfg {cfg} {M}x{N}x{K}", flush=True)
                a, b = make(M, N, K, "small_int", seed=cfg * 101 + r + N)
                assert np.array_equal(_run(g, a, b, "prod", cfg), oracle.gemm(a, b)), (cfg, M, N, K)
                a, b = make(M, N, K, "normal", seed=cfg * 103 + r + K)
                _tol_check(_run(g, a, b, "prod", cfg), oracle.gemm(a, b), K, f"strips cfg {cfg}")


def test_strip_kernel_long_k(g):
    """The thin-M strip kernel with K spanning many of its 128 k-slices,
    column counts that leave a partial last group of 16, odd ldb (rows of B
    only 4-byte aligned) and a single column."""
    for cfg in (0, 12):
        bm = g.gemm_f32_tile("prod", cfg, 1, 1, 1)["BM"]
        for (r, N, K) in [(1, 1001, 2049), (8, 4095, 1500), (3, 16, 5000), (5, 17, 300),
                          (2, 1, 700), (7, 33, 129)]:
            M = bm + r
            print(f"case: strip long-k cfg {cfg} {M}x{N}x{K}", flush=True)
            a, b = make(M, N, K, "small_int", seed=cfg + r * N + K)
            assert np.array_equal(_run(g, a, b, "prod", cfg), oracle.gemm(a, b)), (cfg, M, N, K)
            a, b = make(M, N, K, "normal", seed=cfg + r + N * K)
            _tol_check(_run(g, a, b, "prod", cfg), oracle.gemm(a, b), K, f"strip long-k cfg {cfg}")


def test_strip_entry_whole_product(g):
    """Products of 1-32 rows: the automatic choice runs the thin-M strip kernel
    on the whole product.  Column counts below, at and past a group of 16
    (partial last group), K from 1 to several batches of its k-slices, and
    padded leading dimensions (odd ldb and ldc: rows only 4-byte aligned)
    with the padding left untouched."""
    dev = _dev()
    strip = g.gemm_f32_tile("prod", -1, 1, 4095, 2049)["config"]
    assert strip == STRIP_ENTRY
    for M in list(range(1, 10)) + [12, 16, 17, 24, 31, 32]:
        for (N, K) in [(1, 1), (15, 3), (16, 129), (17, 2049), (300, 40), (4095, 513)]:
            assert g.gemm_f32_tile("prod", -1, M, N, K)["config"] == strip
            print(f"case: strip entry {M}x{N}x{K}", flush=True)
            a, b = make(M, N, K, "small_int", seed=M * 1009 + N + K)
            assert np.array_equal(_run(g, a, b, "prod"), oracle.gemm(a, b)), (M, N, K)
            a, b = make(M, N, K, "normal", seed=M * 1013 + N * K)
            _tol_check(_run(g, a, b, "prod"), oracle.gemm(a, b), K, f"strip entry {M}x{N}x{K}")
    for (M, N, K, lda, ldb, ldc) in [(3, 300, 129, 133, 301, 303), (8, 4095, 2049, 2050, 4097, 4099),
                                     (1, 17, 5, 5, 21, 17), (13, 1000, 1025, 1027, 1001, 1003),
                                     (29, 333, 77, 79, 335, 337), (32, 129, 2049, 2051, 131, 133)]:
        assert g.gemm_f32_tile("prod", -1, M, N, K)["config"] == STRIP_ENTRY
        print(f"case: strip entry padded {M}x{N}x{K} lds {lda},{ldb},{ldc}", flush=True)
        a, b = make(M, N, K, "small_int", seed=lda + ldb)
        abuf = torch.full((M, lda), 7.0, device=dev)
        bbuf = torch.full((K, ldb), 7.0, device=dev)
        cbuf = torch.full((M, ldc), -1.0, device=dev)
        abuf[:, :K] = torch.from_numpy(a).to(dev)
        bbuf[:, :N] = torch.from_numpy(b).to(dev)
        g.matmul(abuf[:, :K], bbuf[:, :N], out=cbuf[:, :N], variant="prod")
        torch.cuda.synchronize()
        c = cbuf.cpu().numpy()
        assert np.array_equal(c[:, :N], oracle.gemm(a, b)), (M, N, K)
        assert np.all(c[:, N:] == -1.0)


def test_colstrip_entry_whole_product(g):
    """Products of more than 32 rows and 1-16 columns: the automatic choice
    runs the thin-N kernel on the whole product.  Row counts past a
    workgroup's 16 (partial last group), K from 1 to past one chunk of B
    (1024 k, or 512 for 9-16 columns: the guarded last chunk with partial
    quads and quads wholly past K), and padded leading dimensions (rows only
    4-byte aligned) with the padding left untouched."""
    dev = _dev()
    assert g.gemm_f32_tile("prod", -1, 4095, 1, 2049)["config"] == COLSTRIP_ENTRY
    for N in list(range(1, 10)) + [12, 16]:
        for (M, K) in [(33, 1), (47, 3), (49, 129), (300, 1024), (1000, 1025), (4097, 2051)]:
            assert g.gemm_f32_tile("prod", -1, M, N, K)["config"] == COLSTRIP_ENTRY
            print(f"case: colstrip entry {M}x{N}x{K}", flush=True)
            a, b = make(M, N, K, "small_int", seed=N * 1019 + M + K)
            assert np.array_equal(_run(g, a, b, "prod"), oracle.gemm(a, b)), (M, N, K)
            a, b = make(M, N, K, "normal", seed=N * 1021 + M * K)
            _tol_check(_run(g, a, b, "prod"), oracle.gemm(a, b), K, f"colstrip entry {M}x{N}x{K}")
    for (M, N, K, lda, ldb, ldc) in [(300, 3, 129, 133, 5, 7), (4097, 8, 2049, 2050, 9, 11),
                                     (70, 1, 5, 9, 1, 2), (1000, 13, 513, 515, 17, 14)]:
        assert g.gemm_f32_tile("prod", -1, M, N, K)["config"] == COLSTRIP_ENTRY
        print(f"case: colstrip entry padded {M}x{N}x{K} lds {lda},{ldb},{ldc}", flush=True)
        a, b = make(M, N, K, "small_int", seed=lda + ldb + ldc)
        abuf = torch.full((M, lda), 7.0, device=dev)
        bbuf = torch.full((K, ldb), 7.0, device=dev)
        cbuf = torch.full((M, ldc), -1.0, device=dev)
        abuf[:, :K] = torch.from_numpy(a).to(dev)
        bbuf[:, :N] = torch.from_numpy(b).to(dev)
        g.matmul(abuf[:, :K], bbuf[:, :N], out=cbuf[:, :N], variant="prod")
        torch.cuda.synchronize()
        c = cbuf.cpu().numpy()
        assert np.array_equal(c[:, :N], oracle.gemm(a, b)), (M, N, K)
        assert np.all(c[:, N:] == -1.0)


def test_guarded_windows_short_rows(g):
    """Rows of exactly 4 and of 1-3 elements (the per-element fallback), and
    K tails of 1-3 past a multiple of 4 (the shifted-window loads)."""
    for (M, N, K) in [(300, 4, 4), (300, 3, 5), (257, 260, 3), (129, 130, 1), (300, 261, 66),
                      (515, 133, 2049), (260, 4095, 7)]:
        for cfg in (0, 2, 3):
            print(f"case: windows cfg {cfg} {M}x{N}x{K}", flush=True)
            a, b = make(M, N, K, "small_int", seed=M + N + K + cfg)
            assert np.array_equal(_run(g, a, b, "prod", cfg), oracle.gemm(a, b)), (cfg, M, N, K)


def test_edge_sweep(g):
    """Every remainder against every tile size: sampled combinations of
    M, N, K around multiples of 16, 32, 64 and 128."""
    sizes = [1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
    rng = np.random.default_rng(2024)
    combos = {(s, s, s) for s in sizes}
    while len(combos) < 60:
        combos.add(tuple(int(x) for x in rng.choice(sizes, 3)))
    for (M, N, K) in sorted(combos):
        a, b = make(M, N, K, "small_int", seed=M * 1000003 + N * 1009 + K)
        ref = oracle.gemm(a, b)
        for variant in LADDER:
            print(f"case: edge {variant} {M}x{N}x{K}", flush=True)
            assert np.array_equal(_run(g, a, b, variant), ref), (variant, M, N, K)


# ---- the pages' worked example ------------------------------------------

def test_block_decomposition_T4_8x8(g):
    """8x8 integer matrices with T = 4 tiles (two k phases): the T = 4 rung
    reproduces C00 = A00 B00 + A01 B10 and the other blocks bit for bit."""
    rng = np.random.default_rng(42)
    a = rng.integers(-7, 8, (8, 8)).astype(np.float32)
    b = rng.integers(-7, 8, (8, 8)).astype(np.float32)
    c = _run(g, a, b, "tiled4")
    assert np.array_equal(c, oracle.gemm(a, b))
    blk = lambda x, r, s: np.ascontiguousarray(x[4 * r:4 * r + 4, 4 * s:4 * s + 4])  # noqa: E731
    for r in range(2):
        for s in range(2):
            want = oracle.gemm(blk(a, r, 0), blk(b, 0, s)) + oracle.gemm(blk(a, r, 1), blk(b, 1, s))
            assert np.array_equal(blk(c, r, s), want)


def test_tiled4_small_shapes(g):
    for (M, N, K) in [(8, 8, 8), (9, 7, 13), (33, 17, 65)]:
        a, b = make(M, N, K, "small_int", seed=M)
        assert np.array_equal(_run(g, a, b, "tiled4"), oracle.gemm(a, b))


# ---- leading dimensions, empty cases ------------------------------------

@pytest.mark.parametrize("variant", LADDER)
def test_leading_dimensions_and_padding_untouched(g, variant):
    M, N, K = 67, 45, 39
    lda, ldb, ldc = 41, 53, 47  # odd, larger than the row lengths
    a, b = make(M, N, K, "small_int", seed=5)
    dev = _dev()
    abuf = torch.full((M * lda,), float("nan"), dtype=torch.float32, device=dev)
    bbuf = torch.full((K * ldb,), float("nan"), dtype=torch.float32, device=dev)
    cbuf = torch.full((M * ldc,), -7.0, dtype=torch.float32, device=dev)
    abuf.view(M, lda)[:, :K] = torch.from_numpy(a).to(dev)
    bbuf.view(K, ldb)[:, :N] = torch.from_numpy(b).to(dev)
    stream = torch.cuda.current_stream().cuda_stream
    g.gemm_f32(M, N, K, abuf.data_ptr(), lda, bbuf.data_ptr(), ldb, cbuf.data_ptr(), ldc,
               variant, stream)
    torch.cuda.synchronize()
    c = cbuf.view(M, ldc).cpu().numpy()
    assert np.array_equal(c[:, :N], oracle.gemm(a, b))
    assert np.all(c[:, N:] == -7.0)


@pytest.mark.parametrize("variant", LADDER)
def test_aligned_padded_leading_dimensions(g, variant):
    """ld a multiple of 4 but larger than the row: the 128-bit path with padding."""
    M, N, K = 130, 132, 72
    lda, ldb, ldc = 80, 136, 140
    a, b = make(M, N, K, "uniform", seed=9)
    dev = _dev()
    abuf = torch.zeros((M, lda), dtype=torch.float32, device=dev)
    bbuf = torch.zeros((K, ldb), dtype=torch.float32, device=dev)
    cbuf = torch.full((M, ldc), 3.0, dtype=torch.float32, device=dev)
    abuf[:, :K] = torch.from_numpy(a).to(dev)
    bbuf[:, :N] = torch.from_numpy(b).to(dev)
    g.matmul(abuf[:, :K], bbuf[:, :N], out=cbuf[:, :N], variant=variant)
    torch.cuda.synchronize()
    c = cbuf.cpu().numpy()
    _tol_check(c[:, :N], oracle.gemm(a, b), K, variant)
    assert np.all(c[:, N:] == 3.0)


@pytest.mark.parametrize("variant", LADDER)
def test_k_zero_gives_zero_and_empty_is_noop(g, variant):
    dev = _dev()
    c = torch.full((5, 7), 9.0, device=dev)
    g.matmul(torch.empty((5, 0), device=dev), torch.empty((0, 7), device=dev), out=c,
             variant=variant)
    torch.cuda.synchronize()
    assert torch.all(c == 0).item()
    e = torch.full((0, 7), 1.0, device=dev)
    g.matmul(torch.empty((0, 3), device=dev), torch.ones((3, 7), device=dev), out=e,
             variant=variant)
    torch.cuda.synchronize()


# ---- named workloads ------------------------------------------------------

@pytest.mark.parametrize("variant", LADDER + ("tiled4",))
def test_workload_square_256(g, variant):
    w, a, b = make_workload("square_256")
    _tol_check(_run(g, a, b, variant), oracle.gemm(a, b), w.K, f"square_256 {variant}")


@pytest.mark.parametrize("variant", LADDER)
def test_workload_square_1024_int_bit_exact(g, variant):
    w, a, b = make_workload("square_1024_int")
    got = _run(g, a, b, variant)
    ref = oracle.gemm(a, b)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("name", ["square_4096", "ragged", "skinny_k64"])
def test_full_size_workload_sampled(g, name):
    """The launch configuration the benchmark times, at full size, checked on
    sampled outputs (plus whole edge rows and columns)."""
    w, a, b = make_workload(name)
    print(f"case: full-size {name} prod auto", flush=True)
    dev = _dev()
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    c = g.matmul(ta, tb, variant="prod")
    torch.cuda.synchronize()
    assert torch.isfinite(c).all().item()
    ii, jj = _sample_indices(w.M, w.N, 20000, seed=w.seed)
    got = c[torch.from_numpy(ii).to(dev), torch.from_numpy(jj).to(dev)].cpu().numpy()
    ref = oracle.gemm_elems(a, b, ii, jj)
    _tol_check(got, ref, w.K, f"{name} sampled")
    del c, ta, tb
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["square_4096", "ragged"])
def test_full_size_tiled_sampled(g, name):
    w, a, b = make_workload(name)
    dev = _dev()
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    for variant in ("tiled", "tiled32", "valu"):
        print(f"case: full-size {name} {variant}", flush=True)
        c = g.matmul(ta, tb, variant=variant)
        torch.cuda.synchronize()
        ii, jj = _sample_indices(w.M, w.N, 4000, seed=w.seed + 1)
        got = c[torch.from_numpy(ii).to(dev), torch.from_numpy(jj).to(dev)].cpu().numpy()
        _tol_check(got, oracle.gemm_elems(a, b, ii, jj), w.K, f"{name} {variant}")


@pytest.mark.parametrize("variant", LADDER)
def test_all_ones_full_ragged_shape(g, variant):
    """C = K everywhere for all-ones inputs at the ragged workload's full shape
    (a property that holds at any size; every edge tile is exercised)."""
    w = WORKLOADS["ragged"]
    dev = _dev()
    M, N, K = w.M, w.N, w.K
    c = g.matmul(torch.ones((M, K), device=dev), torch.ones((K, N), device=dev), variant=variant)
    torch.cuda.synchronize()
    assert torch.all(c == float(K)).item()


@pytest.mark.parametrize("variant", LADDER)
def test_identity_exact(g, variant):
    w, a, _ = make_workload("ragged")
    a = np.ascontiguousarray(a[:513])
    dev = _dev()
    eye = torch.eye(a.shape[1], device=dev)
    c = g.matmul(torch.from_numpy(a).to(dev), eye, variant=variant)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), a)


def test_streams_are_respected(g):
    """A call on a side stream is ordered after work queued before it there."""
    dev = _dev()
    a, b = make(300, 260, 100, "small_int", seed=77)
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = g.matmul(ta, tb, variant="prod")
    s.synchronize()
    assert np.array_equal(c.cpu().numpy(), oracle.gemm(a, b))


# ---- probes -----------------------------------------------------------

def test_stream_probes(g):
    dev = _dev()
    n = (1 << 20) + 3
    x = torch.randn(n, device=dev)
    y = torch.randn(n, device=dev)
    z = torch.empty(n, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    g.gemm_f32_probe_stream(g.PROBE_COPY, n, x.data_ptr(), 0, z.data_ptr(), s)
    torch.cuda.synchronize()
    assert torch.equal(z, x)
    g.gemm_f32_probe_stream(g.PROBE_VADD, n, x.data_ptr(), y.data_ptr(), z.data_ptr(), s)
    torch.cuda.synchronize()
    assert torch.equal(z, x + y)
    g.gemm_f32_probe_stream(g.PROBE_FILL, n, 0, 0, z.data_ptr(), s)
    torch.cuda.synchronize()
    assert torch.all(z == 1.0).item()


def test_mfma_probe_runs(g):
    dev = _dev()
    out = torch.zeros(8 * 4, device=dev)
    g.gemm_f32_probe_mfma(8, 10, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item() and torch.all(out != 0).item()


@pytest.mark.parametrize("shape", [16, 32])
def test_mfma16_probe_runs(g, shape):
    dev = _dev()
    out = torch.zeros(8 * 4, device=dev)
    g.gemm_f32_probe_mfma16(shape, 8, 10, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item() and torch.all(out > 0).item()


def test_valu_probe_runs(g):
    dev = _dev()
    out = torch.zeros(8 * 4, device=dev)
    g.gemm_f32_probe_valu(8, 10, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item() and torch.all(out != 0).item()


def test_lds_probe_runs(g):
    dev = _dev()
    out = torch.full((8 * 4,), -1.0, device=dev)
    g.gemm_f32_probe_lds(8, 10, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item() and torch.all(out >= 0).item()


def test_fused_probe_runs_and_reports_clock(g):
    """Each mode writes what it promises (every 1 KB run of the fused and
    store-only modes; one KB per wave for MFMA-only) and reports a plausible
    engine clock from its shader-clock and real-time counters."""
    dev = _dev()
    wgs, trips = 8, 32
    for mode in (g.FUSED_BOTH, g.FUSED_MFMA, g.FUSED_STORE):
        nbytes = g.gemm_f32_probe_fused_bytes(mode, wgs, trips)
        out = torch.full((nbytes // 4 + 64,), -5.0, device=dev)
        clocks = torch.zeros(2 * wgs * 4, dtype=torch.int64, device=dev)
        g.gemm_f32_probe_fused(mode, wgs, trips, out.data_ptr(), nbytes, clocks.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        body = out[: nbytes // 4]
        assert torch.isfinite(body).all().item() and not torch.any(body == -5.0).item(), mode
        assert torch.all(out[nbytes // 4:] == -5.0).item(), mode  # nothing past the buffer
        c = clocks.view(-1, 2).double()
        assert torch.all(c > 0).item(), mode
        mhz = (c[:, 0] / c[:, 1] * 100.0)
        assert torch.all((mhz > 300) & (mhz < 3500)).item(), (mode, mhz.tolist()[:4])


def test_device_props(g):
    d = g.gemm_f32_device_props(0)
    assert d["cus"] == torch.cuda.get_device_properties(0).multi_processor_count
    assert d["wave_size"] == 64 and d["clock_mhz"] > 500 and d["lds_bytes_per_cu"] >= 65536


@pytest.mark.parametrize("case", [(4608, 4096, 256, "small_int"), (4608, 4100, 128, "normal")])
def test_row_region_entry(g, case):
    """Entry 25 cuts C by rows: 4096 rows in one round of 256x256 tiles
    (entry 19), the other 512 in a second launch on their own entry.  Random
    samples plus every element of the rows on both sides of the cut."""
    M, N, K, dist = case
    assert g.gemm_f32_tile("prod", -1, M, N, K)["config"] == ROW_REGION_ENTRY
    print(f"case: row region {case}", flush=True)
    a, b = make(M, N, K, dist, seed=M + N + K)
    c = _run(g, a, b, "prod")
    ii, jj = _sample_indices(M, N, 20000, seed=K)
    rows = np.repeat(np.arange(4094, 4098), N)
    cols = np.tile(np.arange(N), 4)
    ii, jj = np.concatenate([ii, rows]), np.concatenate([jj, cols])
    want = oracle.gemm_elems(a, b, ii, jj)
    if dist == "small_int":
        assert np.array_equal(c[ii, jj], want)
    else:
        _tol_check(c[ii, jj], want, K, f"row region {case}")


def test_row_region_entry_without_a_cut(g):
    """Where no cut pays, entry 25 runs the product on the model's own entry."""
    a, b = make(600, 520, 96, "small_int", seed=25)
    print("case: row region, no cut, 600x520x96", flush=True)
    assert np.array_equal(_run(g, a, b, "prod", ROW_REGION_ENTRY), oracle.gemm(a, b))
