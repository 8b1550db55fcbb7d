"""GPU parity of the 16-bit-input product (gemm_mixed) against the oracle.

Inputs are bf16 or fp16 codes from the seeded generator; the oracle reads the
same codes (oracle.gemm_mixed).  Bars, from the arithmetic: every product of
two 16-bit values is exact in fp32, so the only error is fp32 accumulation --
  * integer-valued inputs whose partial sums stay below 2^24: bit-exact;
  * other inputs: the fp32 bar of the ladder (max |C - C_ref| <= 1e-4 sqrt(K),
    relative Frobenius <= 1e-5).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gemm_inputs import WORKLOADS, make_mixed, make_mixed_workload  # noqa: E402
from parity_util import sample_indices, tol_check  # noqa: E402

FORMATS = ("bf16", "f16")
DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module")
def g():
    import tiled_fp32_gemm_03_amd as lib
    return lib


def _dev():
    return torch.device("cuda:0")


def _to_dev(codes: np.ndarray, fmt: str):
    return torch.from_numpy(codes.view(np.int16)).to(_dev()).view(DTYPE[fmt])


def _run(g, a, b, fmt, config=-1):
    c = g.matmul_mixed(_to_dev(a, fmt), _to_dev(b, fmt), config=config)
    torch.cuda.synchronize()
    return c.cpu().numpy()


SHAPES = [(1, 1, 1), (5, 7, 3), (64, 64, 64), (100, 37, 129), (257, 255, 130), (300, 513, 65),
          (128, 128, 8), (33, 260, 200)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", SHAPES)
def test_small_integer_bit_exact(g, fmt, shape):
    M, N, K = shape
    print(f"case: mixed {fmt} small_int {shape}", flush=True)
    a, b = make_mixed(M, N, K, "small_int", seed=M + N + K, fmt=fmt)
    assert np.array_equal(_run(g, a, b, fmt), oracle.gemm_mixed(a, b, fmt))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dist", ["uniform", "normal"])
def test_small_tolerance(g, fmt, shape, dist):
    M, N, K = shape
    print(f"case: mixed {fmt} {dist} {shape}", flush=True)
    a, b = make_mixed(M, N, K, dist, seed=7 * M + N + K, fmt=fmt)
    tol_check(_run(g, a, b, fmt), oracle.gemm_mixed(a, b, fmt), K, f"{fmt} {dist} {shape}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_every_config(g, fmt):
    for cfg in range(g.gemm_mixed_num_configs()):
        for (M, N, K) in [(512, 512, 256), (257, 383, 129), (1, 300, 40), (200, 1, 33),
                          (300, 260, 17), (256, 256, 64)]:
            print(f"case: mixed {fmt} config {cfg} {M}x{N}x{K}", flush=True)
            a, b = make_mixed(M, N, K, "small_int", seed=cfg + M, fmt=fmt)
            assert np.array_equal(_run(g, a, b, fmt, cfg), oracle.gemm_mixed(a, b, fmt)), \
                (cfg, M, N, K)
            a, b = make_mixed(M, N, K, "normal", seed=cfg + N, fmt=fmt)
            tol_check(_run(g, a, b, fmt, cfg), oracle.gemm_mixed(a, b, fmt), K, f"cfg {cfg}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_edge_sweep(g, fmt):
    sizes = [1, 7, 8, 9, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
    rng = np.random.default_rng(77)
    combos = {(s, s, s) for s in sizes}
    while len(combos) < 40:
        combos.add(tuple(int(x) for x in rng.choice(sizes, 3)))
    for (M, N, K) in sorted(combos):
        print(f"case: mixed {fmt} edge {M}x{N}x{K}", flush=True)
        a, b = make_mixed(M, N, K, "small_int", seed=M * 1009 + N * 31 + K, fmt=fmt)
        assert np.array_equal(_run(g, a, b, fmt), oracle.gemm_mixed(a, b, fmt)), (M, N, K)


@pytest.mark.parametrize("fmt", FORMATS)
def test_unaligned_operands(g, fmt):
    """A and B start one element into wider buffers with odd leading
    dimensions, so every 128-bit load is only 2-byte aligned."""
    M, N, K = 300, 270, 150
    a, b = make_mixed(M, N, K, "small_int", seed=11, fmt=fmt)
    abuf = np.zeros((M, K + 3), np.uint16)
    bbuf = np.zeros((K, N + 5), np.uint16)
    abuf[:, 1:K + 1] = a
    bbuf[:, 1:N + 1] = b
    ta, tb = _to_dev(abuf, fmt), _to_dev(bbuf, fmt)
    c = torch.empty((M, N), dtype=torch.float32, device=_dev())
    print(f"case: mixed {fmt} unaligned", flush=True)
    g.gemm_mixed(M, N, K, ta.data_ptr() + 2, K + 3, tb.data_ptr() + 2, N + 5, c.data_ptr(), N,
                 fmt, -1, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), oracle.gemm_mixed(a, b, fmt))


@pytest.mark.parametrize("fmt", FORMATS)
def test_padded_leading_dimensions_and_untouched_padding(g, fmt):
    M, N, K = 520, 264, 192
    a, b = make_mixed(M, N, K, "small_int", seed=12, fmt=fmt)
    ta = torch.zeros((M, K + 16), dtype=DTYPE[fmt], device=_dev())
    tb = torch.zeros((K, N + 8), dtype=DTYPE[fmt], device=_dev())
    ta[:, :K] = _to_dev(a, fmt)
    tb[:, :N] = _to_dev(b, fmt)
    cbuf = torch.full((M, N + 3), -7.0, dtype=torch.float32, device=_dev())
    for cfg in range(g.gemm_mixed_num_configs()):
        print(f"case: mixed {fmt} padded ld config {cfg}", flush=True)
        g.matmul_mixed(ta[:, :K], tb[:, :N], out=cbuf[:, :N], config=cfg)
        torch.cuda.synchronize()
        got = cbuf.cpu().numpy()
        assert np.array_equal(got[:, :N], oracle.gemm_mixed(a, b, fmt))
        assert np.all(got[:, N:] == -7.0)


@pytest.mark.parametrize("fmt", FORMATS)
def test_k_zero_gives_zero_and_empty_is_noop(g, fmt):
    c = torch.full((5, 9), 3.0, dtype=torch.float32, device=_dev())
    g.gemm_mixed(5, 9, 0, 0, 1, 0, 9, c.data_ptr(), 9, fmt, -1,
                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(c == 0).item()
    c.fill_(3.0)
    g.gemm_mixed(0, 9, 4, 0, 4, 0, 9, c.data_ptr(), 9, fmt, -1, 0)
    g.gemm_mixed(5, 0, 4, 0, 4, 0, 1, c.data_ptr(), 9, fmt, -1, 0)
    torch.cuda.synchronize()
    assert torch.all(c == 3.0).item()


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("name", ["square_4096", "ragged", "skinny_k64"])
def test_full_size_workload_sampled(g, fmt, name):
    """Each full-size workload rounded to the 16-bit format, in the launch
    configuration the ladder times, on sampled elements and edge lines."""
    w, a, b = make_mixed_workload(name, fmt)
    print(f"case: mixed {fmt} full-size {name}", flush=True)
    c = g.matmul_mixed(_to_dev(a, fmt), _to_dev(b, fmt))
    torch.cuda.synchronize()
    assert torch.isfinite(c).all().item()
    ii, jj = sample_indices(w.M, w.N, 20000, seed=w.seed)
    got = c[torch.from_numpy(ii).to(_dev()), torch.from_numpy(jj).to(_dev())].cpu().numpy()
    tol_check(got, oracle.gemm_mixed_elems(a, b, fmt, ii, jj), w.K, f"{fmt} {name}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_all_ones_full_ragged_shape(g, fmt):
    w = WORKLOADS["ragged"]
    one = 0x3F80 if fmt == "bf16" else 0x3C00
    a = np.full((w.M, w.K), one, np.uint16)
    b = np.full((w.K, w.N), one, np.uint16)
    for cfg in range(g.gemm_mixed_num_configs()):
        print(f"case: mixed {fmt} all-ones ragged config {cfg}", flush=True)
        c = g.matmul_mixed(_to_dev(a, fmt), _to_dev(b, fmt), config=cfg)
        torch.cuda.synchronize()
        assert torch.all(c == float(w.K)).item()


DIRECT_ENTRIES = (3, 4)  # direct loads on 16x16x32 (its own summation order) and 32x32x16 MFMAs


@pytest.mark.parametrize("entry", DIRECT_ENTRIES)
@pytest.mark.parametrize("fmt", FORMATS)
def test_direct_entry_many_tiles(g, fmt, entry):
    """A direct-load entry where workgroups walk two tiles and the last
    tile row and column are moved back inside C: exact on small integers
    (sampled elements plus whole edge rows and columns), within the fp32
    bar on normal inputs (sampled)."""
    M, N, K = 4400, 4352, 128
    for dist in ("small_int", "normal"):
        print(f"case: mixed {fmt} direct entry {entry} {M}x{N}x{K} {dist}", flush=True)
        a, b = make_mixed(M, N, K, dist, seed=M + K, fmt=fmt)
        c = g.matmul_mixed(_to_dev(a, fmt), _to_dev(b, fmt), config=entry)
        torch.cuda.synchronize()
        ii, jj = sample_indices(M, N, 20000, seed=K)
        got = c[torch.from_numpy(ii).to(_dev()), torch.from_numpy(jj).to(_dev())].cpu().numpy()
        ref = oracle.gemm_mixed_elems(a, b, fmt, ii, jj)
        if dist == "small_int":
            assert np.array_equal(got, ref)
            rows = np.array([0, 255, 4143, 4144, M - 1])
            edge_i = np.repeat(rows, N)
            edge_j = np.tile(np.arange(N), len(rows))
            got_e = c[torch.from_numpy(edge_i).to(_dev()),
                      torch.from_numpy(edge_j).to(_dev())].cpu().numpy()
            assert np.array_equal(got_e, oracle.gemm_mixed_elems(a, b, fmt, edge_i, edge_j))
        else:
            tol_check(got, ref, K, f"{fmt} direct entry")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [(512, 768, 64), (1024, 512, 1024), (300, 513, 192)])
def test_direct_32x32_entry_matches_register_staged_bitwise(g, fmt, shape):
    """Entry 4 runs the direct-load pipeline on the 32x32x16 MFMAs of entry
    0, adding each element's k in the same 16-deep groups in ascending
    order, so on float inputs its result equals entry 0's bit for bit
    (these shapes fit its kernel: K a multiple of 64, at least 256 rows and
    columns, one or more tiles per workgroup), and it meets the fp32 bar
    against the oracle."""
    M, N, K = shape
    print(f"case: mixed {fmt} entry 4 against entry 0 {shape}", flush=True)
    a, b = make_mixed(M, N, K, "normal", seed=M + 3 * N + K, fmt=fmt)
    c4 = _run(g, a, b, fmt, 4)
    assert np.array_equal(c4, _run(g, a, b, fmt, 0))
    tol_check(c4, oracle.gemm_mixed(a, b, fmt), K, f"{fmt} entry 4 {shape}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_entries_agree_bitwise_on_ragged_floats(g, fmt):
    """Every 32x32x16 entry sums each element in the same k order, whatever
    the tile size or whether its edge tiles were moved back inside C
    (overlapping a neighbour), so they agree bit for bit on float inputs.
    (On these shapes the direct-load entry takes entry 0's kernel: K is not
    a multiple of its step.)"""
    for (M, N, K) in [(1000, 1003, 515), (700, 300, 129)]:
        a, b = make_mixed(M, N, K, "normal", seed=M + N, fmt=fmt)
        ref = _run(g, a, b, fmt, 0)
        for cfg in range(1, g.gemm_mixed_num_configs()):
            print(f"case: mixed {fmt} bitwise agreement config {cfg} {M}x{N}x{K}", flush=True)
            assert np.array_equal(_run(g, a, b, fmt, cfg), ref), (fmt, cfg, M, N, K)


def test_runs_on_the_given_stream(g):
    a, b = make_mixed(384, 384, 256, "small_int", seed=3, fmt="bf16")
    ta, tb = _to_dev(a, "bf16"), _to_dev(b, "bf16")
    side = torch.cuda.Stream()
    c = torch.empty((384, 384), dtype=torch.float32, device=_dev())
    with torch.cuda.stream(side):
        g.matmul_mixed(ta, tb, out=c)
    side.synchronize()
    assert np.array_equal(c.cpu().numpy(), oracle.gemm_mixed(a, b, "bf16"))


def test_tensor_wrapper_checks(g):
    a = torch.zeros((4, 4), dtype=torch.bfloat16, device=_dev())
    h = torch.zeros((4, 4), dtype=torch.float16, device=_dev())
    with pytest.raises(TypeError):
        g.matmul_mixed(a, h)
    with pytest.raises(TypeError):
        g.matmul_mixed(a.float(), a.float())
    with pytest.raises(TypeError):
        g.matmul_mixed(a, a, format="f16")
    c = g.matmul_mixed(a.view(torch.int16), a.view(torch.int16), format="bf16")
    torch.cuda.synchronize()
    assert torch.all(c == 0).item()
