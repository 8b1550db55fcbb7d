"""GPU parity of the split-K form of the production kernel (gemm_f32_splitk).

Each chunk of K is an ordinary product over a sub-range of k and the slabs
are summed in chunk order, so the bars are the ladder's: bit-exact on
integer inputs (every partial sum is an integer below 2^24), the fp32
tolerance otherwise.  A fixed plan must also give the same bits every run.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gemm_inputs import make, make_workload  # noqa: E402
from parity_util import sample_indices, tol_check  # noqa: E402


@pytest.fixture(scope="module")
def g():
    import tiled_fp32_gemm_03_amd as lib
    return lib


def _dev():
    return torch.device("cuda:0")


def _run(g, a, b, config=-1, splits=0, workspace=None):
    ta = torch.from_numpy(a).to(_dev())
    tb = torch.from_numpy(b).to(_dev())
    c = g.matmul_splitk(ta, tb, config=config, splits=splits, workspace=workspace)
    torch.cuda.synchronize()
    return c.cpu().numpy()


CASES = [  # (M, N, K, config, splits)
    (1024, 1024, 1024, -1, 0), (300, 260, 1000, 0, 3), (257, 383, 129, 0, 2),
    (257, 383, 129, 0, 5), (128, 128, 4096, 0, 16), (65, 70, 1001, 3, 0), (1, 300, 700, -1, 4),
    (200, 1, 333, -1, 3), (512, 512, 40, 0, 2), (777, 555, 2049, 4, 0), (130, 129, 31, 0, 4),
    (512, 384, 2048, 2, 4), (600, 520, 1536, 12, 3), (300, 300, 1000, 7, 2),
    # entry 23: the direct-load kernel per chunk, ragged tiles and a short last
    # chunk; K = 1000 is no multiple of its k step and takes entry 0's kernel
    (512, 512, 8192, 23, 16), (300, 260, 992, 23, 3), (128, 128, 4096, 23, 16),
    (1024, 640, 4096, 23, 4), (260, 300, 1000, 23, 3), (1536, 1280, 2048, -1, 0),
]


@pytest.mark.parametrize("case", CASES)
def test_integer_bit_exact(g, case):
    M, N, K, cfg, splits = case
    plan = g.gemm_f32_splitk_plan(M, N, K, cfg, splits)
    print(f"case: splitk {case} plan {plan}", flush=True)
    a, b = make(M, N, K, "small_int", seed=M + N + K + splits)
    assert np.array_equal(_run(g, a, b, cfg, splits), oracle.gemm(a, b)), (case, plan)


@pytest.mark.parametrize("case", CASES)
def test_float_tolerance(g, case):
    M, N, K, cfg, splits = case
    print(f"case: splitk float {case}", flush=True)
    a, b = make(M, N, K, "normal", seed=3 * M + N + K)
    tol_check(_run(g, a, b, cfg, splits), oracle.gemm(a, b), K, f"splitk {case}")


def test_plans_really_split(g):
    assert g.gemm_f32_splitk_plan(1024, 1024, 4096)["splits"] > 1
    assert g.gemm_f32_splitk_plan(257, 383, 129, 0, 5)["splits"] == 5
    assert g.gemm_f32_splitk_plan(128, 128, 4096, 0, 16)["splits"] == 16


def test_same_bits_every_run(g):
    a, b = make(700, 650, 3000, "uniform", seed=21)
    ta, tb = torch.from_numpy(a).to(_dev()), torch.from_numpy(b).to(_dev())
    first = g.matmul_splitk(ta, tb, splits=6)
    for _ in range(3):
        again = g.matmul_splitk(ta, tb, splits=6)
        torch.cuda.synchronize()
        assert torch.equal(first, again)


def test_workload_square_1024_int(g):
    w, a, b = make_workload("square_1024_int")
    print("case: splitk square_1024_int auto", flush=True)
    assert np.array_equal(_run(g, a, b), oracle.gemm(a, b))


def test_ragged_full_size_sampled(g):
    """The ragged workload's full shape through an explicit 4-way split."""
    w, a, b = make_workload("ragged")
    print("case: splitk ragged 4 splits", flush=True)
    ta, tb = torch.from_numpy(a).to(_dev()), torch.from_numpy(b).to(_dev())
    c = g.matmul_splitk(ta, tb, config=0, splits=4)
    torch.cuda.synchronize()
    ii, jj = sample_indices(w.M, w.N, 20000, seed=w.seed + 7)
    got = c[torch.from_numpy(ii).to(_dev()), torch.from_numpy(jj).to(_dev())].cpu().numpy()
    tol_check(got, oracle.gemm_elems(a, b, ii, jj), w.K, "ragged splitk")


def test_deep_k_workload_full(g):
    """The deep-K workload (few output tiles, long K) in full through the
    automatic plan, which splits it into many chunks."""
    w, a, b = make_workload("deep_k")
    plan = g.gemm_f32_splitk_plan(w.M, w.N, w.K)
    assert plan["splits"] >= 16
    print(f"case: splitk deep_k auto {plan}", flush=True)
    tol_check(_run(g, a, b), oracle.gemm(a, b), w.K, "deep_k splitk")


def test_padding_untouched_and_shared_workspace(g):
    """One oversized, dirty workspace serves several shapes; C's ldc padding
    is never written."""
    ws = torch.full((64 << 20,), float("nan"), dtype=torch.float32, device=_dev())
    for (M, N, K, splits) in [(300, 260, 1000, 3), (520, 264, 700, 5), (64, 64, 4096, 8)]:
        print(f"case: splitk shared workspace {M}x{N}x{K}/{splits}", flush=True)
        a, b = make(M, N, K, "small_int", seed=M * N + K)
        cbuf = torch.full((M, N + 5), -9.0, dtype=torch.float32, device=_dev())
        g.matmul_splitk(torch.from_numpy(a).to(_dev()), torch.from_numpy(b).to(_dev()),
                        out=cbuf[:, :N], config=0, splits=splits, workspace=ws)
        torch.cuda.synchronize()
        got = cbuf.cpu().numpy()
        assert np.array_equal(got[:, :N], oracle.gemm(a, b))
        assert np.all(got[:, N:] == -9.0)


def test_k_zero_and_empty(g):
    c = torch.full((6, 7), 2.0, dtype=torch.float32, device=_dev())
    g.gemm_f32_splitk(6, 7, 0, 0, 1, 0, 7, c.data_ptr(), 7, -1, 0, 0, 0,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(c == 0).item()


def test_runs_on_the_given_stream(g):
    a, b = make(512, 512, 2048, "small_int", seed=5)
    ta, tb = torch.from_numpy(a).to(_dev()), torch.from_numpy(b).to(_dev())
    side = torch.cuda.Stream()
    c = torch.empty((512, 512), dtype=torch.float32, device=_dev())
    with torch.cuda.stream(side):
        ws = torch.empty(g.gemm_f32_splitk_plan(512, 512, 2048, 0, 4)["workspace_bytes"] // 4,
                         dtype=torch.float32, device=_dev())
        g.matmul_splitk(ta, tb, out=c, config=0, splits=4, workspace=ws)
    side.synchronize()
    assert np.array_equal(c.cpu().numpy(), oracle.gemm(a, b))
