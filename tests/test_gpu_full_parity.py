"""GPU parity over EVERY element of the three large workloads.

Each rung of the kernel ladder (naive, textbook T = 16 and T = 32, the
padded T = 32 rung, the register-blocked VALU rung and the production
kernel in the launch configuration the benchmark times) computes the full
product of square 4096^3, ragged 4097x4095x2049 and skinny 16384^2 x 64 on
their seeded inputs, and the whole C is compared with the CPU oracle's
whole C: max |C - C_ref| <= 1e-4 sqrt(K) and ||C - C_ref||_F / ||C_ref||_F
<= 1e-5 over all M x N elements, in fp64 on the host.  The split-K path
(ragged, four chunks) and the 16-bit-input rung (bf16 and fp16 codes of the
same draws, against the 16-bit oracle) are held to the same bar in full.

The pages define every output element (the tiled kernel writes all of C
after its last k phase: ijyty.com steps ② and ⑧) and warn that a missing
second barrier or an edge element not loaded as zero shows only on products
with many k phases and ragged edges (geek-doc.cn "矩阵乘法 tiling", section
六) -- which is why these run at the workloads' full sizes.

The oracle's product of each workload is computed once (about 1.4 s for
4096^3 on 16 host threads) and kept while that workload's tests run.
"""
import time

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gemm_inputs import make_mixed_workload, make_workload  # noqa: E402
from parity_util import full_tol_check  # noqa: E402

LADDER = ("naive", "tiled", "tiled32", "tiled32_pad", "valu", "prod")
LARGE = ("square_4096", "ragged", "skinny_k64")
FORMATS = ("bf16", "f16")
_TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}

_cache: dict = {}


@pytest.fixture(scope="module")
def g():
    import tiled_fp32_gemm_03_amd as lib
    return lib


def _dev():
    return torch.device("cuda:0")


def _workload(key, build):
    """One workload's inputs on the device and the oracle's full product,
    built on first use; switching to another workload frees the last."""
    if key not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        t0 = time.perf_counter()
        _cache[key] = build()
        print(f"oracle: {key} in {time.perf_counter() - t0:.2f} s "
              f"({oracle.num_threads()} threads)", flush=True)
    return _cache[key]


def _fp32(name):
    def build():
        w, a, b = make_workload(name)
        ref = oracle.gemm(a, b)
        return w, torch.from_numpy(a).to(_dev()), torch.from_numpy(b).to(_dev()), ref
    return _workload(("f32", name), build)


def _mixed(name, fmt):
    def build():
        w, a, b = make_mixed_workload(name, fmt)
        ref = oracle.gemm_mixed(a, b, fmt)
        ta = torch.from_numpy(a.view(np.int16)).to(_dev()).view(_TORCH16[fmt])
        tb = torch.from_numpy(b.view(np.int16)).to(_dev()).view(_TORCH16[fmt])
        return w, ta, tb, ref
    return _workload((fmt, name), build)


def _check(c, ref, K, what):
    torch.cuda.synchronize()
    got = c.cpu().numpy()
    e = full_tol_check(got, ref, K, what)
    print(f"  {what}: max err {e['max_err']:.3g} at {e['where']}, rel fro {e['rel_fro']:.3g} "
          f"over {got.size} elements", flush=True)


@pytest.mark.parametrize("name,variant", [(n, v) for n in LARGE for v in LADDER])
def test_every_rung_full_matrix(g, name, variant):
    w, ta, tb, ref = _fp32(name)
    print(f"case: full matrix {name} {variant}", flush=True)
    c = g.matmul(ta, tb, variant=variant)
    _check(c, ref, w.K, f"{name} {variant}")


def test_splitk_ragged_full_matrix(g):
    """The ragged workload through an explicit four-way K split."""
    w, ta, tb, ref = _fp32("ragged")
    print("case: full matrix ragged split-K 4 chunks", flush=True)
    c = g.matmul_splitk(ta, tb, config=0, splits=4)
    _check(c, ref, w.K, "ragged splitk4")


@pytest.mark.parametrize("name,fmt", [(n, f) for n in LARGE for f in FORMATS])
def test_mixed_full_matrix(g, name, fmt):
    """The workload's draws rounded to 16-bit codes, automatic entry."""
    w, ta, tb, ref = _mixed(name, fmt)
    print(f"case: full matrix {name} {fmt}", flush=True)
    c = g.matmul_mixed(ta, tb)
    _check(c, ref, w.K, f"{name} {fmt}")


def test_release_full_size_buffers():
    """Not a check: frees the cached workload before the next module."""
    _cache.clear()
    torch.cuda.empty_cache()
