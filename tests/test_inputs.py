"""The seeded input generator: determinism, distributions, shapes."""
import json
import os

import numpy as np
import pytest

from gemm_inputs import WORKLOADS, make, make_workload, sha256

HASHES = os.path.join(os.path.dirname(__file__), "golden", "input_hashes.json")


def test_workload_table():
    assert [w.name for w in WORKLOADS.values()] == [
        "square_256", "square_1024_int", "square_4096", "ragged", "skinny_k64", "deep_k"]
    r = WORKLOADS["ragged"]
    for d in (r.M, r.N, r.K):
        assert all(d % t for t in (4, 16, 32, 64, 128, 256))
    assert [w.seed for w in WORKLOADS.values()] == [0, 1, 2, 3, 4, 5]


def test_deterministic():
    a1, b1 = make(33, 17, 65, "uniform", 9)
    a2, b2 = make(33, 17, 65, "uniform", 9)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)
    a3, _ = make(33, 17, 65, "uniform", 10)
    assert not np.array_equal(a1, a3)


@pytest.mark.parametrize("dist", ["uniform", "int4", "normal", "small_int", "ones"])
def test_distributions(dist):
    a, b = make(300, 200, 100, dist, 0)
    assert a.shape == (300, 100) and b.shape == (100, 200)
    assert a.dtype == np.float32 and a.flags.c_contiguous and b.flags.c_contiguous
    if dist == "uniform":
        assert a.min() >= -1.0 and a.max() <= 1.0 and abs(float(a.mean())) < 0.02
    elif dist == "int4":
        assert set(np.unique(a).tolist()) == set(range(-4, 5))
    elif dist == "normal":
        assert abs(float(a.std()) - 1.0) < 0.02
    elif dist == "ones":
        assert np.all(a == 1.0)


def test_hashes_match_golden():
    """Generator output is pinned by hash (tests/golden/input_hashes.json,
    written by tests/golden/write_input_hashes.py)."""
    with open(HASHES) as f:
        ref = json.load(f)
    for name in ("square_256", "square_1024_int"):
        w, a, b = make_workload(name)
        assert sha256(a) == ref[name]["A"], name
        assert sha256(b) == ref[name]["B"], name
