"""Pins of the oracle's counting model against numbers the pages print."""
import json
import os

import pytest

from oracle import model

with open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")) as _f:
    G = json.load(_f)


def _close(value, entry):
    ref = entry["value"]
    rel = entry.get("rel", 0.0)
    return abs(value - ref) <= rel * abs(ref) + 1e-12


def test_square_4096_numbers():
    g = G["square_4096"]
    n = g["N"]
    assert model.input_bytes_square(n) == g["input_bytes"]["value"] * 2 ** 20
    assert _close(model.flops(n, n, n), g["flops"])
    assert _close(model.naive_loads(n, n, n), g["naive_loads_elements"])
    assert _close(model.naive_loads(n, n, n) * model.FLOAT_BYTES, g["naive_load_bytes"])
    assert _close(model.tiled_loads(n, n, n, 32), g["tiled32_loads_elements"])
    assert _close(model.tiled_loads(n, n, n, 32) * model.FLOAT_BYTES, g["tiled32_load_bytes"])
    assert model.naive_loads(n, n, n) == g["naive_over_tiled32"]["value"] * model.tiled_loads(n, n, n, 32)


def test_tile_step_numbers():
    g = G["tile_step"]
    tiled, naive = model.tile_step_loads(4)
    assert tiled == g["T4_tiled_elements"]["value"]
    assert tiled // 2 == g["T4_A_tile_elements"]["value"]
    assert model.reuse_factor(4) == g["T4_naive_reads_of_a11"]["value"]
    for t in (2, 4, 8, 16, 32):
        tiled, naive = model.tile_step_loads(t)
        assert (tiled, naive) == (2 * t * t, 2 * t ** 3)
        assert model.reuse_factor(t) == t


@pytest.mark.parametrize("n,t", [(64, 4), (256, 16), (4096, 32), (1024, 16)])
def test_tiled_over_naive_is_T_when_divisible(n, t):
    assert model.naive_loads(n, n, n) == t * model.tiled_loads(n, n, n, t)
    assert model.tiled_loads(n, n, n, t) == 2 * n ** 3 // t


def test_ragged_uses_ceilings():
    # 5 x 5 x 5 with T = 4: 2x2 tiles, 2 k-steps, 32 elements per step.
    assert model.tiled_loads(5, 5, 5, 4) == 4 * 2 * 32
    assert model.blocked_loads(5, 9, 3, 4, 8, 2) == (2 * 2) * 2 * (4 * 2 + 2 * 8)


def test_intensities():
    g = G["intensity"]
    assert model.intensity_naive() == g["naive"]["value"]
    assert model.intensity_tiled(16) == g["tiled16"]["value"]
    assert model.intensity_tiled(32) == g["tiled32"]["value"]
    assert 2 * 32 == g["flop_per_element_block32"]["value"]
    assert _close(model.intensity_vector_add(), g["vector_add"])
    r = G["roofline"]
    ridge = model.ridge(r["h100_peak_fp32_tflops"]["value"] * 1e12, r["h100_peak_tbps"]["value"] * 1e12)
    assert abs(ridge - r["h100_ridge"]["value"]) <= 0.05 * r["h100_ridge"]["value"]
    assert _close(r["h100_ridge"]["value"] / model.intensity_vector_add(), g["vector_add_below_ridge"])


def test_typical_card_roofline():
    r = G["roofline"]
    bw, peak = r["typical_card_bw_Bps"]["value"], r["typical_card_peak_flops"]["value"]
    assert model.attainable(model.intensity_naive(), peak, bw) == r["typical_card_naive_ceiling_flops"]["value"]
    assert peak / model.intensity_naive() == r["typical_card_naive_feed_Bps"]["value"]
    # on the compute roof once past the ridge
    assert model.attainable(1e6, peak, bw) == peak


def test_index_mapping_example():
    g = G["index_mapping"]
    assert model.textbook_owner(g["T"], tuple(g["blockIdx"]), tuple(g["threadIdx"])) == (g["row"], g["col"])


def test_higham_gamma():
    assert model.higham_gamma(0) == 0.0
    u = 2.0 ** -24
    assert abs(model.higham_gamma(4096) - 4096 * u / (1 - 4096 * u)) < 1e-18
    assert model.higham_gamma(2 ** 24) == float("inf")
