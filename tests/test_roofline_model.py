"""The benchmark's per-XCD panel floor (roofline.xcd_panel_bytes), on the CPU.

Hand-derived cases: on 4096^3 with 256 x 256 tiles and one persistent
workgroup per CU, each of the 8 XCDs walks a block of 8 tile rows by 4 tile
columns, so each A row panel is fetched by 4 L2s and each B column panel by
2; with a single L2 every panel is fetched once and the floor is the
compulsory traffic.
"""
from tiled_fp32_gemm_03_amd import roofline as rf


def test_square_4096_panels():
    f = rf.xcd_panel_bytes(4096, 4096, 4096, 256, 256, 256)
    assert f["a_panel_fetches"] == 8 * 8 and f["b_panel_fetches"] == 8 * 4
    panel = 256 * 4096 * 4
    assert f["read_bytes"] == (64 + 32) * panel
    assert f["write_bytes"] == 4096 * 4096 * 4


def test_one_l2_is_compulsory():
    for (M, N, K) in [(4096, 4096, 4096), (1024, 768, 300), (512, 512, 64)]:
        f = rf.xcd_panel_bytes(M, N, K, 256, 256, 64, xcds=1)
        assert f["bytes"] == rf.compulsory_bytes(M, N, K)


def test_every_tile_is_walked_once():
    # A persistent grid smaller than the tile count still touches every row
    # and column panel somewhere.
    f = rf.xcd_panel_bytes(4096, 8192, 1024, 256, 256, 100)
    assert f["a_panel_fetches"] >= 16 and f["b_panel_fetches"] >= 32
