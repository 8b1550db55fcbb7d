"""The C-ABI library on the host: it loads, exports every symbol the headers
declare, validates arguments before touching the GPU, and answers launch-table
queries.  No compute call is made here (no GPU needed)."""
import ctypes
import os
import re

import pytest

import tiled_fp32_gemm_03_amd as g
from oracle import model
from tiled_fp32_gemm_03_amd import roofline

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def _declared_functions():
    names = []
    for fname in sorted(os.listdir(INCLUDE)):
        if not fname.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, fname)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(gemm_\w*)\s*\(", text, re.M):
            names.append(m.group(1))
    return names


def test_headers_declare_expected_entry_points():
    names = set(_declared_functions())
    assert {"gemm_f32", "gemm_f32_ex", "gemm_f32_tile", "gemm_f32_num_configs",
            "gemm_f32_status_string", "gemm_f32_version", "gemm_f32_probe_stream",
            "gemm_f32_probe_mfma", "gemm_f32_probe_mfma_flops", "gemm_f32_probe_mfma16",
            "gemm_f32_probe_mfma16_flops", "gemm_f32_probe_valu",
            "gemm_f32_probe_valu_flops", "gemm_f32_probe_lds", "gemm_f32_probe_lds_bytes",
            "gemm_f32_probe_fused", "gemm_f32_probe_fused_flops", "gemm_f32_probe_fused_bytes",
            "gemm_f32_device_props", "gemm_mixed", "gemm_mixed_num_configs", "gemm_mixed_tile", "gemm_f32_splitk",
            "gemm_f32_splitk_plan"} <= names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(g.library_path())
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert name in g.exported_symbols(), name


def test_noalloc_validation_before_any_gpu_call():
    """The no-allocation split-K entry checks its arguments and its plan's
    size against the fixed scratch before it touches the GPU."""
    lib = g._lib
    f = lib.gemm_f32_splitk_noalloc
    assert f(-1, 4, 4, None, 4, None, 4, None, 4, -1, 0, None) == 1
    assert f(4, 4, 4, None, 3, None, 4, None, 4, -1, 0, None) == 2
    assert f(4, 4, 4, None, 4, None, 4, None, 4, -1, -1, None) == 8
    assert f(4, 4, 4, None, 4, None, 4, None, 4, 99, 0, None) == 7
    assert f(4, 4, 4, None, 4, None, 4, None, 4, -1, 0, None) == 3
    assert f(0, 4, 4, None, 4, None, 4, None, 4, -1, 0, None) == 0
    plan = g.gemm_f32_splitk_plan(2048, 2048, 4096, 0, 8)
    assert plan["workspace_bytes"] > g.NOALLOC_SCRATCH_BYTES
    assert f(2048, 2048, 4096, 256, 4096, 256, 2048, 256, 2048, 0, 8, None) == 10
    assert "scratch" in g.gemm_f32_status_string(10)
    hdr = open(os.path.join(INCLUDE, "gemm_f32.h")).read()
    m = re.search(r"#define GEMM_F32_NOALLOC_SCRATCH_BYTES \((\d+)LL << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == g.NOALLOC_SCRATCH_BYTES


def test_version():
    assert "gfx950" in g.gemm_f32_version()


def _call(M, N, K, A=0, lda=None, B=0, ldb=None, C=0, ldc=None, variant=0, config=-1):
    lda = max(1, K) if lda is None else lda
    ldb = max(1, N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    return g._lib.gemm_f32_ex(M, N, K, A or None, lda, B or None, ldb, C or None, ldc,
                              variant, config, None)


def test_validation_codes():
    ok, bad_dim, bad_ld, null, bad_var, misal, bad_cfg = 0, 1, 2, 3, 4, 6, 7
    assert _call(-1, 4, 4) == bad_dim
    assert _call(4, -1, 4) == bad_dim
    assert _call(4, 4, -1) == bad_dim
    assert _call(4, 4, 4, lda=3) == bad_ld
    assert _call(4, 4, 4, ldb=3) == bad_ld
    assert _call(4, 4, 4, ldc=3) == bad_ld
    assert _call(4, 4, 0, lda=0) == bad_ld          # lda >= max(1, K)
    assert _call(4, 4, 4, variant=7) == bad_var
    assert _call(4, 4, 4, variant=-1) == bad_var
    assert _call(4, 4, 4, variant=2, config=99) == bad_cfg
    assert _call(4, 4, 4, variant=0, config=1) == bad_cfg
    assert _call(4, 4, 4, variant=2, config=-2) == bad_cfg
    assert _call(4, 4, 4) == null                    # C missing
    assert _call(4, 4, 4, C=256) == null             # A, B missing
    assert _call(4, 4, 4, A=256, B=512, C=258) == misal
    assert _call(4, 4, 4, A=257, B=512, C=256) == misal
    # empty output: nothing to do, no pointers needed, nothing launched
    assert _call(0, 4, 4) == ok
    assert _call(4, 0, 4) == ok
    for code in range(0, 10):
        assert g.gemm_f32_status_string(code) != "unknown status"
    assert g.gemm_f32_status_string(1234) == "unknown status"


def _mixed(M, N, K, A=0, lda=None, B=0, ldb=None, C=0, ldc=None, fmt=0, config=-1):
    lda = max(1, K) if lda is None else lda
    ldb = max(1, N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    return g._lib.gemm_mixed(M, N, K, A or None, lda, B or None, ldb, C or None, ldc, fmt,
                             config, None)


def test_mixed_validation_codes():
    ok, bad_dim, bad_ld, null, misal, bad_cfg, bad_arg = 0, 1, 2, 3, 6, 7, 8
    assert _mixed(-1, 4, 4) == bad_dim
    assert _mixed(4, 4, 4, lda=3) == bad_ld
    assert _mixed(4, 4, 4, ldb=3) == bad_ld
    assert _mixed(4, 4, 4, ldc=3) == bad_ld
    assert _mixed(4, 4, 4, fmt=2) == bad_arg
    assert _mixed(4, 4, 4, fmt=-1) == bad_arg
    assert _mixed(4, 4, 4, config=g.gemm_mixed_num_configs()) == bad_cfg
    assert _mixed(4, 4, 4, config=-2) == bad_cfg
    assert _mixed(4, 4, 4) == null
    assert _mixed(4, 4, 4, C=256) == null
    assert _mixed(4, 4, 4, A=257, B=512, C=1024) == misal   # codes need 2-byte alignment
    assert _mixed(4, 4, 4, A=256, B=513, C=1024) == misal
    assert _mixed(4, 4, 4, A=256, B=512, C=1026) == misal   # C needs 4-byte alignment
    assert _mixed(0, 4, 4) == ok
    assert _mixed(4, 0, 4) == ok
    with pytest.raises(ValueError):
        g.gemm_mixed(4, 4, 4, 0, 4, 0, 4, 0, 4, "fp8")


def test_mixed_tile_queries():
    n = g.gemm_mixed_num_configs()
    assert n >= 2
    for i in range(n):
        q = g.gemm_mixed_tile(i, 64, 64, 64)
        assert q["config"] == i and q["BK"] == 64 and q["threads"] % 64 == 0
        assert q["BM"] % 32 == 0 and q["BN"] % 32 == 0
    assert g.gemm_mixed_tile(-1, 4096, 4096, 4096)["config"] in range(n)
    with pytest.raises(g.GemmError):
        g.gemm_mixed_tile(n, 64, 64, 64)
    with pytest.raises(g.GemmError):
        g.gemm_mixed_tile(-1, 64, -1, 64)


def test_splitk_plans():
    # an under-filled product is split, four k steps deep at least
    p = g.gemm_f32_splitk_plan(1024, 1024, 4096)
    t = g.gemm_f32_tile("prod", p["config"], 1024, 1024, 4096)
    tiles = -(-1024 // t["BM"]) * -(-1024 // t["BN"])
    assert p["splits"] > 1 and p["kc"] % t["BK"] == 0 and p["kc"] >= 4 * t["BK"]
    assert tiles * p["splits"] <= 2 * 256
    assert (p["splits"] - 1) * p["kc"] < 4096 <= p["splits"] * p["kc"]
    assert p["workspace_bytes"] == p["splits"] * 1024 * 1024 * 4
    # few tiles and a long K: every CU gets a (tile, chunk) pair
    p = g.gemm_f32_splitk_plan(256, 256, 16384)
    assert p["splits"] * 4 == 256 and p["kc"] * p["splits"] == 16384
    # 1024^3: the plain entry's 64x64 tiles fill every CU, and its modelled
    # time beats the split's
    p = g.gemm_f32_splitk_plan(1024, 1024, 1024)
    assert p["splits"] == 1 and p["config"] == g.gemm_f32_tile("prod", -1, 1024, 1024, 1024)["config"]
    # a product with a tile for every CU is not split and needs no workspace
    p = g.gemm_f32_splitk_plan(4096, 4096, 4096)
    assert p["splits"] == 1 and p["workspace_bytes"] == 0
    # explicit counts are honoured up to one k step per split
    t0 = g.gemm_f32_tile("prod", 0, 1, 1, 1)
    p = g.gemm_f32_splitk_plan(300, 300, 100, 0, 64)
    assert p["splits"] == -(-100 // t0["BK"]) and p["kc"] == t0["BK"]
    p = g.gemm_f32_splitk_plan(300, 300, 1000, 0, 3)
    assert p["splits"] == 3 and p["kc"] % t0["BK"] == 0 and 2 * p["kc"] < 1000 <= 3 * p["kc"]
    p = g.gemm_f32_splitk_plan(8, 8, 0)
    assert p["splits"] == 1 and p["workspace_bytes"] == 0
    # a short k loop is left alone by the automatic plan, which then runs the
    # plain product's own entry
    p = g.gemm_f32_splitk_plan(256, 256, 256)
    assert p["splits"] == 1 and p["config"] == g.gemm_f32_tile("prod", -1, 256, 256, 256)["config"]
    p = g.gemm_f32_splitk_plan(4096, 4096, 4096)
    assert p["config"] == g.gemm_f32_tile("prod", -1, 4096, 4096, 4096)["config"]
    # small-K panel entries cannot split
    panel = g.gemm_f32_tile("prod", -1, 16384, 16384, 64)["config"]
    with pytest.raises(g.GemmError) as e:
        g.gemm_f32_splitk_plan(512, 512, 64, panel, 2)
    assert e.value.status == 7
    with pytest.raises(g.GemmError) as e:
        g.gemm_f32_splitk_plan(512, 512, 64, -1, -1)
    assert e.value.status == 8


def test_splitk_validation_codes():
    lib = g._lib
    need = g.gemm_f32_splitk_plan(1024, 1024, 4096)["workspace_bytes"]
    assert need > 0

    def call(ws, ws_bytes, A=256, B=512, C=1024, lda=4096):
        return lib.gemm_f32_splitk(1024, 1024, 4096, A, lda, B, 1024, C, 1024, -1, 0, ws,
                                   ws_bytes, None)
    assert call(None, 0) == 9
    assert call(4096, need - 4) == 9
    assert call(4098, need) == 9                    # workspace must be 4-byte aligned
    assert call(4096, need, lda=1000) == 2
    assert call(4096, need, A=None) == 3
    assert call(4096, need, C=1026) == 6
    assert lib.gemm_f32_splitk(0, 8, 8, None, 8, None, 8, None, 8, -1, 0, None, 0, None) == 0
    assert lib.gemm_f32_splitk(8, 8, 8, None, 8, None, 8, None, 8, 8, 0, None, 0, None) == 7
    assert lib.gemm_f32_splitk(8, 8, 8, None, 8, None, 8, None, 8, -1, -3, None, 0, None) == 8


def test_python_raw_wrapper_raises():
    with pytest.raises(g.GemmError) as e:
        g.gemm_f32(4, 4, 4, 0, 4, 0, 4, 0, 4, "prod")
    assert e.value.status == 3
    with pytest.raises(ValueError):
        g.gemm_f32(4, 4, 4, 0, 4, 0, 4, 0, 4, "nope")


def test_probe_validation():
    lib = g._lib
    assert lib.gemm_f32_probe_stream(7, 16, 256, 256, 256, None) == 8
    assert lib.gemm_f32_probe_stream(0, -1, 256, 256, 256, None) == 8
    assert lib.gemm_f32_probe_stream(0, 0, None, None, None, None) == 0
    assert lib.gemm_f32_probe_stream(0, 16, None, None, 256, None) == 3
    assert lib.gemm_f32_probe_stream(2, 16, 256, None, 256, None) == 3
    assert lib.gemm_f32_probe_stream(0, 16, 256 + 4, None, 256, None) == 6
    assert lib.gemm_f32_probe_mfma(0, 1, 256, None) == 8
    assert lib.gemm_f32_probe_mfma(1, 1, None, None) == 3
    assert g.gemm_f32_probe_mfma_flops(2, 3) == 2 * 4 * 3 * 8 * (2 * 32 * 32 * 2)
    assert g.gemm_f32_probe_mfma_flops(0, 3) == -1
    assert lib.gemm_f32_probe_mfma16(16, 0, 1, 256, None) == 8
    assert lib.gemm_f32_probe_mfma16(24, 1, 1, 256, None) == 8
    assert lib.gemm_f32_probe_mfma16(32, 1, 1, None, None) == 3
    assert lib.gemm_f32_probe_mfma16(32, 1, 1, 258, None) == 6
    assert g.gemm_f32_probe_mfma16_flops(16, 2, 3) == 2 * 4 * 3 * 32 * (2 * 16 * 16 * 32)
    assert g.gemm_f32_probe_mfma16_flops(32, 2, 3) == 2 * 4 * 3 * 8 * (2 * 32 * 32 * 16)
    assert g.gemm_f32_probe_mfma16_flops(8, 2, 3) == -1
    assert lib.gemm_f32_probe_valu(0, 1, 256, None) == 8
    assert lib.gemm_f32_probe_valu(1, 0, 256, None) == 8
    assert lib.gemm_f32_probe_valu(1, 1, None, None) == 3
    assert lib.gemm_f32_probe_valu(1, 1, 258, None) == 6
    assert g.gemm_f32_probe_valu_flops(2, 3) == 2 * 256 * 3 * 8 * 16 * 2
    assert g.gemm_f32_probe_valu_flops(2, 0) == -1
    assert lib.gemm_f32_probe_lds(0, 1, 256, None) == 8
    assert lib.gemm_f32_probe_lds(1, 1, None, None) == 3
    assert g.gemm_f32_probe_lds_bytes(2, 3) == 2 * 256 * 3 * 8 * 16
    # fused probe: 16 MFMAs of 2048 FLOP and one 1 KB store per wave and round
    assert g.gemm_f32_probe_fused_flops(g.FUSED_BOTH, 256, 1024) == 2 * 16384 * 16384 * 64
    assert g.gemm_f32_probe_fused_bytes(g.FUSED_BOTH, 256, 1024) == 16384 * 16384 * 4
    assert g.gemm_f32_probe_fused_flops(g.FUSED_STORE, 2, 16) == 0
    assert g.gemm_f32_probe_fused_bytes(g.FUSED_MFMA, 2, 32) == 2 * 4 * 1024
    assert g.gemm_f32_probe_fused_flops(g.FUSED_MFMA, 2, 32) == 2 * 4 * 32 * 16 * 2048
    for bad in ((3, 1, 16), (-1, 1, 16), (0, 0, 16), (0, 1, 0), (0, 1, 24)):
        assert g.gemm_f32_probe_fused_flops(*bad) == -1
        assert g.gemm_f32_probe_fused_bytes(*bad) == -1
        assert lib.gemm_f32_probe_fused(*bad, 256, 1 << 30, None, None) == 8
    need = g.gemm_f32_probe_fused_bytes(0, 1, 16)
    assert lib.gemm_f32_probe_fused(0, 1, 16, None, need, None, None) == 3
    assert lib.gemm_f32_probe_fused(0, 1, 16, 256 + 4, need, None, None) == 6
    assert lib.gemm_f32_probe_fused(0, 1, 16, 256, need, 256 + 4, None) == 6
    assert lib.gemm_f32_probe_fused(0, 1, 16, 256, need - 16, None, None) == 8


def test_tile_queries():
    assert g.gemm_f32_tile("naive", -1, 8, 8, 8) == {"BM": 4, "BN": 64, "BK": 1, "threads": 256, "config": 0}
    for name, t in (("tiled", 16), ("tiled32", 32), ("tiled4", 4), ("tiled32_pad", 32)):
        q = g.gemm_f32_tile(name, -1, 100, 100, 100)
        assert (q["BM"], q["BN"], q["BK"], q["threads"]) == (t, t, t, t * t)
    q = g.gemm_f32_tile("valu", -1, 100, 100, 100)
    assert (q["BM"], q["BN"], q["BK"], q["threads"], q["config"]) == (128, 128, 16, 256, 5)
    assert g.gemm_f32_num_configs("valu") == 6
    for i in range(g.gemm_f32_num_configs("valu")):
        q = g.gemm_f32_tile("valu", i, 9, 9, 9)
        assert q["config"] == i and q["BK"] == (8 if i < 4 else 16)
    n = g.gemm_f32_num_configs("prod")
    assert n >= 3
    strip = g.gemm_f32_tile("prod", -1, 1, 4095, 2049)["config"]
    colstrip = g.gemm_f32_tile("prod", -1, 4095, 1, 2049)["config"]
    assert colstrip != strip
    for i in range(n):
        if i in (strip, colstrip):
            continue
        q = g.gemm_f32_tile("prod", i, 64, 64, 64)
        assert q["config"] == i and q["threads"] % 64 == 0
        assert q["BM"] % 32 == 0 and q["BN"] % 32 == 0 and q["BK"] % 8 == 0
    # products of at most 32 rows run the thin-M strip kernel whole; its
    # entry reports the rows a workgroup holds and refuses a 33rd row
    for M, bm in ((1, 1), (2, 2), (3, 4), (4, 4), (5, 8), (8, 8), (9, 16), (16, 16), (17, 32),
                  (32, 32)):
        q = g.gemm_f32_tile("prod", -1, M, 77, 5)
        assert (q["config"], q["BM"], q["BN"], q["threads"]) == (strip, bm, 16, 512)
    assert g.gemm_f32_tile("prod", -1, 33, 4095, 2049)["config"] != strip
    with pytest.raises(g.GemmError) as e:
        g.gemm_f32_tile("prod", strip, 33, 64, 64)
    assert e.value.status == 7
    assert _call(33, 64, 64, A=64, B=64, C=64, variant=2, config=strip) == 7
    # products of at most 16 columns (and more than 32 rows) run the thin-N
    # kernel whole; its entry reports the columns it holds and refuses a 17th
    for N, bn in ((1, 1), (2, 2), (3, 4), (4, 4), (5, 8), (8, 8), (9, 16), (16, 16)):
        q = g.gemm_f32_tile("prod", -1, 77, N, 5)
        assert (q["config"], q["BM"], q["BN"], q["threads"]) == (colstrip, 16, bn, 512)
    assert g.gemm_f32_tile("prod", -1, 32, 16, 16)["config"] == strip
    assert g.gemm_f32_tile("prod", -1, 4095, 17, 2049)["config"] not in (strip, colstrip)
    with pytest.raises(g.GemmError) as e:
        g.gemm_f32_tile("prod", colstrip, 64, 17, 64)
    assert e.value.status == 7
    with pytest.raises(g.GemmError):
        g.gemm_f32_tile("prod", n, 64, 64, 64)
    # automatic choice for the skinny K = 64 shape is a small-K entry; such
    # entries refuse K above their BK with BAD_CONFIG, before any launch
    q = g.gemm_f32_tile("prod", -1, 16384, 16384, 64)
    assert q["BK"] == 64
    with pytest.raises(g.GemmError) as e:
        g.gemm_f32_tile("prod", q["config"], 16384, 16384, 65)
    assert e.value.status == 7
    assert _call(256, 256, 65, A=256, B=512, C=1024, variant=2, config=q["config"]) == 7
    with pytest.raises(g.GemmError):
        g.gemm_f32_tile("prod", -1, -1, 64, 64)
    assert g.gemm_f32_num_configs(17) == 0


def test_package_load_model_matches_oracle_model():
    """The package's issued-load model (used for reports) agrees with the
    oracle's implementation of the pages' counting model."""
    shapes = [(4096, 4096, 4096), (4097, 4095, 2049), (16384, 16384, 64), (5, 7, 3), (256, 256, 256)]
    for M, N, K in shapes:
        assert roofline.issued_load_elements("naive", M, N, K, {}) == model.naive_loads(M, N, K)
        for v in ("tiled", "tiled32", "tiled4", "tiled32_pad"):
            t = g.gemm_f32_tile(v, -1, M, N, K)
            assert roofline.issued_load_elements(v, M, N, K, t) == model.tiled_loads(M, N, K, t["BM"])
        t = g.gemm_f32_tile("valu", -1, M, N, K)
        assert roofline.issued_load_elements("valu", M, N, K, t) == model.blocked_loads(
            M, N, K, 128, 128, t["BK"])
        for i in range(g.gemm_f32_num_configs("prod")):
            try:
                t = g.gemm_f32_tile("prod", i, M, N, K)
            except g.GemmError as e:  # small-K entries reject K above their BK
                assert e.status == 7 and K > g.gemm_f32_tile("prod", i, 1, 1, 1)["BK"]
                continue
            assert roofline.issued_load_elements("prod", M, N, K, t) == model.blocked_loads(
                M, N, K, t["BM"], t["BN"], t["BK"])
        assert roofline.flops(M, N, K) == model.flops(M, N, K)


def test_single_hip_runtime_in_process():
    """The library binds to the HIP runtime torch already loaded (same soname);
    two runtimes in one process cannot share device allocations."""
    import torch  # noqa: F401
    with open("/proc/self/maps") as f:
        libs = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    assert len(libs) == 1, libs


def test_automatic_choice_on_measured_shapes():
    """The plain product's automatic entry on shapes where every large entry
    was timed: the choice that measured fastest (or within 0.5% of it).  A
    change to the model that moves one of these needs new measurements."""
    expected = {
        (4096, 4096, 4096): 19,    # one whole round of 256x256 tiles
        (4097, 4095, 2049): 19,    # K tail: register-staged 256x256, strips
        (16384, 16384, 64): 21,    # small-K A-resident panel
        (1024, 1024, 1024): 16,    # 64x64 tiles, K split over the waves
        (2048, 2048, 2048): 23,    # 128x128, two workgroups per CU
        (3072, 3072, 3072): 22,    # one whole round of 192x192 tiles
        (6144, 6144, 6144): 24,    # three whole rounds of 192x256 tiles
        (3072, 4096, 4096): 24,    # one whole round of 192x256 tiles
        (4608, 4608, 4608): 25,    # row cut: whole round of 256x256 + rest
        (7168, 7168, 7168): 25,
        (5632, 5632, 5632): 19,
    }
    got = {s: g.gemm_f32_tile("prod", -1, *s)["config"] for s in expected}
    assert got == expected
