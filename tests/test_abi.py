"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and checks its arguments before any HIP call (no GPU work is started here)."""
import ctypes
import os
import re
import threading

import pytest

import fp32_gemm_02_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "phobos_sgemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*((?:sgemm|flash_attention)\w*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("sgemm", "sgemm_supertiled", "sgemm_init_leaf", "sgemm_tune", "sgemm_tc",
                 "sgemm_supertiled_host", "sgemm_plan_supertiles", "flash_attention",
                 "flash_attention_supertiled",
                 "sgemm_tune_candidates", "sgemm_set_config", "sgemm_get_config",
                 "sgemm_config_count", "sgemm_config_at", "sgemm_trace_begin",
                 "sgemm_trace_end", "sgemm_status_string", "sgemm_version",
                 "sgemm_tune_cache_load", "sgemm_tune_cache_save", "sgemm_tune_forget"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(g.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and the binding carries a prototype for each
    assert set(declared_functions()) == set(g._SIGNATURES)


def test_version():
    assert g.version() == 1


NULL = None


@pytest.mark.parametrize("args,want", [
    ((-1, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4), -1),
    ((4, -1, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4), -2),
    ((4, 4, -1, 1.0, 8, 4, 8, 4, 0.0, 8, 4), -3),
    ((4, 4, 5, 1.0, 8, 4, 8, 4, 0.0, 8, 4), -6),     # lda < K
    ((4, 4, 0, 1.0, 8, 0, 8, 4, 0.0, 8, 4), -6),     # lda < 1
    ((4, 6, 4, 1.0, 8, 4, 8, 5, 0.0, 8, 6), -8),     # ldb < N
    ((4, 6, 4, 1.0, 8, 4, 8, 6, 0.0, 8, 5), -11),    # ldc < N
    ((4, 4, 4, 1.0, NULL, 4, 8, 4, 0.0, 8, 4), -5),  # A read but NULL
    ((4, 4, 4, 1.0, 8, 4, NULL, 4, 0.0, 8, 4), -7),  # B read but NULL
    ((4, 4, 4, 1.0, 8, 4, 8, 4, 0.0, NULL, 4), -10),  # C NULL
    ((0, 4, 4, 1.0, NULL, 4, NULL, 4, 0.0, NULL, 4), 0),  # M == 0: no-op
    ((4, 0, 4, 1.0, NULL, 4, NULL, 1, 0.0, NULL, 1), 0),  # N == 0: no-op
    ((1 << 31, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4), g.SGEMM_ERR_TOO_LARGE),
])
def test_sgemm_argument_checks(args, want):
    assert g.sgemm_raw(*args, stream=0) == want


@pytest.mark.parametrize("tiles,want", [((0, 4, 4), -12), ((4, 0, 4), -13), ((4, 4, 0), -14),
                                        ((-3, 4, 4), -12)])
def test_supertiled_argument_checks(tiles, want):
    assert g.sgemm_supertiled_raw(4, 4, 4, 1.0, 8, 4, 8, 4, 1.0, 8, 4, *tiles, stream=0) == want
    # the GEMM arguments are checked first, with the same numbering as sgemm
    assert g.sgemm_supertiled_raw(4, 4, 4, 1.0, 8, 3, 8, 4, 1.0, 8, 4, *tiles, stream=0) == -6


def test_init_leaf_argument_checks():
    lib = g.lib()
    assert lib.sgemm_init_leaf(-1, 4, 1.0, 8, 4, None) == -1
    assert lib.sgemm_init_leaf(4, -1, 1.0, 8, 4, None) == -2
    assert lib.sgemm_init_leaf(4, 4, 1.0, None, 4, None) == -4
    assert lib.sgemm_init_leaf(4, 4, 1.0, 8, 3, None) == -5
    assert lib.sgemm_init_leaf(0, 4, 0.0, None, 4, None) == 0


def test_status_strings():
    assert g.status_string(0) == "success"
    assert g.status_string(-6) == "argument 6 is invalid"
    assert "no compiled kernel" in g.status_string(g.SGEMM_ERR_NO_CONFIG)
    assert g.status_string(g.SGEMM_ERR_HIP_BASE + 1)  # HIP's own text
    assert g.status_string(500) == "unknown status"


def test_config_table_and_forcing():
    cfgs = g.configs()
    assert len(cfgs) >= 4
    for c in cfgs:
        if 32 * c.wm > c.bm or 32 * c.wn > c.bn:
            # a split-K entry: a wave grid larger than the tile's 32x32 blocks
            assert c.bm == c.bn and c.bm in (32, 64)
            assert c.wm * c.wn in (4, 8) and c.bk in (16, 32)
            continue
        # each tile is whole 32x32 MFMA blocks per wave, B reads 1 to 4 wide
        assert c.bm % (32 * c.wm) == 0 and c.bn % (32 * c.wn) == 0
        assert (c.bn // c.wn // 32) in (1, 2, 3, 4)
        assert c.bk % 8 == 0
    lib = g.lib()
    assert lib.sgemm_config_at(-1, ctypes.byref(g.sgemm_config())) == -1
    assert lib.sgemm_config_at(len(cfgs), ctypes.byref(g.sgemm_config())) == -1
    try:
        for c in cfgs:
            g.sgemm_set_config(c)
            assert g.sgemm_get_config(4096, 4096, 4096, 4096, 4096, 4096).as_tuple() == c.as_tuple()
        with pytest.raises(g.SgemmError) as e:
            g.sgemm_set_config((48, 48, 16, 1, 1))
        assert e.value.status == g.SGEMM_ERR_NO_CONFIG
    finally:
        g.sgemm_set_config(None)


def test_get_config_checks():
    lib = g.lib()
    out = g.sgemm_config()
    assert lib.sgemm_get_config(-1, 4, 4, 4, 4, 4, ctypes.byref(out)) == -1
    assert lib.sgemm_get_config(4, 4, 8, 4, 4, 4, ctypes.byref(out)) == -4
    assert lib.sgemm_get_config(4, 8, 4, 4, 4, 8, ctypes.byref(out)) == -5
    assert lib.sgemm_get_config(4, 8, 4, 4, 8, 4, ctypes.byref(out)) == -6
    assert lib.sgemm_get_config(4, 4, 4, 4, 4, 4, None) == -7


@pytest.mark.parametrize("shape,want", [
    # small products: 32x32 tiles, their K split over the waves of a
    # workgroup: eight waves for at most 512 tiles or K of 16384 and more ...
    ((512, 512, 512), (32, 32, 32, 4, 2)),
    ((128, 128, 16384), (32, 32, 32, 4, 2)),
    ((960, 960, 16384), (32, 32, 32, 4, 2)),
    # ... four waves of 16-deep chunks up to 2560 tiles ...
    ((256, 256, 256), (32, 32, 16, 2, 2)),
    ((768, 768, 256), (32, 32, 16, 2, 2)),
    ((960, 960, 960), (32, 32, 16, 2, 2)),
    ((1024, 1024, 1024), (32, 32, 16, 2, 2)),
    ((1536, 1536, 1536), (32, 32, 16, 2, 2)),
    ((8192, 128, 2048), (32, 32, 16, 2, 2)),
    # ... and one wave per tile with short K beyond 576 tiles, with 2048
    # tiles (two per SIMD) and K below 4096, with K below 64, or beyond
    # 2560 tiles
    ((1024, 1024, 256), (32, 32, 32, 1, 1)),
    ((1024, 2048, 1024), (32, 32, 32, 1, 1)),
    ((1024, 2048, 4096), (32, 32, 16, 2, 2)),
    ((256, 256, 40), (32, 32, 32, 1, 1)),
    # ... 16 deep when K fits one such chunk, or when a CU holds more than 9
    ((200, 200, 8), (32, 32, 16, 1, 1)),
    ((200, 200, 16), (32, 32, 16, 1, 1)),
    ((1664, 1664, 1664), (32, 32, 16, 1, 1)),
    # beyond 2560 such tiles, from K = 2048 on, the estimate weighs split-K
    # (four waves over a 32x32 tile, rate 0.79, or over a 64x64 one, 0.85)
    # against the other tiles
    ((2304, 2304, 2304), (32, 32, 16, 2, 2)),
    ((3072, 3072, 3072), (64, 64, 16, 4, 1)),
    ((3584, 3584, 3584), (64, 64, 16, 4, 1)),
    ((3072, 3072, 8192), (64, 64, 16, 4, 1)),
    ((2560, 2560, 2560), (32, 32, 16, 2, 2)),
    ((1792, 1792, 8192), (32, 32, 16, 2, 2)),
    # one 128x128 tile per CU beats 13 small ones per CU, and 576 tiles of
    # 256x256 (2.25 rounds of 256 CUs) lose to 2304 of 128x128 (9 rounds)
    ((7168, 7168, 7168), (128, 128, 32, 2, 2)),
    ((13312, 4096, 4096), (128, 128, 32, 2, 2)),
    ((10240, 10240, 4096), (128, 128, 32, 2, 2)),
    ((1792, 1792, 1792), (128, 128, 32, 2, 2)),
    ((2048, 2048, 2048), (128, 128, 32, 2, 2)),
    ((6144, 6144, 6144), (128, 128, 32, 2, 2)),
    ((8192, 512, 4096), (128, 128, 32, 2, 2)),
    # 100 tiles of 256x256 against 200 of 256x128 on 8 waves; with short K
    # two resident 256x128 tiles per CU hide each other's fixed cost
    ((2560, 2560, 1024), (256, 128, 16, 4, 2)),
    ((8192, 8192, 1024), (256, 128, 16, 4, 2)),
    # 16 x 16 tiles of 320x192 (exactly 256 workgroups) where the leading
    # dimensions are multiples of 4, K whole 16-deep chunks or not ...
    ((5120, 3072, 4096), (320, 192, 16, 2, 2)),
    ((2500, 6000, 6000), (320, 192, 16, 2, 2)),
    ((7680, 7680, 7680), (320, 192, 16, 2, 2)),
    ((5120, 3072, 4095, 4096, 3072, 3072), (320, 192, 16, 2, 2)),
    # ... and not where they are not (every chunk through registers), nor
    # where the rows of A are not 64-byte aligned (lda not a multiple of 16)
    ((5120, 3072, 4095), (256, 256, 32, 4, 2)),
    ((7680, 7680, 7681, 7696, 7680, 7680), (320, 192, 16, 2, 2)),
    ((7680, 7680, 7681, 7684, 7680, 7680), (128, 128, 32, 2, 2)),
    ((4800, 2900, 8000, 8004, 2900, 2900), (256, 256, 32, 4, 2)),
    # 286 of them (two rounds of 256 CUs) lose to 256 of 256x256
    ((4095, 4095, 4095, 4096, 4096, 4096), (256, 256, 32, 4, 2)),
    # the five workloads' shapes (with their leading dimensions) and the
    # super-tiled step leaf
    ((4096, 4096, 4096), (256, 256, 32, 4, 2)),
    ((65536, 512, 4096), (256, 256, 32, 4, 2)),
    ((5003, 3001, 2047, 2048, 3008, 3008), (320, 192, 16, 2, 2)),
    ((4096, 4096, 4096, 16384, 16384, 16384), (256, 256, 32, 4, 2)),
    ((16384, 16384, 16384), (256, 256, 32, 4, 2)),
    # the unaligned shape with unpadded rows
    ((5003, 3001, 2047), (256, 128, 16, 4, 2)),
])
def test_default_config_picks(shape, want):
    """The built-in choice at the boundaries of its rule, fixed on the CPU
    (leading dimensions K, N, N unless given)."""
    M, N, K = shape[:3]
    lds = shape[3:] if len(shape) > 3 else (K, N, N)
    assert g.sgemm_get_config(M, N, K, *lds).as_tuple() == want


def test_default_config_needs_direct_loads_for_the_320x192_tile():
    """With leading dimensions that are not multiples of 4 every chunk comes
    through registers, and the 320x192 tile is not taken."""
    assert g.sgemm_get_config(5120, 3072, 4096, 4096, 3072, 3072).as_tuple() == (320, 192, 16, 2, 2)
    for lds in [(4097, 3072, 3072), (4096, 3073, 3072), (4096, 3072, 3075)]:
        assert g.sgemm_get_config(5120, 3072, 4096, *lds).as_tuple() == (256, 256, 32, 4, 2)


def test_default_config_fits_the_shape():
    names = {c.as_tuple() for c in g.configs()}
    for shape in [(1, 1, 1), (31, 17, 5), (256, 256, 256), (4096, 4096, 4096),
                  (65536, 512, 4096), (5003, 3001, 2047)]:
        M, N, K = shape
        c = g.sgemm_get_config(M, N, K, K, N, N)
        assert c.as_tuple() in names
        # a small problem never gets a tile much larger than itself
        assert c.bm <= max(64, 2 * M) and c.bn <= max(64, 2 * N)


def _pow2_between(v, lo, hi):
    return lo <= v <= hi and (v & (v - 1)) == 0


def test_tune_candidates_follow_the_autotune_ranges():
    all_cfgs = g.configs()
    cands = g.sgemm_tune_candidates(4096, 4096, 4096)
    assert len(cands) >= 4
    for c in cands:
        assert _pow2_between(c.bm, 32, 256) and _pow2_between(c.bn, 32, 256)
        assert _pow2_between(c.bk, 4, 32)
    # a small problem prunes tiles larger than it needs
    small = g.sgemm_tune_candidates(40, 70, 100)
    assert small and all(c.bm <= 64 and c.bn <= 96 for c in small)
    assert len(small) < len(all_cfgs)
    tiny = g.sgemm_tune_candidates(1, 1, 1)
    assert [c.as_tuple() for c in tiny] == [(32, 32, 16, 1, 1), (32, 32, 32, 1, 1)]


def test_tune_candidates_and_tune_argument_checks():
    lib = g.lib()
    assert lib.sgemm_tune_candidates(-1, 4, 4, None, 0) == -1
    assert lib.sgemm_tune_candidates(4, 4, 4, None, 3) == -4
    assert lib.sgemm_tune_candidates(4, 4, 4, None, -1) == -5
    assert lib.sgemm_tune_candidates(4, 4, 4, None, 0) > 0   # count only
    assert lib.sgemm_tune(0, 4, 4, 4, 4, 4, 5, None, None, None) == -1
    assert lib.sgemm_tune(4, 4, 4, 3, 4, 4, 5, None, None, None) == -4
    assert lib.sgemm_tune(4, 4, 4, 4, 4, 4, 0, None, None, None) == -7


def test_trace_argument_checks():
    lib = g.lib()
    assert lib.sgemm_trace_begin(0) == -1
    assert lib.sgemm_trace_begin(4) == 0
    n = ctypes.c_int64(-1)
    assert lib.sgemm_trace_end(None, None, 0, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.sgemm_trace_end(None, None, -1, None) == -3
    assert lib.sgemm_trace_begin_sampled(0, 1) == -1
    assert lib.sgemm_trace_begin_sampled(4, 0) == -2
    assert lib.sgemm_trace_begin_sampled(4, 7) == 0
    assert lib.sgemm_trace_end(None, None, 0, ctypes.byref(n)) == 0
    assert n.value == 0


@pytest.mark.parametrize("args,want", [
    ((-1, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4, 1), -1),
    ((4, 4, 5, 1.0, 8, 4, 8, 4, 0.0, 8, 4, 1), -6),      # lda < K
    ((4, 4, 4, 1.0, NULL, 4, 8, 4, 0.0, 8, 4, 1), -5),   # A read but NULL
    ((4, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4, 0), -12),     # unknown format
    ((4, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4, 3), -12),
    ((0, 4, 4, 1.0, NULL, 4, NULL, 4, 0.0, NULL, 4, 2), 0),   # M == 0: no-op
    ((1 << 31, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4, 2), g.SGEMM_ERR_TOO_LARGE),
])
def test_tc_argument_checks(args, want):
    assert g.sgemm_tc_raw(*args, stream=0) == want


@pytest.mark.parametrize("shape,want", [
    # at least 144 tiles of 256x256 and K >= 1024: staged on 256x256x64
    ((3072, 3072, 1024), (256, 256, 64, 4, 2, 1)),
    ((16384, 16384, 16384), (256, 256, 64, 4, 2, 1)),
    ((5003, 3001, 2047), (256, 256, 64, 4, 2, 1)),
    # fewer, K > 2048 and at least 16 tiles of 128x128: staged on 128x128x64
    ((2560, 2560, 2560), (128, 128, 64, 2, 2, 1)),
    ((2048, 2048, 4096), (128, 128, 64, 2, 2, 1)),
    ((512, 512, 4096), (128, 128, 64, 2, 2, 1)),
    # fewer, K <= 2048 and at least 64 tiles of 128x128: fused on 128x128x64
    ((2048, 2048, 2048), (128, 128, 64, 2, 2, 0)),
    ((2048, 2048, 1024), (128, 128, 64, 2, 2, 0)),
    ((1024, 1024, 1024), (128, 128, 64, 2, 2, 0)),
    # otherwise the fused order of before
    ((768, 768, 768), (64, 64, 32, 1, 1, 0)),
    ((4096, 4096, 512), (256, 256, 32, 2, 2, 0)),
    ((256, 256, 65536), (64, 64, 32, 1, 1, 0)),
])
def test_tc_default_config_picks(shape, want):
    """The matrix-core variant's built-in choice at the boundaries of its
    rule, both formats, fixed on the CPU."""
    for fmt in (g.SGEMM_TC_F16, g.SGEMM_TC_BF16):
        assert g.sgemm_tc_get_config(fmt, *shape).as_tuple() == want


def test_tc_configs():
    for fmt in (g.SGEMM_TC_F16, g.SGEMM_TC_BF16):
        cfgs = g.tc_configs(fmt)
        assert len(cfgs) >= 8
        assert any(c.staged for c in cfgs) and any(not c.staged for c in cfgs)
        assert all(c.bk in (32, 64) and c.bm % (32 * c.wm) == 0 and c.bn % (32 * c.wn) == 0
                   for c in cfgs)
        # staged tiles divide the 256 x 256 x 64 padding of the workspace
        assert all(256 % c.bm == 0 and 256 % c.bn == 0 and 64 % c.bk == 0
                   for c in cfgs if c.staged)
        # large products take the staged form, small ones a small fused tile
        big = g.sgemm_tc_get_config(fmt, 16384, 16384, 16384)
        assert big.staged == 1 and (big.bm, big.bn) == (256, 256)
        small = g.sgemm_tc_get_config(fmt, 64, 64, 64)
        assert small.staged == 0 and (small.bm, small.bn) == (64, 64)
        g.sgemm_tc_set_config(fmt, cfgs[0])
        assert g.sgemm_tc_get_config(fmt, 16384, 16384, 16384).as_tuple() == cfgs[0].as_tuple()
        g.sgemm_tc_set_config(fmt, None)
        with pytest.raises(RuntimeError):
            g.sgemm_tc_set_config(fmt, (48, 48, 32, 1, 1, 0))
    lib = g.lib()
    assert lib.sgemm_tc_config_count(0) == -1
    assert lib.sgemm_tc_config_at(1, 999, None) == -2
    assert lib.sgemm_tc_get_config(7, 4, 4, 4, None) == -1


@pytest.mark.parametrize("args,want", [
    ((-1, 4, 64, 8, 64, 8, 64, 8, 64, 8, 64, 0.1), -1),
    ((4, 0, 64, 8, 64, 8, 64, 8, 64, 8, 64, 0.1), -2),     # no keys
    ((4, 4, 32, 8, 64, 8, 64, 8, 64, 8, 64, 0.1), -3),     # only D = 64
    ((4, 4, 64, 8, 63, 8, 64, 8, 64, 8, 64, 0.1), -5),     # ldq < D
    ((4, 4, 64, 8, 64, 8, 60, 8, 64, 8, 64, 0.1), -7),
    ((4, 4, 64, 8, 64, 8, 64, 8, 1, 8, 64, 0.1), -9),
    ((4, 4, 64, 8, 64, 8, 64, 8, 64, 8, 0, 0.1), -11),
    ((4, 4, 64, NULL, 64, 8, 64, 8, 64, 8, 64, 0.1), -4),
    ((4, 4, 64, 8, 64, NULL, 64, 8, 64, 8, 64, 0.1), -6),
    ((4, 4, 64, 8, 64, 8, 64, NULL, 64, 8, 64, 0.1), -8),
    ((4, 4, 64, 8, 64, 8, 64, 8, 64, NULL, 64, 0.1), -10),
    ((0, 4, 64, NULL, 64, NULL, 64, NULL, 64, NULL, 64, 0.1), 0),   # Nq == 0: nothing
    ((1 << 31, 4, 64, 8, 64, 8, 64, 8, 64, 8, 64, 0.1), g.SGEMM_ERR_TOO_LARGE),
])
def test_attention_argument_checks(args, want):
    assert g.flash_attention_raw(*args, stream=0) == want
    assert g.flash_attention_supertiled_raw(*args, 1024, stream=0) == want


def test_attention_supertile_rows_checked():
    assert g.flash_attention_supertiled_raw(4, 4, 64, 8, 64, 8, 64, 8, 64, 8, 64, 0.1, 0,
                                            stream=0) == -13


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No CPU fallback: without the built library every entry point raises."""
    monkeypatch.setattr(g, "LIB_PATH", str(tmp_path / "libphobos_sgemm.so"))
    monkeypatch.setattr(g, "_lib", None)
    for call in (lambda: g.sgemm(4, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, stream=0),
                 lambda: g.sgemm_supertiled(4, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, 2, 2, 2,
                                            stream=0),
                 lambda: g.flash_attention(4, 4, 64, 0, 64, 0, 64, 0, 64, 0, 64, 1.0, stream=0),
                 lambda: g.sgemm_tc(4, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, stream=0),
                 g.version):
        with pytest.raises(RuntimeError, match="not built"):
            call()


@pytest.mark.parametrize("args,want", [
    ((-1, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4, 1), -1),
    ((4, 4, 5, 1.0, 8, 4, 8, 4, 0.0, 8, 4, 1), -6),
    ((4, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4, 5), -12),
    ((0, 4, 4, 1.0, NULL, 4, NULL, 4, 0.0, NULL, 4, 2), 0),        # empty: nothing
    ((4, 4, 0, 1.0, NULL, 4, NULL, 4, 1.0, 8, 4, 1), 0),           # K = 0, beta = 1: nothing
    # workspaces past the static 64 MiB are refused before any HIP call
    ((8192, 8192, 8192, 1.0, 8, 8192, 8, 8192, 0.0, 8, 8192, 1), g.SGEMM_ERR_SCRATCH),
    ((4097, 4096, 4096, 1.0, 8, 4096, 8, 4096, 0.0, 8, 4096, 2), g.SGEMM_ERR_SCRATCH),
    ((1 << 31, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4, 2), g.SGEMM_ERR_TOO_LARGE),
])
def test_tc_noalloc_argument_checks(args, want):
    assert g.sgemm_tc_noalloc_raw(*args, stream=0) == want
    assert "static scratch" in g.status_string(g.SGEMM_ERR_SCRATCH)


def test_host_entry_points_from_many_threads():
    """The host-only entry points called from eight threads at once (ctypes
    drops the GIL for the call): the built-in tile choice, the tuned table's
    reset, the planner and the status strings give each thread what one
    thread alone gets, and nothing crashes."""
    shapes = [((37 * i) % 9000 + 1, (91 * i) % 7000 + 1, (53 * i) % 20000 + 1) for i in range(300)]
    want = [g.sgemm_get_config(M, N, K, K, N, N).as_tuple() for M, N, K in shapes]
    plan_want = g.sgemm_plan_supertiles(4096, 4096, 4096, 1.0, 256 << 20)
    plan_key = (plan_want.TM, plan_want.TN, plan_want.TK, plan_want.walk)
    errors = []

    def work(t):
        try:
            for j in range(len(shapes)):
                i = (t * 41 + j) % len(shapes)
                M, N, K = shapes[i]
                got = g.sgemm_get_config(M, N, K, K, N, N).as_tuple()
                if got != want[i]:
                    errors.append(("config", t, shapes[i], got, want[i]))
                if j % 60 == 0:
                    g.sgemm_tune_forget()
                    p = g.sgemm_plan_supertiles(4096, 4096, 4096, 1.0, 256 << 20)
                    if (p.TM, p.TN, p.TK, p.walk) != plan_key:
                        errors.append(("plan", t))
                if g.status_string(-(j % 12 + 1)) != "argument %d is invalid" % (j % 12 + 1):
                    errors.append(("status", t, j))
        except Exception as e:   # reported below, with the thread's number
            errors.append(("exception", t, repr(e)))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors[:5]
