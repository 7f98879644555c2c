"""The tuning cache on the CPU: a file of tuned choices loaded into the
process's table, saved back, forgotten, and named by SGEMM_TUNE_CACHE.  No GPU
work: the configuration choice is host code."""
import ctypes
import os
import subprocess
import sys

import pytest

import fp32_gemm_02_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# a shape whose built-in choice is the 64x64 tile (too few larger tiles)
SHAPE = (777, 555, 333, 333, 555, 555)
TUNED = (128, 128, 16, 2, 2)
OTHER = (1001, 999, 97, 100, 1000, 1000)
OTHER_TUNED = (256, 128, 16, 4, 2)


def _line(shape, cfg, order=None):
    keys = ["M", "N", "K", "lda", "ldb", "ldc", "bm", "bn", "bk", "wm", "wn"]
    vals = dict(zip(keys, list(shape) + list(cfg)))
    order = order or keys
    return "{" + ", ".join(f'"{k}": {vals[k]}' for k in order) + "}\n"


@pytest.fixture(autouse=True)
def _empty_table():
    g.sgemm_tune_forget()
    yield
    g.sgemm_tune_forget()


def test_default_differs_from_the_cached_choice():
    assert g.sgemm_get_config(*SHAPE).as_tuple() != TUNED
    assert g.sgemm_get_config(*OTHER).as_tuple() != OTHER_TUNED
    assert TUNED in {c.as_tuple() for c in g.configs()}
    assert OTHER_TUNED in {c.as_tuple() for c in g.configs()}


def test_load_takes_valid_lines_and_skips_the_rest(tmp_path):
    p = tmp_path / "tune.jsonl"
    keys = ["wn", "bk", "M", "ldc", "N", "bm", "K", "lda", "wm", "ldb", "bn"]
    text = (_line(SHAPE, TUNED)
            + "\n"                                                   # empty line
            + "not json at all\n"
            + _line((64, 64, 64, 64, 64, 64), (96, 96, 16, 2, 2))    # not compiled
            + _line((64, 64, 64, 32, 64, 64), TUNED)                 # lda < K
            + _line((64, 64, 64, 64, 64, 64), TUNED).replace('"wn": 2', '"wx": 2')  # key missing
            + _line(OTHER, OTHER_TUNED, order=keys).replace(", ", " ,   ")          # any order, spacing
            + '{"M": 5, ' + " " * 400 + _line((5, 6, 7, 7, 6, 6), TUNED)[1:])        # a long line
    p.write_text(text)
    assert g.sgemm_tune_cache_load(str(p)) == 3
    assert g.sgemm_get_config(*SHAPE).as_tuple() == TUNED
    assert g.sgemm_get_config(*OTHER).as_tuple() == OTHER_TUNED
    assert g.sgemm_get_config(5, 6, 7, 7, 6, 6).as_tuple() == TUNED


def test_save_forget_load_round_trip(tmp_path):
    src, dst = tmp_path / "a.jsonl", tmp_path / "b.jsonl"
    src.write_text(_line(SHAPE, TUNED) + _line(OTHER, OTHER_TUNED))
    assert g.sgemm_tune_cache_load(str(src)) == 2
    assert g.sgemm_tune_cache_save(str(dst)) == 2
    assert sorted(dst.read_text().splitlines()) == sorted(src.read_text().splitlines())
    assert not [f for f in os.listdir(tmp_path) if ".tmp." in f]
    assert g.sgemm_tune_forget() == 2
    assert g.sgemm_get_config(*SHAPE).as_tuple() != TUNED
    assert g.sgemm_tune_cache_load(str(dst)) == 2
    assert g.sgemm_get_config(*SHAPE).as_tuple() == TUNED
    # a later line of the same shape replaces the earlier choice
    src.write_text(_line(SHAPE, TUNED) + _line(SHAPE, OTHER_TUNED))
    assert g.sgemm_tune_cache_load(str(src)) == 2
    assert g.sgemm_get_config(*SHAPE).as_tuple() == OTHER_TUNED


def test_file_errors(tmp_path):
    lib = ctypes.CDLL(g.LIB_PATH)
    for f in (lib.sgemm_tune_cache_load, lib.sgemm_tune_cache_save):
        f.argtypes = [ctypes.c_char_p, ctypes.c_void_p]
        assert f(None, None) == -1
    with pytest.raises(g.SgemmError) as e:
        g.sgemm_tune_cache_load(str(tmp_path / "missing.jsonl"))
    assert e.value.status == g.SGEMM_ERR_IO
    with pytest.raises(g.SgemmError) as e:
        g.sgemm_tune_cache_save(str(tmp_path / "no_such_dir" / "x.jsonl"))
    assert e.value.status == g.SGEMM_ERR_IO
    assert "tuning cache" in g.status_string(g.SGEMM_ERR_IO)
    # an empty table saves an empty file
    assert g.sgemm_tune_cache_save(str(tmp_path / "empty.jsonl")) == 0
    assert (tmp_path / "empty.jsonl").read_text() == ""


def test_environment_loads_the_file_before_the_first_choice(tmp_path):
    p = tmp_path / "env.jsonl"
    p.write_text(_line(SHAPE, TUNED))
    code = ("import fp32_gemm_02_amd as g; "
            f"print(g.sgemm_get_config(*{SHAPE!r}).as_tuple())")
    env = dict(os.environ, SGEMM_TUNE_CACHE=str(p))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == repr(TUNED)
    # a cache path that does not exist yet is no error: the first tune creates it
    env["SGEMM_TUNE_CACHE"] = str(tmp_path / "later.jsonl")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() != repr(TUNED)
