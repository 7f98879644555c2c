"""Brute force over small shapes and shapes one off a tile edge, on the GPU.

Every case uses integer inputs in -3..3 with alpha = 1.5 and beta = 0.5: every
partial sum is an integer far below 2^24 and the scalars add at most two
fractional bits, so any correct order of summation gives the oracle's exact
result, and the comparison is bit for bit.  (With random fractions the fp32
bound itself can be exceeded legitimately at K of 1 or 2.)  The pads of A and
B hold NaN and those of C a sentinel, so a read or write outside the logical
matrices shows up too.  Leading dimensions alternate between 16-byte aligned
ones (direct LDS loads) and odd ones (scalar loads)."""
import contextlib

import pytest

import fp32_gemm_02_amd as g
import sgemm_workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def _forced(cfg):
    g.sgemm_set_config(cfg)
    try:
        yield
    finally:
        g.sgemm_set_config(None)


def _run_all(cases, tag):
    for i, (M, N, K) in enumerate(cases):
        if i % 2 == 0:
            lda, ldb, ldc = -(-K // 4) * 4 + 4, -(-N // 4) * 4, -(-N // 4) * 4 + 8
        else:
            lda, ldb, ldc = K + 1 + (K % 2), N + 2 + (N % 2), N + 1 + (N % 2)
        w = wl.custom(M, N, K, 1.5, 0.5, ("I7", "I7", "I7"), seed=1000 + i, lda=lda, ldb=ldb,
                      ldc=ldc, name=f"{tag}_{M}x{N}x{K}")
        x = wl.make_inputs(w)
        gu.check_full(w, x, gu.run(w, x), exact=True)


def _cfg_id(c):
    return "%dx%dx%d_w%dx%d" % c.as_tuple()


def _all_cfgs():
    try:
        return g.configs()
    except Exception:   # library not built: the other tests fail loudly
        return []


def test_brute_force_default_tile():
    """The full set for the tile large shapes use (256x256x32 on 8 waves):
    M, N in 1..9, BM-1..BM+1, 2BM+-1 and K in 1..9, BK-1..BK+1, 2BK-1..2BK+1.
    K = BK and 2BK are whole chunks: with a tile inside N every chunk,
    the last one included, takes the direct loads."""
    cfg = g.sgemm_config(256, 256, 32, 4, 2)
    bm, bn, bk = cfg.bm, cfg.bn, cfg.bk
    ms = list(range(1, 10)) + [bm - 1, bm, bm + 1, 2 * bm - 1, 2 * bm + 1]
    ns = list(range(1, 10)) + [bn - 1, bn, bn + 1, 2 * bn - 1, 2 * bn + 1]
    ks = list(range(1, 10)) + [bk - 1, bk, bk + 1, 2 * bk - 1, 2 * bk, 2 * bk + 1]
    cases = [(M, N, K) for M in ms for N in ns for K in ks]
    print(f"brute force {_cfg_id(cfg)}: {len(cases)} shapes", flush=True)
    with _forced(cfg):
        _run_all(cases, _cfg_id(cfg))


@pytest.mark.parametrize("cfg", _all_cfgs(), ids=_cfg_id)
def test_brute_force_every_tile(cfg):
    """A smaller cross product for each compiled tile (K = BK and 2BK end on
    whole chunks, which a tile inside N loads directly to the end)."""
    bm, bn, bk = cfg.bm, cfg.bn, cfg.bk
    ms = [1, 2, 5, 9, bm - 1, bm + 1]
    ns = [1, 3, 8, bn - 1, bn + 1]
    ks = [1, 2, 7, bk - 1, bk, bk + 1, 2 * bk, 2 * bk + 1]
    cases = [(M, N, K) for M in ms for N in ns for K in ks]
    print(f"brute force {_cfg_id(cfg)}: {len(cases)} shapes", flush=True)
    with _forced(cfg):
        _run_all(cases, _cfg_id(cfg))


def _splitk_cfgs():
    return [c for c in _all_cfgs() if 32 * c.wm > c.bm or 32 * c.wn > c.bn]


@pytest.mark.parametrize("cfg", _splitk_cfgs(), ids=_cfg_id)
def test_brute_force_split_k(cfg):
    """The split-K entries (waves of one workgroup sharing a 32x32 or 64x64
    tile, each taking every KS-th chunk of K): K from one chunk to several
    chunks per wave, with a K tail, on tiles inside and at the edges of C."""
    bk, ks, t = cfg.bk, cfg.wm * cfg.wn, cfg.bm
    ms = [1, t - 1, t, t + 1, 100]
    ns = [1, t - 1, t, t + 1, 100]
    kss = [1, bk, ks * bk - 1, ks * bk, 2 * ks * bk + 7, 1000]
    cases = [(M, N, K) for M in ms for N in ns for K in kss]
    print(f"brute force {_cfg_id(cfg)}: {len(cases)} shapes", flush=True)
    with _forced(cfg):
        _run_all(cases, _cfg_id(cfg))
