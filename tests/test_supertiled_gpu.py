"""The super-tiled entry (init leaf + K cluster loop) against the oracle and
against the monolithic entry, on the GPU."""
import numpy as np
import pytest
import torch

import fp32_gemm_02_amd as g
import sgemm_workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _steps(K, TK):
    return max(1, -(-K // min(TK, max(K, 1))))


@pytest.mark.parametrize("M,N,K,tiles,alpha,beta", [
    (300, 270, 200, (128, 128, 64), 1.5, 0.5),      # ragged super-tiles on every axis
    (256, 256, 256, (128, 128, 128), 1.0, 1.0),     # aligned 2x2 grid, 2 K steps
    (300, 270, 200, (300, 270, 200), -1.0, 0.25),   # one super-tile, one step
    (130, 90, 77, (64, 32, 1000), 0.5, 2.0),        # TK >= K: one step per super-tile
    (100, 90, 70, (48, 40, 7), 1.0, -1.0),          # TK not a multiple of 4: scalar path
    (64, 70, 40, (64, 64, 1), 2.0, 0.5),            # one k per step: 40 steps
    (129, 65, 300, (1000, 1000, 64), 1.0, 0.0),     # tiles larger than the matrix, beta = 0
])
def test_supertiled_matches_oracle_and_monolithic(M, N, K, tiles, alpha, beta):
    cdist = "NaN" if beta == 0 else "U"
    w = wl.custom(M, N, K, alpha, beta, ("U", "U", cdist), seed=M + K, lda=K + 4,
                  ldb=N + 2, ldc=N + 6, entry="sgemm_supertiled", TM=tiles[0], TN=tiles[1],
                  TK=tiles[2])
    x = wl.make_inputs(w)
    st = gu.run(w, x)
    steps = _steps(K, tiles[2])
    gu.check_full(w, x, st, steps=steps, relaxed=True)
    mono = gu.run(w, x, entry="sgemm")
    gu.check_full(w, x, mono, relaxed=True)
    # the two entries agree elementwise within the bound: the printed one,
    # except for the 40 one-deep steps of (64, 70, 40), whose 40 roundings of
    # the running C the tolerance of shapes outside the five workloads covers
    _, bnd = gu.oracle.sgemm(M, N, K, alpha, x.A, x.B, beta, x.C, lda=w.lda, ldb=w.ldb,
                             ldc=w.ldc)
    mag = (bnd - 1e-30) / (2 * K * gu.U)
    tol = max(2 * K, K + 2 * steps + 3) * gu.U * mag + 1e-30
    d = np.abs(gu.logical_c(w, st).astype(np.float64) - gu.logical_c(w, mono))
    assert np.all(d <= tol), f"|st - mono| / tol {(d / tol).max():.3g}"
    if 2 * K >= K + 2 * steps + 3:
        assert np.all(d <= bnd)
    # on integer inputs the two entries agree bit for bit
    wi = w.integer_variant()
    xi = wl.make_inputs(wi)
    sti = gu.run(wi, xi)
    monoi = gu.run(wi, xi, entry="sgemm")
    gu.check_full(wi, xi, sti, exact=True)
    assert np.array_equal(gu.logical_c(wi, sti), gu.logical_c(wi, monoi))


def test_supertiled_zero_k_and_zero_alpha():
    for K, alpha in ((0, 1.0), (50, 0.0)):
        w = wl.custom(90, 70, K, alpha, -2.0, seed=3, lda=max(K, 1), entry="sgemm_supertiled",
                      TM=32, TN=32, TK=16)
        x = wl.make_inputs(w)
        out = gu.run(w, x)
        want = (np.float32(-2.0) * x.logical("C")).astype(np.float32)
        assert np.array_equal(gu.logical_c(w, out).view(np.int32), want.view(np.int32))
        gu.check_pads(w, x, out)


def test_trace_counts_init_and_step_launches():
    M, N, K, TM, TN, TK = 300, 270, 200, 128, 128, 64
    w = wl.custom(M, N, K, 1.0, 0.5, seed=9)
    x = wl.make_inputs(w)
    dA, dB, dC = gu.to_dev(x.A), gu.to_dev(x.B), gu.to_dev(x.C)
    g.sgemm_trace_begin(1000)
    g.sgemm_supertiled(M, N, K, 1.0, dA, K, dB, N, 0.5, dC, N, TM, TN, TK)
    ms, kinds, n = g.sgemm_trace_end()
    tiles = 3 * 3
    assert n == tiles * (1 + 4)
    assert kinds.count(g.SGEMM_KIND_INIT_LEAF) == tiles
    assert kinds.count(g.SGEMM_KIND_GEMM) == tiles * 4
    # launch order: per super-tile, the init leaf then its K steps
    assert kinds[:5] == [1, 0, 0, 0, 0]
    assert all(t > 0 for t in ms)
    torch.cuda.synchronize()
    gu.check_full(w, x, dC.cpu().numpy(), steps=4)


def test_trace_sampling_takes_every_nth_launch():
    M, N, K, TM, TN, TK = 300, 270, 200, 128, 128, 64
    w = wl.custom(M, N, K, 1.0, 0.5, seed=9)
    x = wl.make_inputs(w)
    dA, dB, dC = gu.to_dev(x.A), gu.to_dev(x.B), gu.to_dev(x.C)
    g.sgemm_trace_begin(1000, every=4)
    g.sgemm_supertiled(M, N, K, 1.0, dA, K, dB, N, 0.5, dC, N, TM, TN, TK)
    ms, kinds, n = g.sgemm_trace_end()
    # 45 launches (9 super-tiles, an init leaf and 4 steps each): 0, 4, .., 44
    launch_kinds = [g.SGEMM_KIND_INIT_LEAF if i % 5 == 0 else g.SGEMM_KIND_GEMM
                    for i in range(45)]
    assert n == 12 and kinds == launch_kinds[::4]
    assert all(t > 0 for t in ms)
    torch.cuda.synchronize()
    gu.check_full(w, x, dC.cpu().numpy(), steps=4)


@pytest.mark.timeout(1200)
def test_workload_supertiled_16384():
    """The 16384^3 workload with 4096 super-tiles (4x4 grid, 4 K steps), full
    size: every element of the super-tiled and of the monolithic result
    against the full oracle (computed in slabs of 1024 rows), and the two
    results within the bound of each other, elementwise."""
    w = wl.BY_NAME["supertiled_16384_t4096"]
    x = wl.make_inputs(w)
    st = gu.run(w, x)
    mono = gu.run(w, x, entry="sgemm")
    worst = gu.check_rows(w, x, {"sgemm_supertiled": st, "sgemm": mono}, slab=1024)
    gu.assert_well_inside(w.name, worst["sgemm_supertiled"])
    gu.assert_well_inside("monolithic_16384", worst["sgemm"])
    del x, st, mono
    # integer inputs: the two entries agree bit for bit everywhere, and equal
    # the exact result on full-width slabs around every super-tile row
    # boundary and at the last rows
    wi = w.integer_variant()
    xi = wl.make_inputs(wi)
    sti = gu.run(wi, xi)
    monoi = gu.run(wi, xi, entry="sgemm")
    assert np.array_equal(gu.logical_c(wi, sti), gu.logical_c(wi, monoi))
    slabs = [(0, 64)] + [(b - 32, 64) for b in (4096, 8192, 12288)] + [(w.M - 64, 64)]
    gu.check_rows(wi, xi, {"sgemm_supertiled": sti}, exact=True, row_slabs=slabs)
