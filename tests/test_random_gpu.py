"""Seeded random cases on the GPU: shapes, padded or odd leading dimensions,
scalars (0 included), forced tiles, the super-tiled walk with random
extents, the 16-bit variant in every form and attention with random sizes
and super-tile heights.  Integer inputs are compared bit for bit with the
oracle; fractional ones within the bound.  Every case is a valid call."""
import numpy as np
import pytest

import fp32_gemm_02_amd as g
import oracle
import sgemm_workloads as wl
from tests import gpu_util as gu
from tests.test_attention_gpu import check_attn, run_attn

pytestmark = pytest.mark.gpu


def _pad(rng, x):
    return x + int(rng.choice([0, 0, 1, 3, 4, 8, 17]))


@pytest.mark.parametrize("seed", [1, 2])
def test_random_sgemm_and_supertiled(seed):
    rng = np.random.default_rng(seed)
    cfgs = [None] + [c.as_tuple() for c in g.configs()]
    for i in range(150):
        M, N, K = (int(rng.integers(1, 700)) for _ in range(3))
        lda, ldb, ldc = _pad(rng, K), _pad(rng, N), _pad(rng, N)
        alpha = float(rng.choice([1.0, -1.0, 0.5, 1.5, 0.0, 2.0]))
        beta = float(rng.choice([0.0, 1.0, 0.5, -0.25, 2.0]))
        integer = bool(rng.integers(0, 2))
        supertiled = rng.integers(0, 3) == 0
        tiles = tuple(int(rng.integers(1, 400)) for _ in range(3)) if supertiled else (None,) * 3
        cfg = cfgs[int(rng.integers(0, len(cfgs)))]
        c = "NaN" if beta == 0 else ("I7" if integer else "U")
        dists = ("I7", "I7", c) if integer else ("U", "U", c)
        w = wl.custom(M, N, K, alpha, beta, dists, seed=1000 * seed + i, lda=lda, ldb=ldb,
                      ldc=ldc, entry="sgemm_supertiled" if supertiled else "sgemm",
                      TM=tiles[0], TN=tiles[1], TK=tiles[2], name=f"random{seed}_{i}")
        print(f"case {i}: {w.entry} {M}x{N}x{K} ld {lda},{ldb},{ldc} alpha {alpha} beta {beta} "
              f"tiles {tiles} cfg {cfg}", flush=True)
        g.sgemm_set_config(cfg)
        try:
            x = wl.make_inputs(w)
            out = gu.run(w, x)
        finally:
            g.sgemm_set_config(None)
        steps = -(-K // min(tiles[2], K)) if supertiled and K > 0 and alpha != 0 else 1
        gu.check_full(w, x, out, steps=steps, exact=integer, relaxed=not integer)


def test_random_whole_tiles_with_c_prefetch():
    """Shapes where the 8-wave 256x256 tiles take their C prefetch: beta != 0,
    16-byte aligned operands, K a whole number of chunks, so every tile wholly
    inside C loads 12 (BK = 32) or all 16 (BK = 16) of its lanes' rows of a
    32-row block of C into LDS during the last chunk.  Edge tiles of the same
    launches take the plain epilogue beside them.  The super-tiled walk runs
    the same leaves with beta = 1 on its step launches."""
    rng = np.random.default_rng(5)
    for i in range(40):
        cfg = [(256, 256, 32, 4, 2), (256, 256, 16, 4, 2)][i % 2]
        bk = cfg[2]
        M, N = (int(rng.integers(256, 1100)) for _ in range(2))
        K = bk * int(rng.integers(1, 48))
        lda, ldb, ldc = (-(-v // 4) * 4 + 4 * int(rng.choice([0, 0, 1, 5])) for v in (K, N, N))
        alpha = float(rng.choice([1.0, -1.0, 0.5, 1.5]))
        beta = float(rng.choice([1.0, 0.5, -0.25, 2.0]))
        integer = bool(rng.integers(0, 2))
        supertiled = rng.integers(0, 3) == 0
        tiles = ((int(rng.integers(256, 700)), int(rng.integers(256, 700)),
                  bk * int(rng.integers(1, 20))) if supertiled else (None,) * 3)
        c = "I7" if integer else "U"
        w = wl.custom(M, N, K, alpha, beta, (c, c, c), seed=9000 + i, lda=lda, ldb=ldb, ldc=ldc,
                      entry="sgemm_supertiled" if supertiled else "sgemm", TM=tiles[0],
                      TN=tiles[1], TK=tiles[2], name=f"random_cpf_{i}")
        print(f"case {i}: {w.entry} {M}x{N}x{K} ld {lda},{ldb},{ldc} alpha {alpha} beta {beta} "
              f"tiles {tiles} cfg {cfg}", flush=True)
        g.sgemm_set_config(cfg)
        try:
            x = wl.make_inputs(w)
            out = gu.run(w, x)
        finally:
            g.sgemm_set_config(None)
        steps = -(-K // min(tiles[2], K)) if supertiled else 1
        gu.check_full(w, x, out, steps=steps, exact=integer, relaxed=not integer)


def test_random_matrix_core_variant():
    rng = np.random.default_rng(3)
    for i in range(60):
        fmt = int(rng.choice([g.SGEMM_TC_F16, g.SGEMM_TC_BF16]))
        forms = [None] + [c.as_tuple() for c in g.tc_configs(fmt)]
        form = forms[int(rng.integers(0, len(forms)))]
        M, N, K = (int(rng.integers(1, 600)) for _ in range(3))
        lda, ldb, ldc = _pad(rng, K), _pad(rng, N), _pad(rng, N)
        alpha = float(rng.choice([1.0, -0.5, 0.0, 2.0]))
        beta = float(rng.choice([0.0, 1.0, 0.5]))
        integer = bool(rng.integers(0, 2))
        c = "NaN" if beta == 0 else ("I7" if integer else "U")
        w = wl.custom(M, N, K, alpha, beta, ("I7", "I7", c) if integer else ("U", "U", c),
                      seed=5000 + i, lda=lda, ldb=ldb, ldc=ldc, name=f"random_tc_{i}")
        print(f"case {i}: fmt {fmt} form {form} {M}x{N}x{K} ld {lda},{ldb},{ldc} alpha {alpha} "
              f"beta {beta}", flush=True)
        g.sgemm_tc_set_config(fmt, form)
        try:
            x = wl.make_inputs(w)
            out = gu.run(w, x, fmt=fmt)
        finally:
            g.sgemm_tc_set_config(fmt, None)
        gu.check_full(w, x, out, exact=integer, relaxed=not integer, fmt=fmt)


def test_random_attention():
    rng = np.random.default_rng(4)
    for i in range(40):
        Nq, Nk = int(rng.integers(1, 700)), int(rng.integers(1, 900))
        ldq, ldk, ldv, ldo = (64 + int(rng.choice([0, 0, 1, 4, 9])) for _ in range(4))
        scale = float(rng.choice([0.125, 1.0, -0.5, 0.0, 2.0]))
        BR = int(rng.choice([0, 0, 1, 63, 64, 100, 1000]))
        w = wl.AttnWorkload(f"random_att_{i}", Nq, Nk, 64, scale, ("N", "N", "N"), seed=7000 + i,
                            ldq=ldq, ldk=ldk, ldv=ldv, ldo=ldo)
        print(f"case {i}: Nq {Nq} Nk {Nk} ld {ldq},{ldk},{ldv},{ldo} scale {scale} BR {BR}",
              flush=True)
        x = wl.make_attn_inputs(w)
        check_attn(w, x, run_attn(w, x, BR=BR or None))
