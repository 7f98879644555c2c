"""sgemm_tc_noalloc, the allocation-free form of sgemm_tc's staged path (its
16-bit workspace is the library's static device array), through the C ABI on
the GPU: two calls in a row, the second smaller, each bit for bit equal to
sgemm_tc with the same staged configuration and within the variant oracle's
bound; the largest workspace that fits, and the first that does not."""
import numpy as np
import pytest
import torch

import fp32_gemm_02_amd as g
import sgemm_workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

FMTS = [g.SGEMM_TC_F16, g.SGEMM_TC_BF16]
FMT_IDS = ["f16", "bf16"]
STAGED = (256, 256, 64, 4, 2, 1)


@pytest.fixture(autouse=True)
def _clear_forced():
    yield
    for f in FMTS:
        g.sgemm_tc_set_config(f, None)


def _both(w, x, fmt):
    """C after sgemm_tc (staged, pool workspace) and after sgemm_tc_noalloc,
    from the same inputs."""
    dA, dB = gu.to_dev(x.A), gu.to_dev(x.B)
    c1, c2 = gu.to_dev(x.C), gu.to_dev(x.C)
    g.sgemm_tc_set_config(fmt, STAGED)
    g.sgemm_tc(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, c1, w.ldc, fmt=fmt)
    g.sgemm_tc_noalloc(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, c2, w.ldc, fmt=fmt)
    torch.cuda.synchronize()
    return c1.cpu().numpy(), c2.cpu().numpy()


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_noalloc_equals_staged_sgemm_tc_twice(fmt):
    cases = [wl.custom(2048, 1536, 1000, 1.25, 0.5, seed=31, lda=1004, ldb=1540, ldc=1544),
             wl.custom(300, 1100, 70, -0.75, 2.0, seed=32, lda=73, ldb=1103, ldc=1105)]
    for w in cases:
        print(f"noalloc fmt {fmt} {w.M}x{w.N}x{w.K}", flush=True)
        x = wl.make_inputs(w)
        staged, noalloc = _both(w, x, fmt)
        assert np.array_equal(staged.view(np.int32), noalloc.view(np.int32))
        gu.check_full(w, x, noalloc, fmt=fmt)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_noalloc_largest_workspace(fmt):
    # (4096 + 4096) * 4096 * 2 bytes: exactly the static workspace
    w = wl.custom(4096, 4096, 4096, 1.0, 1.0, seed=33)
    assert (w.M + w.N) * w.K * 2 == g.SGEMM_TC_SCRATCH_BYTES
    print(f"noalloc fmt {fmt} 4096^3", flush=True)
    x = wl.make_inputs(w)
    staged, noalloc = _both(w, x, fmt)
    assert np.array_equal(staged.view(np.int32), noalloc.view(np.int32))
    gu.check_sampled(w, x, noalloc, count=2000, fmt=fmt)
    # one more row of 256 does not fit: refused before anything is enqueued
    d = gu.to_dev(np.zeros(16, np.float32))
    st = g.sgemm_tc_noalloc_raw(4097, 4096, 4096, 1.0, d.data_ptr(), 4096, d.data_ptr(), 4096,
                                1.0, d.data_ptr(), 4096, fmt)
    assert st == g.SGEMM_ERR_SCRATCH
