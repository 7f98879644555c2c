"""The host-resident super-tiled executor on the GPU: A, B and C in host
memory, a bounded set of device tile slots, loads and stores overlapped with
the step leaves ("@cluster" page, "What runs today").  Its result must be bit
for bit that of the device-resident super-tiled entry with the same extents
(the same leaves on the same values), and within the oracle's bound."""
import numpy as np
import pytest
import torch

import fp32_gemm_02_amd as g
import sgemm_workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _plan(TM, TN, TK, a, b, c, walk=g.SGEMM_WALK_ROWS):
    p = g.sgemm_plan()
    p.TM, p.TN, p.TK, p.a_slots, p.b_slots, p.c_slots, p.walk = TM, TN, TK, a, b, c, walk
    return p


def _pinned(buf):
    return torch.from_numpy(np.ascontiguousarray(buf)).pin_memory()


def run_host(w, x, plan, pinned=True, stream=None):
    """The executor on host copies of x's buffers; returns (C, A, B) after the call."""
    if pinned:
        A, B, C = _pinned(x.A), _pinned(x.B), _pinned(x.C)
    else:
        A, B, C = x.A.copy(), x.B.copy(), x.C.copy()
    g.sgemm_supertiled_host(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, plan,
                            stream=stream)
    as_np = (lambda t: t.numpy()) if pinned else (lambda t: t)
    return as_np(C), as_np(A), as_np(B)


def _steps(K, TK):
    return max(1, -(-K // min(TK, max(K, 1))))


def _check(w, x, plan, **kw):
    out, A, B = run_host(w, x, plan, **kw)
    # inputs untouched, C's pads and guard row untouched
    assert np.array_equal(A.view(np.int32), x.A.view(np.int32))
    assert np.array_equal(B.view(np.int32), x.B.view(np.int32))
    gu.check_pads(w, x, out)
    dev = gu.run(w, x, entry="sgemm_supertiled", tiles=(plan.TM, plan.TN, plan.TK))
    got, want = gu.logical_c(w, out), gu.logical_c(w, dev)
    bad = np.argwhere(got.view(np.int32) != want.view(np.int32))
    assert bad.size == 0, f"{len(bad)} elements differ from the device-resident result, " \
                          f"first {bad[:5].tolist()}"
    return out


ROWS, SHELLS, BLOCKS = g.SGEMM_WALK_ROWS, g.SGEMM_WALK_SHELLS, g.SGEMM_WALK_BLOCKS

# (M, N, K), (TM, TN, TK), slots a/b/c, walk, alpha, beta
CASES = [
    ((300, 270, 200), (128, 128, 64), (2, 2, 2), ROWS, 1.5, 0.5),    # A, B evicted and re-loaded
    ((300, 270, 200), (128, 128, 64), (4, 12, 1), ROWS, 1.0, 1.0),   # resident A row and B; 1 C slot
    ((129, 65, 300), (1000, 1000, 64), (2, 2, 2), ROWS, 1.0, 0.0),   # one super-tile, beta = 0
    ((100, 90, 70), (48, 40, 7), (1, 1, 1), ROWS, 1.0, -1.0),        # one slot each; TK % 4 != 0
    ((64, 70, 40), (64, 64, 1), (2, 3, 2), ROWS, 2.0, 0.5),          # one k per step: 40 steps
    ((513, 515, 260), (256, 256, 256), (1, 2, 2), ROWS, -0.5, 2.0),  # ragged tiles on every axis
    ((300, 270, 200), (128, 128, 64), (12, 12, 2), SHELLS, 1.5, 0.5),  # 3x3 grid in shells
    ((500, 200, 130), (96, 64, 64), (18, 12, 2), SHELLS, 1.0, 0.0),    # 6x4 grid: rows past the square
    ((200, 500, 130), (64, 96, 64), (12, 18, 1), SHELLS, 1.0, 1.0),    # 4x6: columns past the square
    ((300, 270, 200), (128, 128, 64), (2, 2, 2), SHELLS, 2.0, -1.0),   # shells with evictions
    # blocks of 2 x 2 output super-tiles, the K loop outside inside a block
    ((300, 270, 200), (128, 128, 64), (2, 2, 4), BLOCKS, 1.5, 0.5),    # 3x3 grid: edge blocks, evictions
    ((300, 270, 200), (128, 128, 64), (8, 12, 8), BLOCKS, 1.0, 1.0),   # a block row of A, all of B
    ((500, 200, 130), (96, 64, 64), (6, 6, 4), BLOCKS, 1.0, 0.0),      # 6x4 grid, beta = 0
    ((64, 200, 70), (64, 64, 16), (1, 1, 2), BLOCKS, 2.0, -1.0),       # 1x4 grid: blocks of two
]


@pytest.mark.parametrize("shape,tiles,slots,walk,alpha,beta", CASES)
def test_host_executor_matches_device_and_oracle(shape, tiles, slots, walk, alpha, beta):
    M, N, K = shape
    print(f"host executor {shape} tiles {tiles} slots {slots} walk {walk}", flush=True)
    cdist = "NaN" if beta == 0 else "U"
    w = wl.custom(M, N, K, alpha, beta, ("U", "U", cdist), seed=M + N + K, lda=K + 4,
                  ldb=N + 2, ldc=N + 6)
    x = wl.make_inputs(w)
    plan = _plan(*tiles, *slots, walk=walk)
    out = _check(w, x, plan)
    gu.check_full(w, x, out, steps=_steps(K, tiles[2]), relaxed=True)
    wi = w.integer_variant()
    xi = wl.make_inputs(wi)
    outi = _check(wi, xi, plan)
    gu.check_full(wi, xi, outi, exact=True)


def test_host_executor_without_steps():
    """K = 0 or alpha = 0: C <- beta*C through load, init leaf, store."""
    for K, alpha, beta in ((0, 1.0, -2.0), (50, 0.0, 0.5), (50, 0.0, 0.0)):
        w = wl.custom(90, 70, K, alpha, beta, seed=3, lda=max(K, 1))
        x = wl.make_inputs(w)
        want = (np.float32(beta) * x.logical("C")).astype(np.float32) if beta else \
            np.zeros((w.M, w.N), np.float32)
        for plan in (_plan(32, 32, 16, 2, 2, 2), _plan(32, 32, 16, 2, 2, 4, walk=BLOCKS)):
            out, _, _ = run_host(w, x, plan)
            assert np.array_equal(gu.logical_c(w, out).view(np.int32), want.view(np.int32))
            gu.check_pads(w, x, out)


def test_host_executor_pageable_memory_and_side_stream():
    w = wl.custom(300, 270, 200, 1.0, 0.5, seed=21, lda=204, ldb=272, ldc=276)
    x = wl.make_inputs(w)
    plan = _plan(128, 128, 64, 2, 2, 2)
    s = torch.cuda.Stream()
    a, _, _ = run_host(w, x, plan, pinned=False, stream=s)
    b, _, _ = run_host(w, x, plan, pinned=True, stream=s)
    assert np.array_equal(gu.logical_c(w, a).view(np.int32), gu.logical_c(w, b).view(np.int32))
    gu.check_full(w, x, a, steps=4, relaxed=True)


def test_host_executor_trace_counts_leaves():
    M, N, K = 300, 270, 200
    w = wl.custom(M, N, K, 1.0, 0.5, seed=9)
    x = wl.make_inputs(w)
    g.sgemm_trace_begin(1000)
    out, _, _ = run_host(w, x, _plan(128, 128, 64, 2, 2, 2))
    ms, kinds, n = g.sgemm_trace_end()
    tiles = 3 * 3
    assert n == tiles * (1 + 4)
    assert kinds[:5] == [g.SGEMM_KIND_INIT_LEAF] + [g.SGEMM_KIND_GEMM] * 4
    gu.check_full(w, x, out, steps=4)


def test_host_executor_planned_small_budget():
    """The planner's plan under a budget far below the operands' size."""
    w = wl.custom(2000, 1800, 1500, 1.0, 1.0, seed=5, lda=1500, ldb=1800, ldc=1800)
    x = wl.make_inputs(w)
    budget = 8 << 20
    plan = g.sgemm_plan_supertiles(w.M, w.N, w.K, w.beta, budget)
    print(f"planned {plan}", flush=True)
    assert plan.device_bytes <= budget
    out = _check(w, x, plan)
    gu.check_full(w, x, out, steps=_steps(w.K, plan.TK), relaxed=True)


@pytest.mark.parametrize("budget", [16 << 30, 2 << 30, 256 << 20])
def test_host_executor_16384(budget):
    """The 16384^3 product from host memory with the planner's plan: bit for
    bit the device-resident super-tiled result with the same extents, sampled
    entries within the oracle's bound."""
    w = wl.BY_NAME["supertiled_16384_t4096"]
    x = wl.make_inputs(w)
    plan = g.sgemm_plan_supertiles(w.M, w.N, w.K, w.beta, budget)
    print(f"16384 budget {budget >> 20} MiB: {plan}", flush=True)
    out = _check(w, x, plan)
    worst = gu.check_sampled(w, x, out, count=2000)
    print(f"sampled max err/bound {worst:.3g}", flush=True)
