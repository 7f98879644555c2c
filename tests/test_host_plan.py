"""The super-tile planner and the host-resident executor's argument checks,
on the CPU (the planner is host-only; the checks return before any HIP call).

The planner follows the tuner of the "@cluster" page ("What runs today",
Tuning): candidates are enumerated, those that do not fit the memory budget
are dropped, and the rest are ranked by a cost model."""
import itertools

import pytest

import fp32_gemm_02_amd as g


def _extents(dim):
    v, p = [], 256
    while p < dim:
        v.append(p)
        p *= 2
    return v + [dim]


def _cdiv(a, b):
    return -(-a // b)


def _slot_bytes(rows, cols):
    # rows x pitch, pitch rounded up to 4 floats, slot rounded up to 256 bytes
    return 4 * ((rows * (_cdiv(cols, 4) * 4) + 63) // 64 * 64)


def _device_bytes(p):
    return (p.a_slots * _slot_bytes(p.TM, p.TK) + p.b_slots * _slot_bytes(p.TK, p.TN)
            + p.c_slots * _slot_bytes(p.TM, p.TN))


SHAPES = [(16384, 16384, 16384), (5003, 3001, 2047), (65536, 512, 4096), (300, 270, 200),
          (1, 1, 1), (4096, 4096, 100000)]
BUDGETS = [1 << 34, 2 << 30, 1 << 30, 256 << 20, 64 << 20, 8 << 20]


def _steps(gm, gn, nk, walk):
    """(pm, pn, kt) of a walk in execution order (kt over range(nk))."""
    if walk == g.SGEMM_WALK_BLOCKS:
        for m0 in range(0, gm, 2):
            for n0 in range(0, gn, 2):
                for kt in range(nk):
                    for pm in range(m0, min(m0 + 2, gm)):
                        for pn in range(n0, min(n0 + 2, gn)):
                            yield pm, pn, kt
        return
    if walk == g.SGEMM_WALK_ROWS:
        tiles = [(pm, pn) for pm in range(gm) for pn in range(gn)]
    else:   # growing squares: shell s = row s left of the diagonal, column s
        tiles = []   # above it, then the corner (s, s)
        for sh in range(max(gm, gn)):
            if sh < gm:
                tiles += [(sh, pn) for pn in range(min(sh, gn))]
            if sh < gn:
                tiles += [(pm, sh) for pm in range(min(sh, gm))]
            if sh < gm and sh < gn:
                tiles.append((sh, sh))
    for pm, pn in tiles:
        for kt in range(nk):
            yield pm, pn, kt


def _lru_loads(seq, slots):
    """Number of loads an LRU set of `slots` slots makes over the tile ids `seq`."""
    from collections import OrderedDict
    held, loads = OrderedDict(), 0
    for t in seq:
        if t in held:
            held.move_to_end(t)
        else:
            loads += 1
            if len(held) == slots:
                held.popitem(last=False)
            held[t] = True
    return loads


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_plan_is_a_candidate_and_fits_the_budget(M, N, K):
    for budget, beta in itertools.product(BUDGETS, (0.0, 1.0)):
        try:
            p = g.sgemm_plan_supertiles(M, N, K, beta, budget)
        except RuntimeError as e:
            assert "no plan fits" in str(e)
            continue
        assert p.TM in _extents(M) and p.TN in _extents(N) and p.TK in _extents(K)
        gm, gn, nk = _cdiv(M, p.TM), _cdiv(N, p.TN), _cdiv(K, p.TK)
        assert p.a_slots in (min(2, nk), nk, min(2 * nk, gm * nk), gm * nk)
        assert p.b_slots in (min(2, nk), min(2 * nk, nk * gn), nk * gn)
        live = min(2, gm) * min(2, gn)
        if p.walk == g.SGEMM_WALK_SHELLS:
            # growing squares only when every A and B super-tile stays resident
            assert p.a_slots == gm * nk and p.b_slots == nk * gn and gm > 1 and gn > 1
            assert p.c_slots == min(2, gm * gn)
        elif p.walk == g.SGEMM_WALK_ROWS:
            assert p.a_slots <= nk and p.b_slots in (min(2, nk), nk * gn)
            assert p.c_slots == min(2, gm * gn)
        else:
            # blocks: a C slot for every tile of a block, or of two blocks
            assert p.walk == g.SGEMM_WALK_BLOCKS and live > 1
            assert p.c_slots in (live, min(2 * live, gm * gn))
        # the slot bytes the executor allocates, within the budget
        assert p.device_bytes == _device_bytes(p) <= budget
        # host<->device bytes: what LRU slot sets load over the walk (all
        # super-tiles of a kind have the same extents when they divide M, N
        # and K), plus C out (and in unless beta == 0)
        c = 4 * M * N * (2 if beta else 1)
        if M % p.TM == 0 and N % p.TN == 0 and K % p.TK == 0 and gm * gn * nk <= 4096:
            steps = list(_steps(gm, gn, nk, p.walk))
            a = _lru_loads([pm * nk + kt for pm, pn, kt in steps], p.a_slots) * 4 * p.TM * p.TK
            b = _lru_loads([kt * gn + pn for pm, pn, kt in steps], p.b_slots) * 4 * p.TK * p.TN
            assert p.transfer_bytes == pytest.approx(a + b + c, rel=1e-12)
        assert p.transfer_bytes >= 4.0 * (M * K + K * N) + c
        assert p.modeled_ms > 0


def test_more_memory_never_models_slower():
    for M, N, K in SHAPES:
        prev = None
        for budget in sorted(BUDGETS):
            try:
                p = g.sgemm_plan_supertiles(M, N, K, 1.0, budget)
            except RuntimeError:
                assert prev is None     # once something fits, a larger budget fits too
                continue
            if prev is not None:
                assert p.modeled_ms <= prev.modeled_ms * (1 + 1e-9)
            prev = p


def test_plan_when_everything_fits_keeps_operands_resident():
    """With room for all of B and a row of A, each element of A and B crosses
    the link once, and loads and stores overlap, so the modeled time is the
    larger of compute and loads plus the pipeline's fill."""
    M = N = K = 16384
    p = g.sgemm_plan_supertiles(M, N, K, 1.0, 16 << 30)
    gm, gn, nk = _cdiv(M, p.TM), _cdiv(N, p.TN), _cdiv(K, p.TK)
    # a row (or a block's rows) of A resident, or all of it; all of B
    assert p.a_slots in (nk, 2 * nk, gm * nk) and p.b_slots == nk * gn
    assert p.transfer_bytes == 4.0 * (M * K + K * N + 2 * M * N)
    # super-tiles large enough to fill the 256 CUs with 256x256 workgroup tiles
    assert _cdiv(p.TM, 256) * _cdiv(p.TN, 256) >= 256
    # a faster link moves the plan toward fewer, larger tiles, never slower
    q = g.sgemm_plan_supertiles(M, N, K, 1.0, 16 << 30, link_gbs=1e6)
    assert q.modeled_ms < p.modeled_ms


def test_plan_struct_layout_matches_the_header():
    import ctypes
    assert ctypes.sizeof(g.sgemm_plan) == 64
    assert g.sgemm_plan.device_bytes.offset == 40
    assert g.sgemm_plan.walk.offset == 36


def test_planner_avoids_rows_when_b_would_arrive_all_at_once():
    """Everything resident, square grid: a row-major walk needs all of B during
    the first row of outputs; growing squares or blocks with the K loop
    outside spread the loads."""
    p = g.sgemm_plan_supertiles(16384, 16384, 16384, 1.0, 16 << 30)
    assert p.walk in (g.SGEMM_WALK_SHELLS, g.SGEMM_WALK_BLOCKS)


def test_blocks_walk_at_small_budgets():
    """With room for a few super-tiles only, blocks with the K loop outside
    share each resident A and B chunk among a block's output tiles: the
    planner takes them, and models them faster than the best row-major plan
    of the same budget."""
    M = N = K = 16384
    p = g.sgemm_plan_supertiles(M, N, K, 1.0, 256 << 20)
    assert p.walk == g.SGEMM_WALK_BLOCKS and p.c_slots >= 4


def test_plan_streams_when_memory_is_short():
    M = N = K = 16384
    p = g.sgemm_plan_supertiles(M, N, K, 1.0, 64 << 20)
    assert p.device_bytes <= 64 << 20
    assert p.transfer_bytes > 4.0 * (M * K + K * N + 2 * M * N)   # some re-loads


def test_plan_budget_error():
    with pytest.raises(RuntimeError, match="no plan fits"):
        g.sgemm_plan_supertiles(16384, 16384, 16384, 1.0, 1 << 20)
    assert g.lib().sgemm_status_string(g.SGEMM_ERR_BUDGET) == b"no plan fits the device memory budget"


def test_plan_argument_checks():
    import ctypes
    lib = g.lib()
    out = g.sgemm_plan()
    ok_model = g.sgemm_plan_model(100.0, 20.0)
    bad_models = [g.sgemm_plan_model(0.0, 20.0), g.sgemm_plan_model(100.0, -1.0),
                  g.sgemm_plan_model(float("nan"), 20.0)]
    assert lib.sgemm_plan_supertiles(0, 4, 4, 1.0, 1 << 30, None, ctypes.byref(out)) == -1
    assert lib.sgemm_plan_supertiles(4, 0, 4, 1.0, 1 << 30, None, ctypes.byref(out)) == -2
    assert lib.sgemm_plan_supertiles(4, 4, 0, 1.0, 1 << 30, None, ctypes.byref(out)) == -3
    assert lib.sgemm_plan_supertiles(4, 4, 4, 1.0, 0, None, ctypes.byref(out)) == -5
    for m in bad_models:
        assert lib.sgemm_plan_supertiles(4, 4, 4, 1.0, 1 << 30, ctypes.byref(m),
                                         ctypes.byref(out)) == -6
    assert lib.sgemm_plan_supertiles(4, 4, 4, 1.0, 1 << 30, ctypes.byref(ok_model), None) == -7
    assert lib.sgemm_plan_supertiles(4, 4, 4, 1.0, 1 << 30, ctypes.byref(ok_model),
                                     ctypes.byref(out)) == 0
    assert (out.TM, out.TN, out.TK) == (4, 4, 4)


def _plan(TM=64, TN=64, TK=64, a=2, b=2, c=2, walk=0):
    p = g.sgemm_plan()
    p.TM, p.TN, p.TK, p.a_slots, p.b_slots, p.c_slots, p.walk = TM, TN, TK, a, b, c, walk
    return p


NULL = None


@pytest.mark.parametrize("args,want", [
    ((-1, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4), -1),
    ((4, -1, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4), -2),
    ((4, 4, -1, 1.0, 8, 4, 8, 4, 0.0, 8, 4), -3),
    ((4, 4, 5, 1.0, 8, 4, 8, 4, 0.0, 8, 4), -6),     # lda < K
    ((4, 6, 4, 1.0, 8, 4, 8, 5, 0.0, 8, 6), -8),     # ldb < N
    ((4, 6, 4, 1.0, 8, 4, 8, 6, 0.0, 8, 5), -11),    # ldc < N
    ((4, 4, 4, 1.0, NULL, 4, 8, 4, 0.0, 8, 4), -5),  # A read but NULL
    ((4, 4, 4, 1.0, 8, 4, NULL, 4, 0.0, 8, 4), -7),  # B read but NULL
    ((4, 4, 4, 1.0, 8, 4, 8, 4, 0.0, NULL, 4), -10),  # C NULL
    ((0, 4, 4, 1.0, NULL, 4, NULL, 4, 0.0, NULL, 4), 0),  # M == 0: no-op
    ((4, 0, 4, 1.0, NULL, 4, NULL, 1, 0.0, NULL, 1), 0),  # N == 0: no-op
    ((4, 4, 4, 0.0, NULL, 4, NULL, 4, 1.0, 8, 4), 0),     # alpha = 0, beta = 1: C unchanged
    ((4, 4, 0, 1.0, NULL, 1, NULL, 4, 1.0, 8, 4), 0),     # K = 0, beta = 1: C unchanged
    ((1 << 31, 4, 4, 1.0, 8, 4, 8, 4, 0.0, 8, 4), g.SGEMM_ERR_TOO_LARGE),
])
def test_host_executor_argument_checks(args, want):
    assert g.sgemm_supertiled_host_raw(*args, plan=_plan(), stream=0) == want


@pytest.mark.parametrize("plan", [None, _plan(TM=0), _plan(TN=-1), _plan(TK=0), _plan(a=0),
                                  _plan(b=0), _plan(c=0), _plan(walk=3), _plan(walk=-1)])
def test_host_executor_plan_checks(plan):
    assert g.sgemm_supertiled_host_raw(4, 4, 4, 1.0, 8, 4, 8, 4, 1.0, 8, 4, plan,
                                       stream=0) == -12


def test_host_executor_blocks_need_a_c_slot_per_tile_of_a_block():
    """A 2 x 2 block of output super-tiles is live at once: fewer C slots are
    rejected before anything is allocated."""
    blocks = g.SGEMM_WALK_BLOCKS
    assert g.sgemm_supertiled_host_raw(200, 200, 64, 1.0, 8, 200, 8, 200, 1.0, 8, 200,
                                       _plan(TM=64, TN=64, c=3, walk=blocks), stream=0) == -12
    # a 1 x 4 grid has blocks of two tiles
    assert g.sgemm_supertiled_host_raw(64, 200, 64, 1.0, 8, 64, 8, 200, 1.0, 8, 200,
                                       _plan(TM=64, TN=64, c=1, walk=blocks), stream=0) == -12
