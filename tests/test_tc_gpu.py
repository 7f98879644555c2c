"""The matrix-core variant (sgemm_tc) on the GPU: A and B rounded to fp16 or
bf16 on load, fp32 accumulation ("Show HN: Phobos", section "Are we cuBLAS
yet?", the side-quest), against the oracle of that variant."""
import numpy as np
import pytest
import torch

import fp32_gemm_02_amd as g
import oracle
import sgemm_workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

FMTS = [g.SGEMM_TC_F16, g.SGEMM_TC_BF16]
FMT_IDS = ["f16", "bf16"]


@pytest.fixture(autouse=True)
def _clear_forced():
    yield
    for f in FMTS:
        g.sgemm_tc_set_config(f, None)


def test_oracle_and_library_agree_on_format_ids():
    assert (oracle.F16, oracle.BF16) == (g.SGEMM_TC_F16, g.SGEMM_TC_BF16)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_every_config_tile_edges(fmt):
    """Each compiled tile of both forms, forced, on shapes that cut its tiles
    on every edge, with padded leading dimensions (NaN pads in A and B,
    sentinel pads in C)."""
    for cfg in g.tc_configs(fmt):
        bm, bn = cfg.bm, cfg.bn
        g.sgemm_tc_set_config(fmt, cfg)
        for (M, N, K) in [(bm, bn, 32), (bm + 7, 2 * bn + 3, 4 * 32 + 5), (bm - 1, bn + 1, 31),
                          (3, 5, 70)]:
            print(f"tc fmt {fmt} cfg {cfg} shape {(M, N, K)}", flush=True)
            for beta in (0.0, 0.75):
                w = wl.custom(M, N, K, 1.25, beta, ("U", "U", "NaN" if beta == 0 else "U"),
                              seed=M * 7 + N + K, lda=K + 4, ldb=N + 4, ldc=N + 8)
                x = wl.make_inputs(w)
                out = gu.run(w, x, fmt=fmt)
                gu.check_full(w, x, out, fmt=fmt)


FUSED = (256, 256, 32, 4, 2, 0)
STAGED = (256, 256, 32, 4, 2, 1)
FORMS = [None, FUSED, STAGED]
FORM_IDS = ["default", "fused", "staged"]


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_unaligned_leading_dimensions(fmt, form):
    """Odd leading dimensions: the scalar-load kernels and cast pass."""
    g.sgemm_tc_set_config(fmt, form)
    w = wl.custom(301, 279, 203, -0.5, 2.0, seed=5, lda=205, ldb=281, ldc=283)
    x = wl.make_inputs(w)
    out = gu.run(w, x, fmt=fmt)
    gu.check_full(w, x, out, fmt=fmt)


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_integer_inputs_are_exact(fmt, form):
    """Integers -3..3 are exact in both formats and every partial sum is below
    2^24: the variant must give the exact product, equal to the fp32 oracle."""
    g.sgemm_tc_set_config(fmt, form)
    w = wl.custom(513, 300, 700, 1.5, 0.5, ("I7", "I7", "I7"), seed=6, lda=704, ldb=300, ldc=304)
    x = wl.make_inputs(w)
    out = gu.run(w, x, fmt=fmt)
    ref = gu.check_full(w, x, out, exact=True, fmt=fmt)
    ref32, _ = oracle.sgemm(w.M, w.N, w.K, w.alpha, x.A, x.B, w.beta, x.C,
                            lda=w.lda, ldb=w.ldb, ldc=w.ldc)
    assert np.array_equal(ref, ref32)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_quick_returns(fmt):
    for K, alpha, beta in ((0, 1.0, -2.0), (64, 0.0, 0.5), (64, 0.0, 0.0)):
        w = wl.custom(90, 70, K, alpha, beta, seed=3, lda=max(K, 1))
        x = wl.make_inputs(w)
        out = gu.run(w, x, fmt=fmt)
        want = (np.float32(beta) * x.logical("C")).astype(np.float32) if beta else \
            np.zeros((w.M, w.N), np.float32)
        assert np.array_equal(gu.logical_c(w, out).view(np.int32), want.view(np.int32))
        gu.check_pads(w, x, out)


# the staged 256x256 tile with 64-k chunks in the ring of five one-operand slots
STAGED64 = (256, 256, 64, 4, 2, 1)


@pytest.mark.parametrize("staged", [STAGED, STAGED64], ids=["k32_ring4", "k64_ring5"])
@pytest.mark.parametrize("shape", [(1000, 777, 300), (512, 512, 1024), (300, 1100, 70)])
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_staged_equals_fused(fmt, shape, staged):
    """Same wave tile, same k order, same conversion: the staged form (cast
    pass + 16-bit GEMM) gives the fused form's values exactly, whatever its
    chunk depth."""
    M, N, K = shape
    w = wl.custom(M, N, K, 0.75, -1.25, seed=M + K, lda=K + 3, ldb=N + 1, ldc=N + 5)
    x = wl.make_inputs(w)
    g.sgemm_tc_set_config(fmt, FUSED)
    fused = gu.logical_c(w, gu.run(w, x, fmt=fmt))
    print(f"tc fmt {fmt} staged {staged} shape {shape}", flush=True)
    g.sgemm_tc_set_config(fmt, staged)
    staged_out = gu.run(w, x, fmt=fmt)
    staged = gu.logical_c(w, staged_out)
    bad = np.argwhere(fused != staged)
    assert bad.size == 0, f"{len(bad)} elements differ, first {bad[:5].tolist()}"
    gu.check_full(w, x, staged_out, fmt=fmt)


def test_values_past_the_fp16_range_become_infinite():
    """A value above 65504 rounds to +inf in fp16 (and stays finite in bf16):
    with positive B the whole row of C is +inf for fp16, finite for bf16."""
    w = wl.custom(64, 96, 80, 1.0, 0.0, seed=8)
    x = wl.make_inputs(w)
    A = x.logical("A")
    A[5, 3] = 70000.0
    B = x.logical("B")
    B[:] = np.abs(B) + 0.5
    out16 = gu.logical_c(w, gu.run(w, x, fmt=g.SGEMM_TC_F16))
    assert np.all(np.isposinf(out16[5]))
    rest = np.delete(out16, 5, axis=0)
    assert np.all(np.isfinite(rest))
    ref, bnd = oracle.sgemm(w.M, w.N, w.K, 1.0, x.A, x.B, 0.0, None, lda=w.lda, ldb=w.ldb,
                            fmt=oracle.F16)
    assert np.all(np.isposinf(ref[5]))
    keep = np.arange(w.M) != 5
    assert np.all(np.abs(out16[keep] - ref[keep]) <= bnd[keep])
    outbf = gu.run(w, x, fmt=g.SGEMM_TC_BF16)
    gu.check_full(w, x, outbf, fmt=g.SGEMM_TC_BF16)


def test_variant_differs_from_fp32_by_the_input_rounding_only():
    """Against the fp32 product, the fp16 variant stays within the input
    rounding bound (d(x) = max(2^-11 |x|, 2^-25)) plus the accumulation bound,
    and is not the fp32 result itself."""
    w = wl.custom(256, 256, 1024, 1.0, 0.0, seed=9)
    x = wl.make_inputs(w)
    out = gu.logical_c(w, gu.run(w, x, fmt=g.SGEMM_TC_F16))
    A = x.logical("A").astype(np.float64)
    B = x.logical("B").astype(np.float64)
    exact = A @ B
    dA = np.maximum(2.0 ** -11 * np.abs(A), 2.0 ** -25)
    dB = np.maximum(2.0 ** -11 * np.abs(B), 2.0 ** -25)
    rounding = np.abs(A) @ dB + dA @ np.abs(B) + dA @ dB
    Ar, Br = oracle.round_to(oracle.F16, x.logical("A")), oracle.round_to(oracle.F16, x.logical("B"))
    accum = 2 * w.K * gu.U * (np.abs(Ar.astype(np.float64)) @ np.abs(Br.astype(np.float64)))
    err = np.abs(out - exact)
    assert np.all(err <= rounding + accum + 1e-30)
    ref32, _ = oracle.sgemm(w.M, w.N, w.K, 1.0, x.A, x.B, 0.0, None, lda=w.lda, ldb=w.ldb)
    assert not np.array_equal(out, ref32)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_side_stream_and_trace(fmt):
    w = wl.custom(600, 520, 300, 1.0, 1.0, seed=10)
    x = wl.make_inputs(w)
    dA, dB, dC = gu.to_dev(x.A), gu.to_dev(x.B), gu.to_dev(x.C)
    s = torch.cuda.Stream()
    g.sgemm_trace_begin(16)
    g.sgemm_tc(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc, fmt=fmt,
               stream=s)
    ms, kinds, n = g.sgemm_trace_end()
    assert n == 1 and kinds == [g.SGEMM_KIND_TC] and ms[0] > 0
    s.synchronize()
    gu.check_full(w, x, dC.cpu().numpy(), fmt=fmt)
    # the staged form: the cast pass, then the GEMM, on the same stream
    g.sgemm_tc_set_config(fmt, STAGED)
    dC = gu.to_dev(x.C)
    g.sgemm_trace_begin(16)
    g.sgemm_tc(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc, fmt=fmt,
               stream=s)
    ms, kinds, n = g.sgemm_trace_end()
    assert n == 2 and kinds == [g.SGEMM_KIND_TC_CAST, g.SGEMM_KIND_TC]
    s.synchronize()
    gu.check_full(w, x, dC.cpu().numpy(), fmt=fmt)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_tc_16384(fmt):
    """The 16384^3 product (the bench shape): sampled entries against the
    variant's oracle, the row-sum property over all rows, pads untouched."""
    w = wl.custom(16384, 16384, 16384, 1.0, 1.0, seed=2, name="tc_16384")
    x = wl.make_inputs(w)
    out = gu.run(w, x, fmt=fmt)
    worst = gu.check_sampled(w, x, out, count=2000, fmt=fmt)
    print(f"tc fmt {fmt} 16384: sampled max err/bound {worst:.3g}", flush=True)
    gu.check_freivalds(w, x, out, fmt=fmt)
    gu.check_pads(w, x, out)


_T24, _T133 = 2.0 ** -24, 2.0 ** -133
SUBNORMALS = {
    g.SGEMM_TC_F16: [_T24, 1.5 * _T24, 2.5 * _T24, 2.0 ** -25, 0.75 * _T24, 2.0 ** -14 - _T24,
                     3.3e-6, -1.5 * _T24, 2.0 ** -14, 0.4 * _T24, 1023.5 * _T24, 6.1e-5],
    g.SGEMM_TC_BF16: [_T133, 1.5 * _T133, 2.5 * _T133, 2.0 ** -134, 2.0 ** -126 - _T133, 1.3e-39,
                      -3.7e-40, 2.0 ** -126, 9.1e-39, 0.4 * _T133, 5e-41, 1e-45],
}


@pytest.mark.parametrize("form", FORMS + [STAGED64], ids=FORM_IDS + ["staged_k64_ring5"])
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_subnormals_of_the_format_round_as_the_oracle(fmt, form):
    """Values in the 16-bit format's subnormal range, ties between its
    subnormals, and values that round to zero or to the smallest normal, on
    A's diagonal with B the identity: C's diagonal is each value as the
    format rounds it, the oracle's bits exactly, in every form."""
    M, N, K = 300, 300, 64
    vals = SUBNORMALS[fmt]
    A = np.zeros((M, K), np.float32)
    B = np.zeros((K, N), np.float32)
    for i in range(K):
        A[i, i] = np.float32(vals[i % len(vals)])
        B[i, i] = 1.0
    g.sgemm_tc_set_config(fmt, form)
    dA, dB = torch.from_numpy(A).to(gu.device()), torch.from_numpy(B).to(gu.device())
    dC = torch.full((M, N), float("nan"), device=gu.device())
    g.sgemm_tc(M, N, K, 1.0, dA, K, dB, N, 0.0, dC, N, fmt=fmt)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    ref, _ = oracle.sgemm(M, N, K, 1.0, A, B, 0.0, None, fmt=fmt)
    bad = np.argwhere(out.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, f"{len(bad)} elements differ, first {bad[:5].tolist()}"
    assert np.count_nonzero(np.diagonal(out)[:K]) > K // 2   # not everything flushed
