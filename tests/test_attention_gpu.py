"""Attention, the pages' second @cluster example (O = softmax(scale Q K^T) V,
D = 64), on the GPU against the attention oracle."""
import numpy as np
import pytest
import torch

import fp32_gemm_02_amd as g
import oracle
import sgemm_workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def run_attn(w, x, BR=None, stream=None):
    dQ, dK, dV, dO = (gu.to_dev(b) for b in (x.Q, x.K, x.V, x.O))
    if BR is None:
        g.flash_attention(w.Nq, w.Nk, w.D, dQ, w.ldq, dK, w.ldk, dV, w.ldv, dO, w.ldo, w.scale,
                          stream=stream)
    else:
        g.flash_attention_supertiled(w.Nq, w.Nk, w.D, dQ, w.ldq, dK, w.ldk, dV, w.ldv, dO, w.ldo,
                                     w.scale, BR, stream=stream)
    torch.cuda.synchronize()
    return dO.cpu().numpy()


def logical_o(w, flat):
    return flat[: w.Nq * w.ldo].reshape(w.Nq, w.ldo)[:, : w.D]


def check_attn(w, x, out, rows=None):
    """Rows of O against the oracle within its bound; pads and guard row untouched."""
    ref, bnd = oracle.attention(w.Nq, w.Nk, w.D, x.Q, x.K, x.V, w.scale, rows=rows,
                                ldq=w.ldq, ldk=w.ldk, ldv=w.ldv)
    got = logical_o(w, out) if rows is None else logical_o(w, out)[rows]
    assert np.all(np.isfinite(got)), f"{w.name}: non-finite output"
    err = np.abs(got.astype(np.float64) - ref)
    ratio = err / bnd
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(err <= bnd), f"{w.name}: max err/bound {ratio.max():.3g} at {worst}"
    pads = wl.attn_pad_mask(w)
    assert np.array_equal(out[pads].view(np.int32), x.O[pads].view(np.int32)), "pads changed"
    return float(ratio.max())


@pytest.mark.parametrize("Nq,Nk,scale", [(1, 1, 0.125), (64, 64, 0.125), (100, 70, 1.0),
                                         (129, 200, -0.5), (300, 1000, 0.125), (65, 130, 2.0)])
def test_attention_matches_oracle(Nq, Nk, scale):
    print(f"attention Nq={Nq} Nk={Nk} scale={scale}", flush=True)
    w = wl.AttnWorkload("small", Nq, Nk, 64, scale, ("N", "N", "N"), seed=Nq + Nk, ldq=68,
                        ldk=72, ldv=76, ldo=80)
    x = wl.make_attn_inputs(w)
    worst = check_attn(w, x, run_attn(w, x))
    print(f"  max err/bound {worst:.3g}", flush=True)


def test_attention_unaligned_leading_dimensions():
    w = wl.AttnWorkload("odd", 150, 222, 64, 0.125, seed=3, ldq=65, ldk=67, ldv=69, ldo=71)
    x = wl.make_attn_inputs(w)
    check_attn(w, x, run_attn(w, x))


def test_attention_one_key_is_exact():
    """One key: every weight is exactly 1, so every output row is V's row."""
    w = wl.AttnWorkload("one_key", 70, 1, 64, 0.3, seed=4)
    x = wl.make_attn_inputs(w)
    out = logical_o(w, run_attn(w, x))
    assert np.array_equal(out, np.repeat(x.logical("V")[:1], w.Nq, axis=0))


def test_attention_large_scores():
    """Scores in the hundreds: the running maximum keeps the exponentials finite."""
    w = wl.AttnWorkload("large", 128, 500, 64, 1.0, ("N", "N", "U"), seed=6)
    x = wl.make_attn_inputs(w)
    x.logical("Q")[:] *= 3.0
    x.logical("K")[:] *= 3.0
    check_attn(w, x, run_attn(w, x))


@pytest.mark.parametrize("order", ["rising", "falling"])
def test_attention_running_maximum_paths(order):
    """Scores that rise along the keys move every query's running maximum at
    every step (the kernel rescales its running sums each step); scores that
    fall leave it where the first step put it (the rescale is skipped from
    then on).  Both against the oracle, over several steps and a ragged last
    one."""
    w = wl.AttnWorkload("max_" + order, 200, 2000, 64, 0.125, seed=8)
    x = wl.make_attn_inputs(w)
    rng = np.random.default_rng(9)
    q, k = x.logical("Q"), x.logical("K")
    q[:] = rng.uniform(0.5, 1.0, q.shape).astype(np.float32)
    base = rng.uniform(0.5, 1.0, (1, w.D)).astype(np.float32)
    ramp = np.arange(w.Nk, dtype=np.float32)[:, None] / w.Nk
    if order == "falling":
        ramp = ramp[::-1]
    k[:] = (base * (1.0 + 4.0 * ramp)).astype(np.float32)
    check_attn(w, x, run_attn(w, x))


@pytest.mark.parametrize("BR", [64, 100, 1000, 5000])
def test_supertiled_equals_monolithic(BR):
    """Super-tiles of BR query rows (a grouped launch; BR not a multiple of 64
    leaves partly filled workgroups) give the monolithic result bit for bit."""
    w = wl.AttnWorkload("st", 1234, 777, 64, 0.125, ("U", "U", "U"), seed=7, ldo=68)
    x = wl.make_attn_inputs(w)
    mono = run_attn(w, x)
    st = run_attn(w, x, BR=BR, stream=torch.cuda.Stream())
    assert np.array_equal(logical_o(w, mono).view(np.int32), logical_o(w, st).view(np.int32))
    check_attn(w, x, st)


def test_attention_trace_one_grouped_launch():
    """The leaves of all super-tiles go out as one launch."""
    w = wl.AttnWorkload("tr", 1000, 300, 64, 0.125, seed=8)
    x = wl.make_attn_inputs(w)
    g.sgemm_trace_begin(64)
    out = run_attn(w, x, BR=256)
    ms, kinds, n = g.sgemm_trace_end()
    assert n == 1 and kinds == [g.SGEMM_KIND_ATTENTION] and ms[0] > 0
    check_attn(w, x, out)


def test_attention_16384():
    """The pages' job shape (Nq = Nk = 16384, D = 64): every row against the
    oracle; the cluster form (BR = 4096) equals the monolithic one."""
    w = wl.ATTN_16384
    x = wl.make_attn_inputs(w)
    mono = run_attn(w, x)
    worst = check_attn(w, x, mono)
    gu.report("attention_16384", worst)
    st = run_attn(w, x, BR=w.BR)
    assert np.array_equal(logical_o(w, mono).view(np.int32), logical_o(w, st).view(np.int32))


def test_attention_repeats_bit_for_bit():
    """The four key parts of a query group are merged in a fixed order: two
    calls give the same bits."""
    w = wl.AttnWorkload("repeat", 700, 3000, 64, 0.125, ("N", "N", "N"), seed=77, ldq=64,
                        ldk=64, ldv=64, ldo=64)
    x = wl.make_attn_inputs(w)
    first, second = run_attn(w, x), run_attn(w, x)
    assert np.array_equal(first.view(np.int32), second.view(np.int32))
    check_attn(w, x, first)
