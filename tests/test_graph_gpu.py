"""The device-resident entry points under HIP stream capture.

A caller may record sgemm, sgemm_supertiled or the attention entries into a
graph and replay it: on that path the library allocates nothing, clears
nothing with memset nodes and synchronises nothing.  Each case runs once
eagerly (which also leaves the library's lazy state initialised), is captured
into a graph on the capturing stream, and is replayed three times with eager
work (a reset of the output) and a synchronisation between replays.  Every
replay must equal the eager result bit for bit, and the result the oracle.
The matrix-core variant's staged form takes its workspace from a
stream-ordered pool: captured, the allocation and the free become nodes of
the graph, and the replays must still equal the eager call."""
import numpy as np
import pytest
import torch

import fp32_gemm_02_amd as g
import oracle
import sgemm_workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


def _capture_and_replay(call, out, out0):
    """call(out) on the current stream: eager once, then captured and replayed.
    Returns the eager result; asserts every replay equals it."""
    out.copy_(out0)
    call(out)
    torch.cuda.synchronize()
    eager = _bits(out)
    graph = torch.cuda.CUDAGraph()
    out.copy_(out0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        call(out)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        out.copy_(out0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _bits(out)
        bad = np.flatnonzero(got != eager)
        assert bad.size == 0, f"replay {r}: {bad.size} elements differ, first {bad[:5].tolist()}"
    return eager


@pytest.mark.parametrize("entry,tiles,beta", [
    ("sgemm", None, 0.5),
    ("sgemm_supertiled", (256, 256, 128), 0.5),     # 3x3 ragged grid, init leaves, 3 K steps
    ("sgemm_supertiled", (256, 256, 128), 0.0),     # beta = 0: the init leaves write zeros
])
def test_gemm_graph_replays_equal_eager(entry, tiles, beta):
    M, N, K = 600, 520, 300
    w = wl.custom(M, N, K, 1.25, beta, ("U", "U", "NaN" if beta == 0 else "U"), seed=71,
                  lda=K + 4, ldb=N + 4, ldc=N + 8)
    x = wl.make_inputs(w)
    dA, dB, dC0 = gu.to_dev(x.A), gu.to_dev(x.B), gu.to_dev(x.C)
    dC = dC0.clone()
    print(f"graph {entry} tiles {tiles} beta {beta}", flush=True)

    def call(C):
        if entry == "sgemm":
            g.sgemm(M, N, K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, C, w.ldc)
        else:
            g.sgemm_supertiled(M, N, K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, C, w.ldc,
                               *tiles)

    eager = _capture_and_replay(call, dC, dC0)
    gu.check_full(w, x, eager.view(np.float32),
                  steps=1 if tiles is None else -(-K // tiles[2]), relaxed=True)


@pytest.mark.parametrize("BR", [None, 64])
def test_attention_graph_replays_equal_eager(BR):
    Nq, Nk, D, scale = 200, 300, 64, 0.125
    rng = np.random.default_rng(72)
    Q, K, V = (rng.uniform(-1, 1, (n, D)).astype(np.float32) for n in (Nq, Nk, Nk))
    dQ, dK, dV = gu.to_dev(Q), gu.to_dev(K), gu.to_dev(V)
    dO0 = torch.zeros(Nq, D, dtype=torch.float32, device=gu.device())
    dO = dO0.clone()
    print(f"graph attention BR {BR}", flush=True)

    def call(O):
        if BR is None:
            g.flash_attention(Nq, Nk, D, dQ, D, dK, D, dV, D, O, D, scale)
        else:
            g.flash_attention_supertiled(Nq, Nk, D, dQ, D, dK, D, dV, D, O, D, scale, BR)

    eager = _capture_and_replay(call, dO, dO0)
    ref, bnd = oracle.attention(Nq, Nk, D, Q, K, V, scale)
    err = np.abs(eager.view(np.float32).reshape(Nq, D).astype(np.float64) - ref)
    assert np.all(err <= bnd)


@pytest.mark.parametrize("fmt", [g.SGEMM_TC_F16, g.SGEMM_TC_BF16], ids=["f16", "bf16"])
def test_tc_staged_graph_replays_equal_eager(fmt):
    M, N, K = 2048, 2048, 4096            # long enough K for the staged form
    assert g.sgemm_tc_get_config(fmt, M, N, K).staged == 1
    w = wl.custom(M, N, K, 1.0, 0.5, seed=73)
    x = wl.make_inputs(w)
    dA, dB, dC0 = gu.to_dev(x.A), gu.to_dev(x.B), gu.to_dev(x.C)
    dC = dC0.clone()
    print(f"graph sgemm_tc fmt {fmt}", flush=True)

    def call(C):
        g.sgemm_tc(M, N, K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, C, w.ldc, fmt=fmt)

    eager = _capture_and_replay(call, dC, dC0)
    gu.check_sampled(w, x, eager.view(np.float32), count=2000, fmt=fmt)
