"""Leading dimensions too large for the kernels' 32-bit load offsets.

The GEMM kernels address a chunk's rows from a wave-uniform base with 32-bit
byte offsets per lane, the attention kernel a step's K and V rows from a
buffer descriptor.  Past 4 GiB of row span they must fall back to 64-bit
addressing (the fp32 GEMM's register path, the fused form of the 16-bit
variant, the plain loads of attention).  Each case places a small logical
matrix in a device buffer with that leading dimension (the rest of the buffer
is left uninitialised) and checks the result against the oracle on a compact
copy."""
import numpy as np
import pytest
import torch

import fp32_gemm_02_amd as g
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

_2_32 = 1 << 32


def _strided(host, ld):
    """A device buffer of (rows-1)*ld + cols floats holding `host` (rows x
    cols) with leading dimension ld; the rest is left unset."""
    rows, cols = host.shape
    buf = torch.empty((rows - 1) * ld + cols, dtype=torch.float32, device=gu.device())
    buf.as_strided((rows, cols), (ld, 1)).copy_(torch.from_numpy(host).to(gu.device()))
    return buf


def _check(got, ref, bnd, what):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= bnd), f"{what}: max err/bound {(err / bnd).max():.3g}"


@pytest.mark.parametrize("which", ["lda", "ldb"])
def test_sgemm_row_span_past_4_gib(which):
    """256 rows of A, or 32 rows of B, span more than 4 GiB: every chunk takes
    the register path."""
    M, N, K = 260, 300, 96
    rng = np.random.default_rng(11)
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    lda, ldb = K, N
    if which == "lda":
        lda = 4_300_000                     # 255 * lda * 4 > 2^32
        assert 255 * lda * 4 > _2_32
    else:
        ldb = 34_700_000                    # 31 * ldb * 4 > 2^32
        assert 31 * ldb * 4 > _2_32
    print(f"sgemm {which} lda={lda} ldb={ldb}", flush=True)
    dA, dB = _strided(A, lda), _strided(B, ldb)
    dC = torch.from_numpy(C.copy()).to(gu.device())
    g.sgemm(M, N, K, 1.25, dA, lda, dB, ldb, -0.5, dC, N)
    torch.cuda.synchronize()
    ref, bnd = oracle.sgemm(M, N, K, 1.25, A, B, -0.5, C)
    _check(dC.cpu().numpy(), ref, bnd, f"sgemm {which}")
    del dA, dB
    torch.cuda.empty_cache()


# One entry of each kernel family: the 8-wave 256x256 tile, the 320x192 tile,
# a single-wave 32x32 tile and the two split-K tile sizes.
_FAMILIES = [(256, 256, 32, 4, 2), (320, 192, 16, 2, 2), (32, 32, 32, 1, 1),
             (32, 32, 16, 2, 2), (64, 64, 16, 4, 1)]


def _round4(x):
    return (x + 3) // 4 * 4


@pytest.mark.parametrize("which", ["lda", "ldb"])
@pytest.mark.parametrize("cfg", _FAMILIES, ids=lambda c: "%dx%dx%d_w%dx%d" % c)
def test_sgemm_row_span_past_4_gib_each_kernel(cfg, which):
    """For each kernel family, forced: the BM rows of A, or the BK rows of B,
    of one chunk span more than 4 GiB (leading dimensions that are multiples
    of 4, so only the span rules out the direct loads).  One whole tile and a
    ragged one in M, two whole chunks and a tail in K."""
    bm, bn, bk = cfg[:3]
    M, N, K = bm + 3, bn + 5, 2 * bk + 8
    lda, ldb = K, N
    if which == "lda":
        lda = _round4(_2_32 // (4 * (bm - 1)) + 64)
        assert ((bm - 1) * lda + bk) * 4 > _2_32
    else:
        ldb = _round4(_2_32 // (4 * (bk - 1)) + 64)
        assert ((bk - 1) * ldb + bn) * 4 > _2_32
    rng = np.random.default_rng(14)
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    print(f"sgemm cfg {cfg} {which} M={M} N={N} K={K} lda={lda} ldb={ldb}", flush=True)
    dA, dB = _strided(A, lda), _strided(B, ldb)
    dC = torch.from_numpy(C.copy()).to(gu.device())
    g.sgemm_set_config(cfg)
    try:
        g.sgemm(M, N, K, -0.75, dA, lda, dB, ldb, 1.5, dC, N)
        torch.cuda.synchronize()
    finally:
        g.sgemm_set_config(None)
    ref, bnd = oracle.sgemm(M, N, K, -0.75, A, B, 1.5, C)
    _check(dC.cpu().numpy(), ref, bnd, f"sgemm {cfg} {which}")
    del dA, dB
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [g.SGEMM_TC_F16, g.SGEMM_TC_BF16], ids=["f16", "bf16"])
def test_tc_staged_k_past_4_gib(fmt):
    """A K so long that the staged form's 16-bit rows span more than 4 GiB per
    tile: the call falls back to the fused form and stays correct."""
    M, N, K = 40, 24, 8_450_048              # 255 * K * 2 > 2^32
    assert 255 * K * 2 > _2_32
    rng = np.random.default_rng(12)
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    print(f"tc fmt {fmt} K={K}", flush=True)
    g.sgemm_tc_set_config(fmt, (256, 256, 64, 4, 2, 1))
    try:
        dA = torch.from_numpy(A).to(gu.device())
        dB = torch.from_numpy(B).to(gu.device())
        dC = torch.from_numpy(C.copy()).to(gu.device())
        g.sgemm_tc(M, N, K, 1.0, dA, K, dB, N, 0.5, dC, N, fmt=fmt)
        torch.cuda.synchronize()
    finally:
        g.sgemm_tc_set_config(fmt, None)
    ref, bnd = oracle.sgemm(M, N, K, 1.0, A, B, 0.5, C, fmt=fmt)
    _check(dC.cpu().numpy(), ref, bnd, f"tc fmt {fmt}")
    del dA, dB
    torch.cuda.empty_cache()


def test_attention_key_rows_past_4_gib():
    """128 rows of K and V (one step) span more than 4 GiB: plain loads, with
    the keys past Nk masked in the last step."""
    Nq, Nk, D = 70, 130, 64
    ld = 8_500_000                            # 127 * ld * 4 > 2^32
    assert 127 * ld * 4 > _2_32
    rng = np.random.default_rng(13)
    Q = rng.uniform(-1, 1, (Nq, D)).astype(np.float32)
    K = rng.uniform(-1, 1, (Nk, D)).astype(np.float32)
    V = rng.uniform(-1, 1, (Nk, D)).astype(np.float32)
    print(f"attention ldk=ldv={ld}", flush=True)
    dK, dV = _strided(K, ld), _strided(V, ld)
    dQ = torch.from_numpy(Q).to(gu.device())
    dO = torch.empty(Nq, D, dtype=torch.float32, device=gu.device())
    g.flash_attention(Nq, Nk, D, dQ, D, dK, ld, dV, ld, dO, D, 0.125)
    torch.cuda.synchronize()
    ref, bnd = oracle.attention(Nq, Nk, D, Q, K, V, 0.125)
    _check(dO.cpu().numpy(), ref, bnd, "attention")
    del dK, dV
    torch.cuda.empty_cache()
