"""Seeded synthetic inputs for C = alpha*A*B + beta*C.

This module holds the workload table and the input generators, nothing of
the method's arithmetic.  The GPU path's tests, the oracle's tests, the
smoke check and the benchmark all draw their inputs from here, so both sides
see the same bits.

Recipe (one torch CPU generator per matrix set, seeded with the workload's
seed; draws in the order A, B, C, each in its logical row-major shape):
  "U"    uniform on [-1, 1):        torch.rand(shape) * 2 - 1
  "N"    standard normal:           torch.randn(shape)
  "N/64" normal with std 1/64:      torch.randn(shape) / 64   (1/sqrt(K), K = 4096)
  "I7"   integers -3..3 as floats:  torch.randint(-3, 4, shape)
  "NaN"  no draw; every element is NaN (beta = 0 must not read C)

Every matrix is stored as a flat float32 buffer of (rows + 1) * ld elements:
the logical rows x cols matrix, row-major with leading dimension ld, then one
guard row.  Pad columns (cols..ld-1) and the guard row of A and B hold NaN,
so a read of them poisons the product; those of C hold the sentinel 12345.0,
which a correct run leaves untouched bit for bit.

The five workloads are the SGEMM shapes the Phobos pages measure or describe
("Show HN: Phobos", section "Are we cuBLAS yet?": 4096^3 FP32 SGEMM; section
"The Cluster Prototype": a large square SGEMM cut into square super-tiles),
plus a 256^3 case small enough for the CPU oracle, a tall-skinny case and an
unaligned case with padded leading dimensions.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

C_SENTINEL = np.float32(12345.0)


@dataclass(frozen=True)
class Workload:
    name: str
    entry: str                      # "sgemm" or "sgemm_supertiled"
    M: int
    N: int
    K: int
    lda: int
    ldb: int
    ldc: int
    alpha: float
    beta: float
    dists: Tuple[str, str, str]     # A, B, C
    seed: int
    TM: Optional[int] = None
    TN: Optional[int] = None
    TK: Optional[int] = None

    @property
    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def integer_variant(self):
        """The same shape, scalars and seed with every entry drawn from -3..3.

        With these inputs every partial sum is an integer below 2^24 and the
        scalars add at most two fractional bits, so every intermediate value is
        exact in fp32 and any order of summation gives the same bits.
        """
        c = "NaN" if self.dists[2] == "NaN" else "I7"
        return Workload(self.name + "_int", self.entry, self.M, self.N, self.K,
                        self.lda, self.ldb, self.ldc, self.alpha, self.beta,
                        ("I7", "I7", c), self.seed + 100, self.TM, self.TN, self.TK)

    def with_dists(self, dists, suffix):
        return Workload(self.name + suffix, self.entry, self.M, self.N, self.K,
                        self.lda, self.ldb, self.ldc, self.alpha, self.beta,
                        tuple(dists), self.seed, self.TM, self.TN, self.TK)


WORKLOADS = [
    Workload("sgemm_256", "sgemm", 256, 256, 256, 256, 256, 256, 1.5, 0.5,
             ("U", "U", "U"), 0),
    Workload("sgemm_4096_beta0", "sgemm", 4096, 4096, 4096, 4096, 4096, 4096, 1.0, 0.0,
             ("N", "N", "NaN"), 1),
    Workload("supertiled_16384_t4096", "sgemm_supertiled", 16384, 16384, 16384,
             16384, 16384, 16384, 1.0, 1.0, ("U", "U", "U"), 2, 4096, 4096, 4096),
    Workload("tall_skinny_65536x512x4096", "sgemm", 65536, 512, 4096, 4096, 512, 512,
             0.5, 2.0, ("N", "N/64", "U"), 3),
    Workload("unaligned_5003x3001x2047", "sgemm", 5003, 3001, 2047, 2048, 3008, 3008,
             -1.0, 0.25, ("U", "U", "U"), 4),
    # the super-tiled product's shape and inputs (same seed) as one monolithic call
    Workload("monolithic_16384", "sgemm", 16384, 16384, 16384, 16384, 16384, 16384, 1.0, 1.0,
             ("U", "U", "U"), 2),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def custom(M, N, K, alpha, beta, dists=("U", "U", "U"), seed=0, lda=None, ldb=None,
           ldc=None, entry="sgemm", TM=None, TN=None, TK=None, name="custom"):
    return Workload(name, entry, M, N, K, K if lda is None else lda,
                    N if ldb is None else ldb, N if ldc is None else ldc,
                    alpha, beta, tuple(dists), seed, TM, TN, TK)


def _draw(dist, rows, cols, gen):
    shape = (rows, cols)
    if dist == "U":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2 - 1
    if dist == "N":
        return torch.randn(shape, generator=gen, dtype=torch.float32)
    if dist == "N/64":
        return torch.randn(shape, generator=gen, dtype=torch.float32) / 64
    if dist == "I7":
        return torch.randint(-3, 4, shape, generator=gen).to(torch.float32)
    if dist == "ZERO":
        return torch.zeros(shape, dtype=torch.float32)
    if dist == "NaN":
        return torch.full(shape, float("nan"), dtype=torch.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def _embed(mat, rows, cols, ld, pad_value):
    """Flat buffer of (rows + 1) * ld floats: the matrix, pads, a guard row."""
    buf = np.empty((rows + 1) * ld, dtype=np.float32)
    view = buf[: rows * ld].reshape(rows, ld) if rows > 0 else None
    if view is not None and cols > 0:
        view[:, :cols] = mat
    if view is not None and cols < ld:
        view[:, cols:] = pad_value
    buf[rows * ld:] = pad_value
    return buf


@dataclass
class Inputs:
    w: Workload
    A: np.ndarray       # flat, (M + 1) * lda
    B: np.ndarray       # flat, (K + 1) * ldb
    C: np.ndarray       # flat, (M + 1) * ldc

    def logical(self, name):
        """The logical matrix (a view into the padded buffer)."""
        w = self.w
        rows, cols, ld = {"A": (w.M, w.K, w.lda), "B": (w.K, w.N, w.ldb),
                          "C": (w.M, w.N, w.ldc)}[name]
        buf = getattr(self, name)
        return buf[: rows * ld].reshape(rows, ld)[:, :cols]


def make_inputs(w: Workload) -> Inputs:
    gen = torch.Generator().manual_seed(w.seed)
    a = _draw(w.dists[0], w.M, w.K, gen).numpy()
    b = _draw(w.dists[1], w.K, w.N, gen).numpy()
    c = _draw(w.dists[2], w.M, w.N, gen).numpy()
    nan = np.float32(np.nan)
    return Inputs(w, _embed(a, w.M, w.K, w.lda, nan), _embed(b, w.K, w.N, w.ldb, nan),
                  _embed(c, w.M, w.N, w.ldc, C_SENTINEL))


def c_pad_mask(w: Workload):
    """Boolean mask over the flat C buffer: True on pad columns and the guard row."""
    mask = np.ones((w.M + 1) * w.ldc, dtype=bool)
    if w.M > 0 and w.N > 0:
        mask[: w.M * w.ldc].reshape(w.M, w.ldc)[:, : w.N] = False
    return mask


def sample_entries(w: Workload, count, seed=12345, edges=True):
    """Row/column indices to check at sizes where the full oracle is too slow.

    Uniform random entries plus, with edges=True, every corner and entries on
    the last rows and columns (the ragged tails of any tiling).
    """
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, w.M, count))
    cols = list(rng.integers(0, w.N, count))
    if edges:
        for i in (0, 1, w.M - 2, w.M - 1):
            for j in (0, 1, w.N - 2, w.N - 1):
                if 0 <= i < w.M and 0 <= j < w.N:
                    rows.append(i)
                    cols.append(j)
        tail = max(1, count // 8)
        rows += list(np.full(tail, w.M - 1))
        cols += list(rng.integers(0, w.N, tail))
        rows += list(rng.integers(0, w.M, tail))
        cols += list(np.full(tail, w.N - 1))
    return np.asarray(rows, dtype=np.int64), np.asarray(cols, dtype=np.int64)


# ---------------------------------------------------------------------------
# Attention inputs (the pages' flash_attention: Q[Nq, D], K, V[Nk, D], O[Nq, D]).
# The pages' job reads 16384 x 64 tensors from files of unstated content;
# seeded synthetic values of that shape stand in for them.

@dataclass
class AttnWorkload:
    name: str
    Nq: int
    Nk: int
    D: int
    scale: float
    dists: tuple = ("U", "U", "U")    # Q, K, V
    seed: int = 0
    ldq: int = 0                      # 0: D
    ldk: int = 0
    ldv: int = 0
    ldo: int = 0
    BR: int = 0                       # query rows per super-tile (0: monolithic)

    def __post_init__(self):
        for f in ("ldq", "ldk", "ldv", "ldo"):
            if getattr(self, f) == 0:
                setattr(self, f, self.D)


@dataclass
class AttnInputs:
    w: AttnWorkload
    Q: np.ndarray       # flat, (Nq + 1) * ldq, NaN pads
    K: np.ndarray       # flat, (Nk + 1) * ldk, NaN pads
    V: np.ndarray       # flat, (Nk + 1) * ldv, NaN pads
    O: np.ndarray       # flat, (Nq + 1) * ldo, every element C_SENTINEL

    def logical(self, name):
        w = self.w
        rows, ld = {"Q": (w.Nq, w.ldq), "K": (w.Nk, w.ldk), "V": (w.Nk, w.ldv),
                    "O": (w.Nq, w.ldo)}[name]
        return getattr(self, name)[: rows * ld].reshape(rows, ld)[:, : w.D]


# The pages' job: Nq = Nk = 16384, D = 64 (scale 1/sqrt(D)), cluster row block 4096.
ATTN_16384 = AttnWorkload("attention_16384_d64", 16384, 16384, 64, 0.125, seed=5, BR=4096)


def make_attn_inputs(w: AttnWorkload) -> AttnInputs:
    gen = torch.Generator().manual_seed(w.seed)
    q = _draw(w.dists[0], w.Nq, w.D, gen).numpy()
    k = _draw(w.dists[1], w.Nk, w.D, gen).numpy()
    v = _draw(w.dists[2], w.Nk, w.D, gen).numpy()
    nan = np.float32(np.nan)
    out = np.full((w.Nq + 1) * w.ldo, C_SENTINEL, dtype=np.float32)
    return AttnInputs(w, _embed(q, w.Nq, w.D, w.ldq, nan), _embed(k, w.Nk, w.D, w.ldk, nan),
                      _embed(v, w.Nk, w.D, w.ldv, nan), out)


def attn_pad_mask(w: AttnWorkload):
    """Boolean mask over the flat O buffer: True on pad columns and the guard row."""
    mask = np.ones((w.Nq + 1) * w.ldo, dtype=bool)
    if w.Nq > 0:
        mask[: w.Nq * w.ldo].reshape(w.Nq, w.ldo)[:, : w.D] = False
    return mask
