"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``check_*`` function takes an ``oracle.Oracle`` and raises
AssertionError when the oracle disagrees with:
  - hand-worked products (tests/golden/matmul_small.txt),
  - exact rational arithmetic (Python ``fractions``) rounded once to fp32,
  - closed forms of C = alpha*A*B + beta*C (identity and permutation
    operands, alpha = 0, beta = 0 with a NaN C, A = 0, K = 0, all-ones),
  - exact integer matrix products (numpy int64),
  - an independent fp64 library product (numpy float64 matmul),
  - the bound's formula evaluated exactly,
and, for the matrix-core variant (inputs rounded to fp16 or bf16 first):
  - hand-worked roundings (tests/golden/round16.txt),
  - numpy's binary16 conversion and the bfloat16 bit rule,
  - exact rational products of the rounded inputs.
The definition being pinned is the one the Phobos blog states ("Show HN:
Phobos", section "Matrix Multiplication": C = alpha*A*B + beta*C in 32-bit
floats) and the naive SGEMM it quotes (section "Introducing the Phobos
Language").  tests/test_oracle_pins.py runs every check on the oracle;
tests/test_oracle_mutants.py runs them on deliberately broken copies of it
and requires each copy to fail at least one.
"""
import os
from fractions import Fraction

import numpy as np

import sgemm_workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U24 = Fraction(1, 2 ** 24)


def rn32(q):
    """Round a Fraction to the nearest fp32 (ties to even); normal range only."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length() - 24
    two = Fraction(2)
    while q / two ** e >= 2 ** 24:
        e += 1
    while q / two ** e < 2 ** 23:
        e -= 1
    n = round(q / two ** e)          # Fraction.__round__ rounds half to even
    return np.float32(sign * n * 2.0 ** e)


def exact_product(M, N, K, alpha, A, B, beta, C):
    """alpha*A*B + beta*C and sum|A||B| as Fractions (lists of lists)."""
    F = Fraction
    out, absum = [], []
    for i in range(M):
        row, arow = [], []
        for j in range(N):
            s = F(0)
            sa = F(0)
            for k in range(K):
                p = F(float(A[i, k])) * F(float(B[k, j]))
                s += p
                sa += abs(p)
            v = F(float(np.float32(alpha))) * s
            if beta != 0:
                v += F(float(np.float32(beta))) * F(float(C[i, j]))
            row.append(v)
            arow.append(sa)
        out.append(row)
        absum.append(arow)
    return out, absum


def exact_bound(K, alpha, beta, absum, c):
    # the scalars reach the oracle as fp32 values
    bt = 0 if beta == 0 else abs(Fraction(float(np.float32(beta))) * Fraction(float(c)))
    a = abs(Fraction(float(np.float32(alpha))))
    return float(2 * K * U24 * (a * absum + bt)) + 1e-30


def ulp_diff(x, y):
    """Distance in fp32 units in the last place between same-sign finite arrays."""
    xi = np.asarray(x, np.float32).view(np.int32).astype(np.int64)
    yi = np.asarray(y, np.float32).view(np.int32).astype(np.int64)
    xi = np.where(xi < 0, -(xi & 0x7FFFFFFF), xi)
    yi = np.where(yi < 0, -(yi & 0x7FFFFFFF), yi)
    return np.abs(xi - yi)


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
def load_golden():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "matmul_small.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0]}
                cases.append(cur)
            elif key in ("M", "N", "K"):
                cur[key] = int(vals[0])
            elif key in ("alpha", "beta"):
                cur[key] = float(vals[0])
            else:
                cur[key] = np.array([float(v) for v in vals], dtype=np.float32)
    return cases


def check_golden(orc):
    for c in load_golden():
        M, N, K = c["M"], c["N"], c["K"]
        got, _ = orc.sgemm(M, N, K, c["alpha"], c["A"].reshape(M, K), c["B"].reshape(K, N),
                           c["beta"], c["C"].reshape(M, N))
        want = c["expect"].reshape(M, N)
        assert np.array_equal(got, want), (c["name"], got, want)


def check_exact_dyadic(orc):
    """Inputs k/8 with |k| <= 32: fp64 sums are exact, so oracle == RN32(exact)."""
    rng = _rng(1)
    for M, N, K in [(1, 1, 1), (2, 3, 5), (5, 2, 3), (3, 5, 8), (8, 3, 2), (4, 7, 13)]:
        for alpha, beta in [(1.0, 0.0), (0.75, -1.25), (-2.0, 0.5)]:
            A = (rng.integers(-32, 33, (M, K)) / 8).astype(np.float32)
            B = (rng.integers(-32, 33, (K, N)) / 8).astype(np.float32)
            C = (rng.integers(-32, 33, (M, N)) / 8).astype(np.float32)
            got, bnd = orc.sgemm(M, N, K, alpha, A, B, beta, C)
            ex, absum = exact_product(M, N, K, alpha, A, B, beta, C)
            want = np.array([[rn32(v) for v in r] for r in ex], dtype=np.float32)
            assert np.array_equal(got, want), ((M, N, K, alpha, beta), got, want)
            wb = np.array([[exact_bound(K, alpha, beta, absum[i][j], C[i, j])
                            for j in range(N)] for i in range(M)])
            np.testing.assert_allclose(bnd, wb, rtol=1e-13, atol=0)


def check_exact_general(orc):
    """Random fp32 inputs: within 1 ulp of RN32(exact), almost always equal."""
    rng = _rng(2)
    total = equal = 0
    for M, N, K in [(3, 4, 5), (6, 5, 17), (2, 9, 33)]:
        for alpha, beta in [(1.3, -0.7), (-1.0, 0.25), (0.1, 0.0)]:
            A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
            B = rng.standard_normal((K, N)).astype(np.float32)
            C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
            got, bnd = orc.sgemm(M, N, K, alpha, A, B, beta, C)
            ex, absum = exact_product(M, N, K, alpha, A, B, beta, C)
            want = np.array([[rn32(v) for v in r] for r in ex], dtype=np.float32)
            d = ulp_diff(got, want)
            assert d.max() <= 1, ((M, N, K), d.max())
            total += d.size
            equal += int((d == 0).sum())
            wb = np.array([[exact_bound(K, alpha, beta, absum[i][j], C[i, j])
                            for j in range(N)] for i in range(M)])
            np.testing.assert_allclose(bnd, wb, rtol=1e-13, atol=0)
    assert equal >= 0.97 * total, (equal, total)


def check_bound_covers_fp32_loop(orc):
    """A plain fp32 left-to-right loop is within the bound of the reference.

    The bound 2*K*u*(...) is at least the classical worst case of a K-term fp32
    dot product plus the epilogue, so it must cover a naive fp32 computation.
    """
    rng = _rng(3)
    M, N, K = 24, 20, 300
    alpha, beta = 1.5, 0.5
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    s = np.zeros((M, N), np.float32)
    for k in range(K):
        s = (s + np.outer(A[:, k], B[k, :]).astype(np.float32)).astype(np.float32)
    c32 = (np.float32(alpha) * s + np.float32(beta) * C).astype(np.float32)
    ref, bnd = orc.sgemm(M, N, K, alpha, A, B, beta, C)
    err = np.abs(c32.astype(np.float64) - ref.astype(np.float64))
    assert (err <= bnd).all(), (err / bnd).max()
    # and it is a genuine check: the naive loop does differ from the reference
    assert (err > 0).any()


def check_closed_forms(orc):
    rng = _rng(4)
    M, K = 37, 29
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    # B = I, alpha = 2, beta = 0.5: C = RN(2a + 0.5c) (two exact scalings, one rounding)
    got, _ = orc.sgemm(M, K, K, 2.0, A, np.eye(K, dtype=np.float32), 0.5, C)
    want = (np.float32(2) * A + np.float32(0.5) * C).astype(np.float32)
    assert np.array_equal(got, want)
    # alpha = 0: C = RN(beta*c); A and B arbitrary (finite)
    B = rng.standard_normal((K, K)).astype(np.float32)
    got, _ = orc.sgemm(M, K, K, 0.0, A, B, -0.3, C)
    assert np.array_equal(got, (np.float32(-0.3) * C).astype(np.float32))
    # beta = 0 with C = NaN: no NaN, equal to the result with a finite C
    nanC = np.full_like(C, np.nan)
    g1, b1 = orc.sgemm(M, K, K, 1.25, A, B, 0.0, nanC)
    g2, b2 = orc.sgemm(M, K, K, 1.25, A, B, 0.0, C)
    assert not np.isnan(g1).any() and not np.isnan(b1).any()
    assert np.array_equal(g1, g2) and np.array_equal(b1, b2)
    # A = 0, beta = 1: C unchanged bit for bit
    got, _ = orc.sgemm(M, K, K, 1.0, np.zeros_like(A), B, 1.0, C)
    assert np.array_equal(got.view(np.int32), C.view(np.int32))
    # K = 0: C = RN(beta*c), bound is exactly the 1e-30 floor
    got, bnd = orc.sgemm(M, K, 0, 3.0, np.zeros((M, 1), np.float32),
                         np.zeros((1, K), np.float32), 0.75, C, lda=1, ldb=K)
    assert np.array_equal(got, (np.float32(0.75) * C).astype(np.float32))
    assert np.all(bnd == 1e-30)
    # column permutation: A @ P with P[k, perm[k]] = 1 moves column k of A to perm[k]
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.float32)
    P[np.arange(K), perm] = 1
    got, _ = orc.sgemm(M, K, K, 1.0, A, P, 0.0, None)
    want = np.empty_like(A)
    want[:, perm] = A
    assert np.array_equal(got, want)
    # row permutation: Q @ B with Q[i, q[i]] = 1 takes row q[i] of B
    N = 11
    B2 = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    q = rng.permutation(K)
    Q = np.zeros((K, K), np.float32)
    Q[np.arange(K), q] = 1
    got, _ = orc.sgemm(K, N, K, 1.0, Q, B2, 0.0, None)
    assert np.array_equal(got, B2[q])
    # all ones: every sum is K exactly
    got, _ = orc.sgemm(5, 6, 7, 0.5, np.ones((5, 7), np.float32),
                       np.ones((7, 6), np.float32), -2.0, np.ones((5, 6), np.float32))
    assert np.all(got == np.float32(0.5 * 7 - 2.0))


def _int_case(orc, w):
    """Integer-valued inputs: the oracle equals exact int64 arithmetic bit for bit."""
    x = wl.make_inputs(w)
    M = w.M
    A = x.logical("A")
    B = x.logical("B")
    C = x.logical("C")
    got, _ = orc.sgemm(M, w.N, w.K, w.alpha, x.A, x.B, w.beta, x.C,
                       lda=w.lda, ldb=w.ldb, ldc=w.ldc)
    prod = A.astype(np.int64) @ B.astype(np.int64)
    want = w.alpha * prod.astype(np.float64)
    if w.beta != 0:
        want = want + w.beta * C.astype(np.float64)
    assert np.array_equal(got, want.astype(np.float32)), w.name


def check_integer_exact(orc):
    _int_case(orc, wl.WORKLOADS[0].integer_variant())
    # padded leading dimensions (NaN pads) and ragged sizes, on a slab of rows
    w5 = wl.WORKLOADS[4]
    small5 = wl.custom(71, 301, 205, w5.alpha, w5.beta, ("I7", "I7", "I7"), seed=104,
                       lda=208, ldb=304, ldc=305)
    _int_case(orc, small5)
    # tall-skinny scalars and K, on a slab of rows
    w4 = wl.WORKLOADS[3]
    _int_case(orc, wl.custom(16, w4.N, w4.K, w4.alpha, w4.beta, ("I7", "I7", "I7"),
                             seed=103, lda=w4.lda, ldb=w4.ldb, ldc=w4.ldc))


def check_numpy_fp64(orc):
    """Against an independent fp64 product (numpy matmul): within 1 ulp."""
    for w in (wl.WORKLOADS[0],
              wl.custom(90, 3001, 2047, -1.0, 0.25, seed=4, lda=2048, ldb=3008, ldc=3008)):
        x = wl.make_inputs(w)
        A = x.logical("A").astype(np.float64)
        B = x.logical("B").astype(np.float64)
        C = x.logical("C").astype(np.float64)
        got, bnd = orc.sgemm(w.M, w.N, w.K, w.alpha, x.A, x.B, w.beta, x.C,
                             lda=w.lda, ldb=w.ldb, ldc=w.ldc)
        ref = (w.alpha * (A @ B) + w.beta * C).astype(np.float32)
        d = ulp_diff(got, ref)
        assert d.max() <= 1 and (d == 0).mean() > 0.99, (w.name, d.max(), (d == 0).mean())
        wb = 2 * w.K * 2.0 ** -24 * (abs(w.alpha) * (np.abs(A) @ np.abs(B))
                                      + np.abs(w.beta * C)) + 1e-30
        np.testing.assert_allclose(bnd, wb, rtol=1e-12, atol=0)


def check_entries(orc):
    """The per-entry routine: equal to the full one, and to numpy at K = 16384."""
    w = wl.custom(150, 130, 333, 0.5, 2.0, seed=7, lda=340, ldb=131, ldc=133)
    x = wl.make_inputs(w)
    full, fb = orc.sgemm(w.M, w.N, w.K, w.alpha, x.A, x.B, w.beta, x.C,
                         lda=w.lda, ldb=w.ldb, ldc=w.ldc)
    r, c = wl.sample_entries(w, 500)
    got, gb = orc.sgemm_entries(w.M, w.N, w.K, w.alpha, x.A, x.B, w.beta, x.C, r, c,
                                lda=w.lda, ldb=w.ldb, ldc=w.ldc)
    assert np.array_equal(got, full[r, c]) and np.array_equal(gb, fb[r, c])
    # long K, as in the 16384^3 workload
    wk = wl.custom(8, 64, 16384, 1.0, 1.0, seed=2)
    xk = wl.make_inputs(wk)
    r, c = wl.sample_entries(wk, 40)
    got, gb = orc.sgemm_entries(wk.M, wk.N, wk.K, 1.0, xk.A, xk.B, 1.0, xk.C, r, c)
    A = xk.logical("A").astype(np.float64)
    B = xk.logical("B").astype(np.float64)
    C = xk.logical("C").astype(np.float64)
    ref = ((A @ B) + C)[r, c].astype(np.float32)
    d = ulp_diff(got, ref)
    assert d.max() <= 1, d.max()
    wb = 2 * wk.K * 2.0 ** -24 * ((np.abs(A) @ np.abs(B)) + np.abs(C))[r, c] + 1e-30
    np.testing.assert_allclose(gb, wb, rtol=1e-12, atol=0)


# --------------------------------------------------------------------------
# The matrix-core variant: A and B rounded to fp16 or bf16, then the product.
F16, BF16 = 1, 2


def round16_ref(fmt, x):
    """Rounding by routes independent of the oracle: numpy's binary16
    conversion, and for bfloat16 the bit rule on the fp32 encoding (add
    0x7FFF plus the lowest kept bit, then drop the low 16 bits), which is
    round to nearest even on the top 16 bits and overflows into the
    infinity encoding; NaN stays NaN."""
    x = np.asarray(x, np.float32)
    if fmt == F16:
        with np.errstate(over="ignore"):
            return x.astype(np.float16).astype(np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), x, r)


def _same_bits(a, b):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        a[~np.isnan(a)].view(np.int32), b[~np.isnan(b)].view(np.int32))


def load_round_golden():
    rows = []
    with open(os.path.join(GOLDEN, "round16.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            fmt, x, want = line.split()[:3]
            rows.append(({"f16": F16, "bf16": BF16}[fmt], float.fromhex(x), float(want)
                         if want.lstrip("-") == "inf" else float.fromhex(want)))
    return rows


def check_round_golden(orc):
    """Hand-worked roundings (ties, carries, subnormals, overflow)."""
    for fmt, x, want in load_round_golden():
        got = orc.round(fmt, np.array([x], np.float32))[0]
        assert _same_bits([got], [want]), (fmt, x.hex(), float(got).hex(), want)


def check_round_libraries(orc):
    """Many values, all binades and random encodings, against round16_ref."""
    rng = _rng(11)
    e = rng.uniform(-150, 128, 40000)
    v = (np.sign(rng.uniform(-1, 1, e.size)) * rng.uniform(1, 2, e.size) * 2.0 ** e)
    bits = rng.integers(0, 2 ** 32, 40000, dtype=np.uint64).astype(np.uint32)
    with np.errstate(over="ignore"):
        v = np.concatenate([v.astype(np.float32), bits.view(np.float32),
                            rng.uniform(-1, 1, 20000).astype(np.float32)])
    for fmt in (F16, BF16):
        assert _same_bits(orc.round(fmt, v), round16_ref(fmt, v)), fmt


def check_tc_exact(orc):
    """The variant on random fp32 inputs: within 1 ulp of RN32 of the exact
    product of the rounded inputs, almost always equal, and the bound is the
    fp32 rule on the rounded inputs."""
    rng = _rng(12)
    total = equal = 0
    for fmt in (F16, BF16):
        for M, N, K in [(3, 4, 5), (5, 3, 19)]:
            for alpha, beta in [(1.3, -0.7), (0.5, 0.0)]:
                A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
                B = rng.standard_normal((K, N)).astype(np.float32)
                C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
                got, bnd = orc.sgemm(M, N, K, alpha, A, B, beta, C, fmt=fmt)
                Ar, Br = round16_ref(fmt, A), round16_ref(fmt, B)
                ex, absum = exact_product(M, N, K, alpha, Ar, Br, beta, C)
                want = np.array([[rn32(v) for v in r] for r in ex], dtype=np.float32)
                d = ulp_diff(got, want)
                assert d.max() <= 1, (fmt, (M, N, K), d.max())
                total += d.size
                equal += int((d == 0).sum())
                wb = np.array([[exact_bound(K, alpha, beta, absum[i][j], C[i, j])
                                for j in range(N)] for i in range(M)])
                np.testing.assert_allclose(bnd, wb, rtol=1e-13, atol=0)
    assert equal >= 0.97 * total, (equal, total)


def check_tc_representable(orc):
    """Inputs that both formats hold exactly (integers -3..3): the variant is
    the fp32 product, bit for bit, and equals the exact integer result."""
    rng = _rng(13)
    M, N, K = 20, 17, 300
    A = rng.integers(-3, 4, (M, K)).astype(np.float32)
    B = rng.integers(-3, 4, (K, N)).astype(np.float32)
    C = rng.integers(-3, 4, (M, N)).astype(np.float32)
    want = (A.astype(np.int64) @ B.astype(np.int64) * 2 + C.astype(np.int64)).astype(np.float32)
    for fmt in (F16, BF16):
        got, _ = orc.sgemm(M, N, K, 2.0, A, B, 1.0, C, fmt=fmt)
        assert np.array_equal(got, want), fmt


def check_tc_entries(orc):
    """The variant's per-entry routine equals its full routine."""
    w = wl.custom(90, 70, 700, -1.5, 0.5, seed=14, lda=703, ldb=71, ldc=75)
    x = wl.make_inputs(w)
    r, c = wl.sample_entries(w, 300)
    for fmt in (F16, BF16):
        full, fb = orc.sgemm(w.M, w.N, w.K, w.alpha, x.A, x.B, w.beta, x.C,
                             lda=w.lda, ldb=w.ldb, ldc=w.ldc, fmt=fmt)
        got, gb = orc.sgemm_entries(w.M, w.N, w.K, w.alpha, x.A, x.B, w.beta, x.C, r, c,
                                    lda=w.lda, ldb=w.ldb, ldc=w.ldc, fmt=fmt)
        assert np.array_equal(got, full[r, c]) and np.array_equal(gb, fb[r, c]), fmt


# --------------------------------------------------------------------------
# Attention, O = softmax(scale * Q K^T) V over the keys (the pages' second
# @cluster example; the body is the FlashAttention paper's exact attention).
def _att_inputs(rng, Nq, Nk, D, dist="n"):
    f = (lambda s: rng.standard_normal(s)) if dist == "n" else (lambda s: rng.uniform(-1, 1, s))
    return (f((Nq, D)).astype(np.float32), f((Nk, D)).astype(np.float32),
            f((Nk, D)).astype(np.float32))


def _att_fp64(Q, K, V, scale):
    """numpy/scipy in fp64: scipy's softmax over the keys, then the product."""
    from scipy.special import softmax
    S = np.float64(np.float32(scale)) * (Q.astype(np.float64) @ K.astype(np.float64).T)
    return softmax(S, axis=1) @ V.astype(np.float64)


def check_att_library(orc):
    """Against scipy's softmax in fp64, rounded once: within half an ulp plus
    fp64 noise, on shapes with Nk != D and scales of both signs."""
    rng = _rng(31)
    for Nq, Nk, D, scale in [(9, 50, 64, 0.125), (5, 3, 64, 1.0), (17, 200, 16, -0.3),
                             (4, 129, 64, 0.7)]:
        Q, K, V = _att_inputs(rng, Nq, Nk, D)
        got, _ = orc.attention(Nq, Nk, D, Q, K, V, scale)
        ref = _att_fp64(Q, K, V, scale)
        assert np.all(np.abs(got - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-12), (Nq, Nk, D)


def check_att_closed_forms(orc):
    rng = _rng(32)
    D = 64
    Q, K, V = _att_inputs(rng, 6, 40, D)
    # one key: every weight is 1, the output is that key's value row, exactly
    got, _ = orc.attention(6, 1, D, Q, K[:1], V[:1], 0.125)
    assert np.array_equal(got, np.repeat(V[:1], 6, axis=0))
    # scale 0, or identical keys: uniform weights, the mean of the value rows
    want = V.astype(np.float64).mean(axis=0).astype(np.float32)
    got, _ = orc.attention(6, 40, D, Q, K, V, 0.0)
    assert np.all(ulp_diff(got, np.repeat(want[None], 6, axis=0)) <= 1)
    Ks = np.repeat(K[:1], 40, axis=0)
    got, _ = orc.attention(6, 40, D, Q, Ks, V, 0.9)
    assert np.all(ulp_diff(got, np.repeat(want[None], 6, axis=0)) <= 1)
    # one dominant key (score gap above 745: the others' weights are 0 in fp64)
    Qd = np.zeros((3, D), np.float32)
    Qd[:, 0] = 1.0
    Kd = np.zeros((40, D), np.float32)
    Kd[17, 0] = 1000.0
    got, _ = orc.attention(3, 40, D, Qd, Kd, V, 1.0)
    assert np.array_equal(got, np.repeat(V[17:18], 3, axis=0))


def check_att_invariances(orc):
    """A shift of all of a row's scores (through a coordinate every key shares)
    and a permutation of the keys leave the output unchanged."""
    rng = _rng(33)
    Nq, Nk, D = 8, 90, 64
    Q, K, V = _att_inputs(rng, Nq, Nk, D)
    Q[:, 5] = 0.0
    K[:, 5] = 1.0
    base, _ = orc.attention(Nq, Nk, D, Q, K, V, 0.125)
    Qs = Q.copy()
    Qs[:, 5] = np.linspace(1e4, 3e4, Nq, dtype=np.float32)   # scores shifted by 1250..3750
    shifted, _ = orc.attention(Nq, Nk, D, Qs, K, V, 0.125)
    assert np.all(np.isfinite(shifted)) and np.all(ulp_diff(shifted, base) <= 4)
    perm = rng.permutation(Nk)
    permuted, _ = orc.attention(Nq, Nk, D, Q, K[perm], V[perm], 0.125)
    assert np.all(ulp_diff(permuted, base) <= 2)


def check_att_bound_covers_fp32(orc):
    """A plain fp32 attention (numpy float32: scores, running maximum, exp, sums)
    lies within the oracle's bound, and the bound is not vacuous."""
    rng = _rng(34)
    for Nq, Nk, D, scale, dist in [(16, 300, 64, 0.125, "n"), (8, 1000, 64, 1.0, "u"),
                                   (8, 64, 16, 2.0, "n")]:
        Q, K, V = _att_inputs(rng, Nq, Nk, D, dist)
        got, bnd = orc.attention(Nq, Nk, D, Q, K, V, scale)
        S = (Q @ K.T) * np.float32(scale)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        O32 = (P @ V) / P.sum(axis=1, keepdims=True, dtype=np.float32)
        ref = _att_fp64(Q, K, V, scale)
        assert np.all(np.abs(O32.astype(np.float64) - ref) <= bnd), (Nq, Nk, D)
        assert np.all(np.abs(got.astype(np.float64) - ref) <= bnd)
        # not vacuous: far below the scale of the values themselves
        assert bnd.max() < 1e-2 * np.abs(V).max()


def _att_fp32_sequential(Q, K, V, scale):
    """Attention in fp32 with sequential (left to right) sums: dot products,
    weight sum and weighted sum accumulated one term at a time."""
    Q, K, V = (np.asarray(a, np.float32) for a in (Q, K, V))
    prod = Q[:, None, :] * K[None, :, :]                       # exact-ish fp32 products
    S = np.cumsum(prod, axis=2, dtype=np.float32)[:, :, -1] * np.float32(scale)
    P = np.exp(S - S.max(axis=1, keepdims=True)).astype(np.float32)
    l = np.cumsum(P, axis=1, dtype=np.float32)[:, -1:]
    out = np.empty((Q.shape[0], V.shape[1]), np.float32)
    for i in range(Q.shape[0]):
        out[i] = np.cumsum(P[i][:, None] * V, axis=0, dtype=np.float32)[-1] / l[i]
    return out


def check_att_bound_needs_every_term(orc):
    """Sequential fp32 sums stay within the bound where each of its terms is
    needed: long key ranges (the output and weight sums drift by many ulps)
    and scores with a large common part (the dot products' rounding changes
    the weights)."""
    rng = _rng(36)
    # 50k keys, uniform weights, values near 1: the running fp32 sum drifts
    Nq, Nk, D = 2, 50000, 8
    Q = np.zeros((Nq, D), np.float32)
    K = np.zeros((Nk, D), np.float32)
    V = rng.uniform(0.5, 1.5, (Nk, D)).astype(np.float32)
    _, bnd = orc.attention(Nq, Nk, D, Q, K, V, 1.0)
    ref = _att_fp64(Q, K, V, 1.0)
    got = _att_fp32_sequential(Q, K, V, 1.0)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= bnd) and err.max() > 64 * 2.0 ** -24 * np.abs(ref).max()
    # every score = 2^20 + 63 terms below 1.5: each fp32 addition onto 2^20
    # loses up to 1/16, so the scores, and with them the weights, differ from
    # the exact ones far more than the scores' own rounding (u*|S|) would
    # allow; only the dot products' error term (2*D*u*sum|q*k|) covers it
    rng = _rng(36)
    Nq, Nk, D = 16, 64, 64
    Q = np.ones((Nq, D), np.float32)
    Q[:, 0] = 2.0 ** 20
    Q[:, 1:] = rng.uniform(0.5, 1.5, (Nq, D - 1)).astype(np.float32)
    K = rng.uniform(0, 1, (Nk, D)).astype(np.float32)
    K[:, 0] = 1.0
    V = rng.standard_normal((Nk, D)).astype(np.float32)
    _, bnd = orc.attention(Nq, Nk, D, Q, K, V, 1.0)
    ref = _att_fp64(Q, K, V, 1.0)
    got = _att_fp32_sequential(Q, K, V, 1.0)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= bnd) and err.max() > 0.1


def check_att_rows(orc):
    """Selected rows equal the same rows of the full output."""
    rng = _rng(35)
    Q, K, V = _att_inputs(rng, 40, 77, 64)
    full, fb = orc.attention(40, 77, 64, Q, K, V, 0.2)
    rows = np.array([39, 0, 17, 17, 5])
    got, gb = orc.attention(40, 77, 64, Q, K, V, 0.2, rows=rows)
    assert np.array_equal(got, full[rows]) and np.array_equal(gb, fb[rows])


ALL_CHECKS = [check_golden, check_exact_dyadic, check_exact_general,
              check_bound_covers_fp32_loop, check_closed_forms, check_integer_exact,
              check_numpy_fp64, check_entries, check_round_golden, check_round_libraries,
              check_tc_exact, check_tc_representable, check_tc_entries, check_att_library,
              check_att_closed_forms, check_att_invariances, check_att_bound_covers_fp32,
              check_att_bound_needs_every_term, check_att_rows]
