"""Helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the CPU oracle."""
import numpy as np
import torch

import fp32_gemm_02_amd as g
import oracle
import sgemm_workloads as wl

U = 2.0 ** -24

# (workload, largest err/bound) of the checks run in this session; the
# conftest prints them at the end of the run
REPORT = []


def report(name, worst):
    REPORT.append((name, float(worst)))
    print(f"{name}: max err/bound {worst:.3g}", flush=True)


def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(buf):
    return torch.from_numpy(np.ascontiguousarray(buf)).to(device())


def run(w, x, entry=None, tiles=None, offset_c=0, fmt=None):
    """Run the HIP path on the inputs x; returns the flat C buffer after the call.
    fmt: the matrix-core variant (sgemm_tc) with that input format."""
    entry = entry or w.entry
    dA, dB, dC = to_dev(x.A), to_dev(x.B), to_dev(x.C)
    if fmt is not None or entry == "sgemm_tc":
        g.sgemm_tc(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc, fmt=fmt)
    elif entry == "sgemm":
        g.sgemm(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc)
    else:
        TM, TN, TK = tiles or (w.TM, w.TN, w.TK)
        g.sgemm_supertiled(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc,
                           TM, TN, TK)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


def logical_c(w, flat):
    return flat[: w.M * w.ldc].reshape(w.M, w.ldc)[:, : w.N]


def check_full(w, x, out, steps=1, exact=False, relaxed=False, fmt=None):
    """Every element against the full oracle; pads and guard row untouched.
    fmt: against the oracle of the matrix-core variant with that input format."""
    ref, bnd = oracle.sgemm(w.M, w.N, w.K, w.alpha, x.A, x.B, w.beta, x.C,
                            lda=w.lda, ldb=w.ldb, ldc=w.ldc, fmt=fmt)
    got = logical_c(w, out)
    assert not np.isnan(got).any(), f"{w.name}: NaN in C"
    if exact:
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{w.name}: {len(bad)} elements differ, first {bad[:5].tolist()}"
    else:
        tol = bnd
        if relaxed and w.K > 0:
            # Shapes outside the five workloads (tiny K, many super-tile steps):
            # first-order fp32 error of the path is at most K + 2 roundings of
            # alpha*sum, two per super-tile step on the running C, and half an
            # ulp of the oracle's own rounding; for K >= 3 and one step that is
            # below the printed 2*K*u bound, which then applies unchanged.
            mag = (bnd - 1e-30) / (2 * w.K * U)       # |alpha|*S + |beta*c|
            tol = max(2 * w.K, w.K + 2 * steps + 3) * U * mag + 1e-30
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        ratio = err / tol
        worst = np.unravel_index(np.argmax(ratio), ratio.shape)
        assert np.all(err <= tol), (f"{w.name}: max err/bound {ratio.max():.3g} at {worst}, "
                                    f"got {got[worst]} want {ref[worst]}")
    check_pads(w, x, out)
    return ref


def assert_well_inside(name, worst, limit=0.25):
    """The bound 2Ku(...) is a worst case: the error of a correct fp32 path is
    a random walk far inside it (a largest err/bound of order 1e-2 at these
    sizes).  A ratio above a quarter of the bound marks a path that is wrong
    yet still within it, e.g. one that drops or repeats a small term."""
    report(name, worst)
    assert worst < limit, f"{name}: max err/bound {worst:.3g}, expected well below {limit}"


def check_rows(w, x, outs, exact=False, slab=None, row_slabs=None):
    """Every element of the named outputs (dict name -> flat C buffer after a
    run on the inputs x) against the full oracle, computed slab by slab of
    rows (all rows when `slab` is None; only the (first, count) ranges of
    `row_slabs` when given).  exact: bit for bit (integer inputs); else each
    element within the oracle's bound, and with two outputs their difference
    within the same bound too.  Pads and the guard row of every output must be
    unchanged.  Returns {name: largest err/bound} ({} when exact)."""
    names = list(outs)
    worst = {n: 0.0 for n in names}
    pair_worst = 0.0
    if row_slabs is None:
        step = slab or w.M
        row_slabs = [(r0, min(step, w.M - r0)) for r0 in range(0, w.M, step)]
    got_all = {n: logical_c(w, outs[n]) for n in names}
    for r0, rows in row_slabs:
        a = x.A[r0 * w.lda:]
        c = x.C[r0 * w.ldc:]
        ref, bnd = oracle.sgemm(rows, w.N, w.K, w.alpha, a, x.B, w.beta, c,
                                lda=w.lda, ldb=w.ldb, ldc=w.ldc, bound=not exact)
        for n in names:
            got = got_all[n][r0:r0 + rows]
            assert not np.isnan(got).any(), f"{w.name}/{n}: NaN in rows {r0}..{r0 + rows - 1}"
            if exact:
                bad = np.argwhere(got != ref)
                assert bad.size == 0, (f"{w.name}/{n}: {len(bad)} elements differ in rows "
                                       f"{r0}..{r0 + rows - 1}, first {(bad[:5] + [r0, 0]).tolist()}")
                continue
            err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
            ratio = err / bnd
            at = np.unravel_index(np.argmax(ratio), ratio.shape)
            assert np.all(err <= bnd), (f"{w.name}/{n}: err/bound {ratio.max():.3g} at row "
                                        f"{r0 + at[0]}, column {at[1]}")
            worst[n] = max(worst[n], float(ratio.max()))
        if not exact and len(names) == 2:
            d = np.abs(got_all[names[0]][r0:r0 + rows].astype(np.float64)
                       - got_all[names[1]][r0:r0 + rows])
            assert np.all(d <= bnd), (f"{w.name}: |{names[0]} - {names[1]}| above the bound, "
                                      f"ratio {(d / bnd).max():.3g}")
            pair_worst = max(pair_worst, float((d / bnd).max()))
        if len(row_slabs) > 1:
            print(f"  {w.name}: rows {r0}..{r0 + rows - 1} checked", flush=True)
    for n in names:
        check_pads(w, x, outs[n])
    if exact:
        return {}
    if len(names) == 2:
        report(f"{w.name}: |{names[0]} - {names[1]}|", pair_worst)
    return worst


def check_pads(w, x, out):
    pads = wl.c_pad_mask(w)
    same = out[pads].view(np.int32) == x.C[pads].view(np.int32)
    assert same.all(), f"{w.name}: {int((~same).sum())} pad/guard elements of C changed"


def check_sampled(w, x, out, count=4000, exact=False, seed=7, fmt=None):
    """Sampled entries against the oracle's per-entry routine (fmt: the
    matrix-core variant's)."""
    rows, cols = wl.sample_entries(w, count, seed=seed)
    ref, bnd = oracle.sgemm_entries(w.M, w.N, w.K, w.alpha, x.A, x.B, w.beta, x.C, rows, cols,
                                    lda=w.lda, ldb=w.ldb, ldc=w.ldc, fmt=fmt)
    got = logical_c(w, out)[rows, cols]
    assert not np.isnan(got).any(), f"{w.name}: NaN at sampled entries"
    if exact:
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, f"{w.name}: {bad.size} sampled entries differ"
    else:
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        assert np.all(err <= bnd), f"{w.name}: sampled max err/bound {(err / bnd).max():.3g}"
    return float((np.abs(got.astype(np.float64) - ref) / bnd).max())


def check_freivalds(w, x, out, seed=3, chunk=2048, fmt=None):
    """A property that holds at any size: C_out @ v against alpha*A@(B@v) + beta*C0@v.

    For every row i, |sum_j (C_out - C_exact)_ij v_j| <= sum_j |v_j| Bnd_ij, and
    the right side is 2Ku(|alpha| |A|(|B||v|) + |beta| |C0||v|) + 1e-30 sum|v|,
    which needs only matrix-vector products (fp64, on the CPU).  A wrong tile,
    a lost K chunk or a misplaced row shows up as a violation.
    """
    rng = np.random.default_rng(seed)
    v = rng.choice([-1.0, 1.0], size=w.N)
    A = x.logical("A")
    B = x.logical("B")
    if fmt is not None:
        # the matrix-core variant multiplies the inputs as rounded by the oracle
        A = oracle.round_to(fmt, A)
        B = oracle.round_to(fmt, B)
    C0 = x.logical("C")
    Cout = logical_c(w, out)

    def mv(Mat, vec):
        res = np.empty(Mat.shape[0])
        for r in range(0, Mat.shape[0], chunk):
            res[r:r + chunk] = Mat[r:r + chunk].astype(np.float64) @ vec
        return res

    def amv(Mat, vec):
        res = np.empty(Mat.shape[0])
        for r in range(0, Mat.shape[0], chunk):
            res[r:r + chunk] = np.abs(Mat[r:r + chunk].astype(np.float64)) @ vec
        return res

    bv = mv(B, v)
    abv = amv(B, np.abs(v))
    y_ref = w.alpha * mv(A, bv)
    mag = abs(w.alpha) * amv(A, abv)
    if w.beta != 0:
        y_ref += w.beta * mv(C0, v)
        mag += abs(w.beta) * amv(C0, np.abs(v))
    y = mv(Cout, v)
    # fp64 rounding of the two sides is far below the fp32 bound; allow it anyway
    tol = 2 * w.K * U * mag + 1e-30 * w.N + 1e-12 * (mag + np.abs(y))
    err = np.abs(y - y_ref)
    assert np.all(err <= tol), f"{w.name}: Freivalds row check, max err/tol {(err / tol).max():.3g}"
