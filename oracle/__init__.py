"""CPU oracle for C = alpha*A*B + beta*C (test infrastructure only), for its
matrix-core variant with A and B rounded to fp16 or bf16 first, and for the
pages' second example, attention O = softmax(scale*Q K^T) V.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and the two share no code.

The arithmetic lives in ``sgemm_oracle.c`` (plain C, fp64 accumulation, see
its header for the definition it follows and the readings it takes).  This
module only compiles it with gcc and marshals numpy arrays through ctypes.

Matrices are passed as numpy ``float32`` buffers holding a row-major matrix
with a leading dimension: a 2-D array of shape (rows, ld) or a flat array
with at least (rows-1)*ld + cols elements.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgemm_oracle.c")
_SRC_ATT = os.path.join(_HERE, "attention_oracle.c")
LIB_PATH = os.path.join(_HERE, "libsgemm_oracle.so")

def build(force=True, src=_SRC, out=LIB_PATH, src_att=_SRC_ATT):
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-shared", "-fPIC", src, src_att, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _buf(x, rows, cols, ld, name):
    if x is None:
        return None
    a = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    if rows > 0 and cols > 0 and a.size < (rows - 1) * ld + cols:
        raise ValueError(f"{name}: buffer of {a.size} floats is too small for "
                         f"{rows}x{cols} with ld={ld}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _ld_of(x, default):
    if x is not None and getattr(x, "ndim", 1) == 2:
        return x.shape[1]
    return default


class Oracle:
    """ctypes front end of one build of ``sgemm_oracle.c``."""

    def __init__(self, lib_path=LIB_PATH):
        if not os.path.exists(lib_path):
            build(out=lib_path)
        lib = ctypes.CDLL(lib_path)
        i64, f32, vp = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        lib.oracle_sgemm.argtypes = [i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64,
                                     vp, i64, vp, i64]
        lib.oracle_sgemm.restype = ctypes.c_int
        lib.oracle_sgemm_entries.argtypes = [i64, i64, i64, f32, vp, i64, vp, i64, f32,
                                             vp, i64, i64, vp, vp, vp, vp]
        lib.oracle_sgemm_entries.restype = ctypes.c_int
        lib.oracle_round.argtypes = [ctypes.c_int, i64, vp, vp]
        lib.oracle_round.restype = ctypes.c_int
        lib.oracle_sgemm_tc.argtypes = [ctypes.c_int] + lib.oracle_sgemm.argtypes
        lib.oracle_sgemm_tc.restype = ctypes.c_int
        lib.oracle_sgemm_tc_entries.argtypes = [ctypes.c_int] + lib.oracle_sgemm_entries.argtypes
        lib.oracle_sgemm_tc_entries.restype = ctypes.c_int
        lib.oracle_attention_rows.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, f32,
                                              i64, vp, vp, i64, vp, i64]
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def max_threads(self):
        """Number of OpenMP threads the full-matrix routine runs on."""
        return int(self.lib.oracle_max_threads())

    def round(self, fmt, x):
        """x (float32 values) rounded to format fmt (F16 or BF16), as float32."""
        a = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty_like(a)
        rc = self.lib.oracle_round(int(fmt), a.size, _ptr(a), _ptr(out))
        if rc != 0:
            raise RuntimeError(f"oracle_round failed with code {rc}")
        return out

    def sgemm(self, M, N, K, alpha, A, B, beta, C, lda=None, ldb=None, ldc=None,
              bound=True, fmt=None):
        """Reference C_ref (float32, M x N) and bound (float64, M x N, or None).

        fmt (F16 or BF16): the matrix-core variant, A and B rounded to that
        format first; None: the fp32 product."""
        lda = _ld_of(A, K) if lda is None else lda
        ldb = _ld_of(B, N) if ldb is None else ldb
        ldc = _ld_of(C, N) if ldc is None else ldc
        a = _buf(A, M, K, lda, "A")
        b = _buf(B, K, N, ldb, "B")
        c = _buf(C, M, N, ldc, "C") if beta != 0 else None
        out = np.empty((M, N), dtype=np.float32)
        bnd = np.empty((M, N), dtype=np.float64) if bound else None
        args = (M, N, K, float(alpha), _ptr(a), lda, _ptr(b), ldb, float(beta), _ptr(c), ldc,
                _ptr(out), max(N, 1), _ptr(bnd), max(N, 1))
        rc = (self.lib.oracle_sgemm(*args) if fmt is None
              else self.lib.oracle_sgemm_tc(int(fmt), *args))
        if rc != 0:
            raise RuntimeError(f"oracle_sgemm failed with code {rc}")
        return out, bnd

    def sgemm_entries(self, M, N, K, alpha, A, B, beta, C, rows, cols, lda=None,
                      ldb=None, ldc=None, fmt=None):
        """Reference values and bounds at the entries (rows[t], cols[t]); fmt as
        for sgemm."""
        lda = _ld_of(A, K) if lda is None else lda
        ldb = _ld_of(B, N) if ldb is None else ldb
        ldc = _ld_of(C, N) if ldc is None else ldc
        a = _buf(A, M, K, lda, "A")
        b = _buf(B, K, N, ldb, "B")
        c = _buf(C, M, N, ldc, "C") if beta != 0 else None
        r = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        q = np.ascontiguousarray(cols, dtype=np.int64).reshape(-1)
        if r.size != q.size:
            raise ValueError("rows and cols differ in length")
        out = np.empty(r.size, dtype=np.float32)
        bnd = np.empty(r.size, dtype=np.float64)
        args = (M, N, K, float(alpha), _ptr(a), lda, _ptr(b), ldb, float(beta), _ptr(c), ldc,
                r.size, _ptr(r), _ptr(q), _ptr(out), _ptr(bnd))
        rc = (self.lib.oracle_sgemm_entries(*args) if fmt is None
              else self.lib.oracle_sgemm_tc_entries(int(fmt), *args))
        if rc != 0:
            raise RuntimeError(f"oracle_sgemm_entries failed with code {rc}")
        return out, bnd


    def attention(self, Nq, Nk, D, Q, K, V, scale, rows=None, ldq=None, ldk=None, ldv=None,
                  bound=True):
        """Rows of O = softmax(scale*Q K^T) V (all rows when rows is None), as a
        float32 (len(rows) x D) array, and their bound (float64) or None."""
        ldq = _ld_of(Q, D) if ldq is None else ldq
        ldk = _ld_of(K, D) if ldk is None else ldk
        ldv = _ld_of(V, D) if ldv is None else ldv
        q = _buf(Q, Nq, D, ldq, "Q")
        k = _buf(K, Nk, D, ldk, "K")
        v = _buf(V, Nk, D, ldv, "V")
        r = np.arange(Nq, dtype=np.int64) if rows is None else \
            np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        out = np.empty((r.size, D), dtype=np.float32)
        bnd = np.empty((r.size, D), dtype=np.float64) if bound else None
        rc = self.lib.oracle_attention_rows(Nq, Nk, D, _ptr(q), ldq, _ptr(k), ldk, _ptr(v), ldv,
                                            float(scale), r.size, _ptr(r), _ptr(out), D,
                                            _ptr(bnd), D)
        if rc != 0:
            raise RuntimeError(f"oracle_attention_rows failed with code {rc}")
        return out, bnd


# Input formats of the matrix-core variant.
F16 = 1
BF16 = 2

_default = None


def default():
    """The oracle built from ``sgemm_oracle.c`` in this directory."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def max_threads():
    return default().max_threads()


def sgemm(*args, **kwargs):
    return default().sgemm(*args, **kwargs)


def sgemm_entries(*args, **kwargs):
    return default().sgemm_entries(*args, **kwargs)


def round_to(fmt, x):
    return default().round(fmt, x)


def attention(*args, **kwargs):
    return default().attention(*args, **kwargs)
