"""Python binding of the gfx950 FP32 SGEMM library (libphobos_sgemm.so).

Argument marshalling only: every step of C <- alpha*A*B + beta*C runs in the
library's HIP kernels.  The functions carry the names of the C entry points
declared in include/phobos_sgemm.h and take the same arguments; pointers may
be given as integers or as tensors (their data_ptr()), the stream as a
torch.cuda.Stream, an integer hipStream_t or None (torch's current stream on
the current device).  A non-zero status raises SgemmError, except in the
``raw`` entry points, which return it.

Tensors are checked before the call: device operands must be float32,
contiguous tensors on the current GPU that hold the whole matrix their
shape and leading dimension span (host operands of sgemm_supertiled_host:
float32 host arrays or tensors of that size); anything else raises
ValueError before the library is called.  Integer addresses are passed on
unchecked.

The library is loaded from this directory.  There is no fallback: if it has
not been built (python -m fp32_gemm_02_amd.build), importing works but the
first call raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# PHOBOS_SGEMM_LIB names another build of the library (e.g. the CPU-only
# sanitizer build of the host code); by default the one built in place here
LIB_PATH = os.environ.get("PHOBOS_SGEMM_LIB") or os.path.join(HERE, "libphobos_sgemm.so")

SGEMM_OK = 0
SGEMM_ERR_NO_CONFIG = 2
SGEMM_ERR_TOO_LARGE = 3
SGEMM_ERR_ALLOC = 4
SGEMM_ERR_BUDGET = 5
SGEMM_ERR_IO = 6
SGEMM_ERR_SCRATCH = 7
SGEMM_TC_SCRATCH_BYTES = 64 * 1024 * 1024
SGEMM_ERR_HIP_BASE = 1000
SGEMM_WALK_ROWS = 0
SGEMM_WALK_SHELLS = 1
SGEMM_WALK_BLOCKS = 2
SGEMM_KIND_GEMM = 0
SGEMM_KIND_INIT_LEAF = 1
SGEMM_KIND_TC = 2
SGEMM_KIND_TC_CAST = 3
SGEMM_KIND_ATTENTION = 4
SGEMM_TC_F16 = 1
SGEMM_TC_BF16 = 2


class SgemmError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class sgemm_config(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("wm", ctypes.c_int32), ("wn", ctypes.c_int32)]

    def as_tuple(self):
        return (self.bm, self.bn, self.bk, self.wm, self.wn)

    def __repr__(self):
        return "sgemm_config(bm=%d, bn=%d, bk=%d, wm=%d, wn=%d)" % self.as_tuple()


class sgemm_tc_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("bm", "bn", "bk", "wm", "wn", "staged")]

    def as_tuple(self):
        return (self.bm, self.bn, self.bk, self.wm, self.wn, self.staged)

    def __repr__(self):
        return ("sgemm_tc_config(bm=%d, bn=%d, bk=%d, wm=%d, wn=%d, staged=%d)"
                % self.as_tuple())


class sgemm_plan_model(ctypes.Structure):
    _fields_ = [("gemm_tflops", ctypes.c_double), ("link_gbs", ctypes.c_double)]


class sgemm_plan(ctypes.Structure):
    _fields_ = [("TM", ctypes.c_int64), ("TN", ctypes.c_int64), ("TK", ctypes.c_int64),
                ("a_slots", ctypes.c_int32), ("b_slots", ctypes.c_int32),
                ("c_slots", ctypes.c_int32), ("walk", ctypes.c_int32),
                ("device_bytes", ctypes.c_int64),
                ("transfer_bytes", ctypes.c_double), ("modeled_ms", ctypes.c_double)]

    def __repr__(self):
        return ("sgemm_plan(TM=%d, TN=%d, TK=%d, slots a/b/c=%d/%d/%d, walk=%s, "
                "device_bytes=%d, transfer_bytes=%.4g, modeled_ms=%.4g)" % (
                    self.TM, self.TN, self.TK, self.a_slots, self.b_slots, self.c_slots,
                    {SGEMM_WALK_ROWS: "rows", SGEMM_WALK_SHELLS: "shells", SGEMM_WALK_BLOCKS: "blocks"}.get(self.walk, self.walk),
                    self.device_bytes, self.transfer_bytes, self.modeled_ms))


_lib = None

_i64, _f32, _i32, _vp = ctypes.c_int64, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p
_SIGNATURES = {
    "sgemm": ([_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64, _vp], ctypes.c_int),
    "sgemm_supertiled": ([_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64,
                          _i64, _i64, _i64, _vp], ctypes.c_int),
    "sgemm_init_leaf": ([_i64, _i64, _f32, _vp, _i64, _vp], ctypes.c_int),
    "sgemm_config_count": ([], ctypes.c_int),
    "sgemm_config_at": ([_i32, ctypes.POINTER(sgemm_config)], ctypes.c_int),
    "sgemm_get_config": ([_i64, _i64, _i64, _i64, _i64, _i64, ctypes.POINTER(sgemm_config)],
                         ctypes.c_int),
    "sgemm_set_config": ([ctypes.POINTER(sgemm_config)], ctypes.c_int),
    "sgemm_tune_candidates": ([_i64, _i64, _i64, ctypes.POINTER(sgemm_config), _i32],
                              ctypes.c_int),
    "sgemm_tune": ([_i64, _i64, _i64, _i64, _i64, _i64, _i32, _vp,
                    ctypes.POINTER(sgemm_config), ctypes.POINTER(_f32)], ctypes.c_int),
    "sgemm_tune_cache_load": ([ctypes.c_char_p, ctypes.POINTER(_i32)], ctypes.c_int),
    "sgemm_tune_cache_save": ([ctypes.c_char_p, ctypes.POINTER(_i32)], ctypes.c_int),
    "sgemm_tune_forget": ([], ctypes.c_int),
    "sgemm_tc": ([_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64, _i32, _vp],
                 ctypes.c_int),
    "sgemm_tc_noalloc": ([_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64, _i32,
                          _vp], ctypes.c_int),
    "sgemm_tc_config_count": ([_i32], ctypes.c_int),
    "sgemm_tc_config_at": ([_i32, _i32, ctypes.POINTER(sgemm_tc_config)], ctypes.c_int),
    "sgemm_tc_get_config": ([_i32, _i64, _i64, _i64, ctypes.POINTER(sgemm_tc_config)],
                            ctypes.c_int),
    "sgemm_tc_set_config": ([_i32, ctypes.POINTER(sgemm_tc_config)], ctypes.c_int),
    "flash_attention": ([_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _f32,
                         _vp], ctypes.c_int),
    "flash_attention_supertiled": ([_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                    _i64, _f32, _i64, _vp], ctypes.c_int),
    "sgemm_plan_supertiles": ([_i64, _i64, _i64, _f32, _i64, ctypes.POINTER(sgemm_plan_model),
                               ctypes.POINTER(sgemm_plan)], ctypes.c_int),
    "sgemm_supertiled_host": ([_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64,
                               ctypes.POINTER(sgemm_plan), _vp], ctypes.c_int),
    "sgemm_trace_begin": ([_i64], ctypes.c_int),
    "sgemm_trace_begin_sampled": ([_i64, _i64], ctypes.c_int),
    "sgemm_trace_end": ([ctypes.POINTER(_f32), ctypes.POINTER(_i32), _i64,
                         ctypes.POINTER(_i64)], ctypes.c_int),
    "sgemm_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "sgemm_version": ([], ctypes.c_int),
    "sgemm_set_log": ([_i32], ctypes.c_int),
}


def lib():
    """The loaded library with its prototypes set (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m fp32_gemm_02_amd.build")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _need(rows, cols, ld):
    """Floats a row-major rows x cols matrix with leading dimension ld spans."""
    return (rows - 1) * ld + cols if rows > 0 and cols > 0 else 0


def _dev_shape(x, rows, cols, ld, name, where):
    """ValueError unless the tensor x is float32, contiguous and holds at least
    (rows-1)*ld + cols elements from its first one (integers pass)."""
    if x is None or not hasattr(x, "data_ptr"):
        return
    import torch
    if x.dtype != torch.float32:
        raise ValueError(f"{where}: {name} must be a float32 tensor, got {x.dtype}")
    need = _need(rows, cols, ld)
    if need:
        if not x.is_contiguous():
            raise ValueError(f"{where}: {name} must be contiguous (or pass its address)")
        if x.numel() < need:
            raise ValueError(f"{where}: {name} holds {x.numel()} floats, a {rows}x{cols} "
                             f"matrix with leading dimension {ld} spans {need}")


def _dev_addr(x, name, where, cur):
    """Address of a device operand: an integer (or None) as it is; a tensor
    only if it lives on GPU `cur`, the current one (ValueError otherwise)."""
    if x is None or not hasattr(x, "data_ptr"):
        return _ptr(x)
    dev = x.get_device()          # -1 for a tensor in host memory
    if dev < 0:
        raise ValueError(f"{where}: {name} is on {x.device}, not on a GPU")
    if dev != cur:
        raise ValueError(f"{where}: {name} is on {x.device}, the current device is "
                         f"cuda:{cur}")
    return x.data_ptr()


def _dev_ptrs(where, *ops):
    """Checked addresses of device operands given as (x, rows, cols, ld, name):
    every operand's dtype and extent first, then where each lives, so that
    nothing reaches the library unless all of them pass.  The current device
    is read once per call."""
    cur = None
    for x, rows, cols, ld, name in ops:
        _dev_shape(x, rows, cols, ld, name, where)
        if cur is None and hasattr(x, "data_ptr") and x.is_cuda:
            import torch
            cur = torch.cuda.current_device()
    return tuple(_dev_addr(x, name, where, cur) for x, _, _, _, name in ops)


def _dev(x, rows, cols, ld, name, where):
    return _dev_ptrs(where, (x, rows, cols, ld, name))[0]


def _gemm_ptrs(M, N, K, alpha, A, lda, B, ldb, C, ldc, where):
    """Checked addresses of A, B and C for an M x N x K product (A and B are
    only sized when the product reads them)."""
    reads = M > 0 and N > 0 and K > 0 and alpha != 0
    return _dev_ptrs(where, (A, M if reads else 0, K, lda, "A"),
                     (B, K if reads else 0, N, ldb, "B"), (C, M if N > 0 else 0, N, ldc, "C"))


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def _check(status, where):
    if status != SGEMM_OK:
        raise SgemmError(status, where)


def status_string(status):
    return lib().sgemm_status_string(int(status)).decode()


def version():
    return lib().sgemm_version()


def sgemm_set_log(on):
    """Turn the library's dispatch log (one stderr line per decision) on or
    off; returns whether it was on."""
    return bool(lib().sgemm_set_log(1 if on else 0))


def sgemm_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    a, b, c = _gemm_ptrs(M, N, K, alpha, A, lda, B, ldb, C, ldc, "sgemm")
    return lib().sgemm(M, N, K, alpha, a, lda, b, ldb, beta, c, ldc, _stream(stream))


def sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """C <- alpha*A*B + beta*C (row-major, device pointers); asynchronous."""
    _check(sgemm_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream), "sgemm")


def sgemm_supertiled_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, TM, TN, TK,
                         stream=None):
    a, b, c = _gemm_ptrs(M, N, K, alpha, A, lda, B, ldb, C, ldc, "sgemm_supertiled")
    return lib().sgemm_supertiled(M, N, K, alpha, a, lda, b, ldb, beta, c, ldc, TM, TN, TK,
                                  _stream(stream))


def sgemm_supertiled(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, TM, TN, TK, stream=None):
    """The same product through TM x TN x TK super-tiles (init leaf + K steps)."""
    _check(sgemm_supertiled_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, TM, TN, TK,
                                stream), "sgemm_supertiled")


def sgemm_init_leaf(M, N, beta, C, ldc, stream=None):
    """C <- beta*C (C <- 0 without reading C when beta == 0)."""
    c = _dev(C, M if N > 0 else 0, N, ldc, "C", "sgemm_init_leaf")
    _check(lib().sgemm_init_leaf(M, N, beta, c, ldc, _stream(stream)), "sgemm_init_leaf")


def sgemm_tc_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, fmt, stream=None):
    a, b, c = _gemm_ptrs(M, N, K, alpha, A, lda, B, ldb, C, ldc, "sgemm_tc")
    return lib().sgemm_tc(M, N, K, alpha, a, lda, b, ldb, beta, c, ldc, fmt, _stream(stream))


def sgemm_tc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, fmt=None, stream=None):
    """C <- alpha*A'*B' + beta*C with A, B rounded to fp16 (fmt SGEMM_TC_F16,
    the default) or bf16 (SGEMM_TC_BF16) on load, fp32 accumulation."""
    fmt = SGEMM_TC_F16 if fmt is None else fmt
    _check(sgemm_tc_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, fmt, stream), "sgemm_tc")


def sgemm_tc_noalloc_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, fmt, stream=None):
    a, b, c = _gemm_ptrs(M, N, K, alpha, A, lda, B, ldb, C, ldc, "sgemm_tc_noalloc")
    return lib().sgemm_tc_noalloc(M, N, K, alpha, a, lda, b, ldb, beta, c, ldc, fmt,
                                  _stream(stream))


def sgemm_tc_noalloc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, fmt=None, stream=None):
    """sgemm_tc's staged form on the library's static 16-bit workspace (no
    allocation; the workspace must fit in SGEMM_TC_SCRATCH_BYTES)."""
    fmt = SGEMM_TC_F16 if fmt is None else fmt
    _check(sgemm_tc_noalloc_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, fmt, stream),
           "sgemm_tc_noalloc")


def tc_configs(fmt):
    """The compiled configurations of the matrix-core variant for one format
    (fused ones first, then staged ones)."""
    out = []
    for i in range(lib().sgemm_tc_config_count(fmt)):
        c = sgemm_tc_config()
        _check(lib().sgemm_tc_config_at(fmt, i, ctypes.byref(c)), "sgemm_tc_config_at")
        out.append(c)
    return out


def sgemm_tc_get_config(fmt, M, N, K):
    c = sgemm_tc_config()
    _check(lib().sgemm_tc_get_config(fmt, M, N, K, ctypes.byref(c)), "sgemm_tc_get_config")
    return c


def sgemm_tc_set_config(fmt, cfg):
    """Force one matrix-core configuration for format fmt (None clears)."""
    if cfg is not None and not isinstance(cfg, sgemm_tc_config):
        cfg = sgemm_tc_config(*cfg)
    _check(lib().sgemm_tc_set_config(fmt, None if cfg is None else ctypes.byref(cfg)),
           "sgemm_tc_set_config")


def _attn_ptrs(Nq, Nk, D, Q, ldq, K, ldk, V, ldv, O, ldo, where):
    rows = Nq if Nq > 0 else 0
    keys = Nk if Nq > 0 else 0
    return _dev_ptrs(where, (Q, rows, D, ldq, "Q"), (K, keys, D, ldk, "K"),
                     (V, keys, D, ldv, "V"), (O, rows, D, ldo, "O"))


def flash_attention_raw(Nq, Nk, D, Q, ldq, K, ldk, V, ldv, O, ldo, scale, stream=None):
    q, k, v, o = _attn_ptrs(Nq, Nk, D, Q, ldq, K, ldk, V, ldv, O, ldo, "flash_attention")
    return lib().flash_attention(Nq, Nk, D, q, ldq, k, ldk, v, ldv, o, ldo, scale,
                                 _stream(stream))


def flash_attention(Nq, Nk, D, Q, ldq, K, ldk, V, ldv, O, ldo, scale, stream=None):
    """O <- softmax(scale * Q K^T) V (row-major device buffers, D = 64)."""
    _check(flash_attention_raw(Nq, Nk, D, Q, ldq, K, ldk, V, ldv, O, ldo, scale, stream),
           "flash_attention")


def flash_attention_supertiled_raw(Nq, Nk, D, Q, ldq, K, ldk, V, ldv, O, ldo, scale, BR,
                                   stream=None):
    q, k, v, o = _attn_ptrs(Nq, Nk, D, Q, ldq, K, ldk, V, ldv, O, ldo,
                            "flash_attention_supertiled")
    return lib().flash_attention_supertiled(Nq, Nk, D, q, ldq, k, ldk, v, ldv, o, ldo, scale, BR,
                                            _stream(stream))


def flash_attention_supertiled(Nq, Nk, D, Q, ldq, K, ldk, V, ldv, O, ldo, scale, BR,
                               stream=None):
    """The same through super-tiles of BR query rows (one leaf launch each)."""
    _check(flash_attention_supertiled_raw(Nq, Nk, D, Q, ldq, K, ldk, V, ldv, O, ldo, scale, BR,
                                          stream), "flash_attention_supertiled")


def configs():
    """Every compiled configuration, as sgemm_config structures."""
    out = []
    for i in range(lib().sgemm_config_count()):
        c = sgemm_config()
        _check(lib().sgemm_config_at(i, ctypes.byref(c)), "sgemm_config_at")
        out.append(c)
    return out


def sgemm_get_config(M, N, K, lda, ldb, ldc):
    c = sgemm_config()
    _check(lib().sgemm_get_config(M, N, K, lda, ldb, ldc, ctypes.byref(c)), "sgemm_get_config")
    return c


def sgemm_set_config(cfg):
    """Force one configuration for every later call (None clears)."""
    if cfg is None:
        _check(lib().sgemm_set_config(None), "sgemm_set_config")
        return
    if not isinstance(cfg, sgemm_config):
        cfg = sgemm_config(*cfg)
    _check(lib().sgemm_set_config(ctypes.byref(cfg)), "sgemm_set_config")


def sgemm_tune_candidates(M, N, K):
    cap = lib().sgemm_config_count()
    arr = (sgemm_config * cap)()
    n = lib().sgemm_tune_candidates(M, N, K, arr, cap)
    if n < 0:
        raise SgemmError(n, "sgemm_tune_candidates")
    return [arr[i] for i in range(min(n, cap))]


def sgemm_tune(M, N, K, lda, ldb, ldc, reps=20, stream=None):
    """Time the candidates, record the winner for this shape; returns (config, ms)."""
    c = sgemm_config()
    ms = ctypes.c_float()
    _check(lib().sgemm_tune(M, N, K, lda, ldb, ldc, reps, _stream(stream), ctypes.byref(c),
                            ctypes.byref(ms)), "sgemm_tune")
    return c, ms.value


def sgemm_tune_cache_load(path):
    """Add a tuning cache file's entries to the process's table; returns their number."""
    n = _i32()
    _check(lib().sgemm_tune_cache_load(os.fsencode(path), ctypes.byref(n)),
           "sgemm_tune_cache_load")
    return n.value


def sgemm_tune_cache_save(path):
    """Write the process's tuned table to a cache file; returns the entries written."""
    n = _i32()
    _check(lib().sgemm_tune_cache_save(os.fsencode(path), ctypes.byref(n)),
           "sgemm_tune_cache_save")
    return n.value


def sgemm_tune_forget():
    """Empty the process's tuned table; returns the number of entries removed."""
    return lib().sgemm_tune_forget()


def sgemm_plan_supertiles(M, N, K, beta, device_bytes, gemm_tflops=None, link_gbs=None):
    """Super-tile extents and device slots for the host-resident product (host only)."""
    model = None
    if gemm_tflops is not None or link_gbs is not None:
        model = ctypes.byref(sgemm_plan_model(gemm_tflops or 140.0, link_gbs or 55.0))
    plan = sgemm_plan()
    _check(lib().sgemm_plan_supertiles(M, N, K, beta, device_bytes, model, ctypes.byref(plan)),
           "sgemm_plan_supertiles")
    return plan


def _host_ptr(x, rows=0, cols=0, ld=0, name="", where=""):
    """Address of a host buffer (numpy array, CPU tensor or integer).  Arrays
    and tensors must be float32, contiguous, in host memory and hold at least
    (rows-1)*ld + cols elements; otherwise ValueError."""
    if x is None:
        return None
    need = _need(rows, cols, ld)
    if hasattr(x, "ctypes") and hasattr(x, "dtype"):
        import numpy as np
        if x.dtype != np.float32:
            raise ValueError(f"{where}: {name} must be float32, got {x.dtype}")
        if need and not x.flags.c_contiguous:
            raise ValueError(f"{where}: {name} must be C-contiguous")
        if x.size < need:
            raise ValueError(f"{where}: {name} holds {x.size} floats, a {rows}x{cols} "
                             f"matrix with leading dimension {ld} spans {need}")
        return x.ctypes.data
    if hasattr(x, "data_ptr"):
        import torch
        if x.dtype != torch.float32:
            raise ValueError(f"{where}: {name} must be float32, got {x.dtype}")
        if x.is_cuda:
            raise ValueError(f"{where}: {name} must be in host memory, not on {x.device}")
        if need and not x.is_contiguous():
            raise ValueError(f"{where}: {name} must be contiguous")
        if x.numel() < need:
            raise ValueError(f"{where}: {name} holds {x.numel()} floats, a {rows}x{cols} "
                             f"matrix with leading dimension {ld} spans {need}")
        return x.data_ptr()
    return int(x)


def sgemm_supertiled_host_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, plan, stream=None):
    where = "sgemm_supertiled_host"
    reads = M > 0 and N > 0 and K > 0 and alpha != 0
    return lib().sgemm_supertiled_host(M, N, K, alpha,
                                       _host_ptr(A, M if reads else 0, K, lda, "A", where), lda,
                                       _host_ptr(B, K if reads else 0, N, ldb, "B", where), ldb,
                                       beta, _host_ptr(C, M if N > 0 else 0, N, ldc, "C", where),
                                       ldc, None if plan is None else ctypes.byref(plan),
                                       _stream(stream))


def sgemm_supertiled_host(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, plan, stream=None):
    """C <- alpha*A*B + beta*C with A, B, C in host memory; synchronous."""
    _check(sgemm_supertiled_host_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, plan, stream),
           "sgemm_supertiled_host")


def sgemm_trace_begin(capacity, every=1):
    """Bracket the next launches with HIP events (one in every `every`)."""
    _check(lib().sgemm_trace_begin_sampled(capacity, every), "sgemm_trace_begin_sampled")


def sgemm_trace_end(cap=1 << 16):
    """Durations (ms) and kinds of the traced launches, in launch order."""
    ms = (ctypes.c_float * cap)()
    kinds = (ctypes.c_int32 * cap)()
    n = ctypes.c_int64()
    _check(lib().sgemm_trace_end(ms, kinds, cap, ctypes.byref(n)), "sgemm_trace_end")
    k = min(n.value, cap)
    return list(ms[:k]), list(kinds[:k]), n.value
