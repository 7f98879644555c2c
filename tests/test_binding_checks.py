"""The Python binding's checks of its tensor arguments, the dispatch log and
the status of host-side failures, on the CPU (nothing reaches a GPU here:
every call below is refused, or returns, before the library launches)."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import fp32_gemm_02_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _f32(n):
    return torch.zeros(n, dtype=torch.float32)


GEMM_ENTRIES = {
    "sgemm": lambda A, B, C, M=8, N=8, K=8, ld=(8, 8, 8): g.sgemm(
        M, N, K, 1.0, A, ld[0], B, ld[1], 0.5, C, ld[2], stream=0),
    "sgemm_supertiled": lambda A, B, C, M=8, N=8, K=8, ld=(8, 8, 8): g.sgemm_supertiled(
        M, N, K, 1.0, A, ld[0], B, ld[1], 0.5, C, ld[2], 4, 4, 4, stream=0),
    "sgemm_tc": lambda A, B, C, M=8, N=8, K=8, ld=(8, 8, 8): g.sgemm_tc(
        M, N, K, 1.0, A, ld[0], B, ld[1], 0.5, C, ld[2], stream=0),
}


@pytest.mark.parametrize("entry", sorted(GEMM_ENTRIES))
def test_wrong_dtype_is_refused(entry):
    call = GEMM_ENTRIES[entry]
    good = _f32(64)
    for which in range(3):
        args = [good, good, good]
        args[which] = torch.zeros(64, dtype=torch.float64)
        with pytest.raises(ValueError, match="float32"):
            call(*args)
    with pytest.raises(ValueError, match="float32"):
        call(good, torch.zeros(64, dtype=torch.float16), good)


@pytest.mark.parametrize("entry", sorted(GEMM_ENTRIES))
def test_short_buffers_are_refused(entry):
    call = GEMM_ENTRIES[entry]
    full = _f32(10 * 16)
    # 8 x 8 with leading dimension 16 spans 7*16 + 8 = 120 floats
    for which, name in enumerate("ABC"):
        args = [full, full, full]
        args[which] = _f32(119)
        with pytest.raises(ValueError, match=f"{name} holds 119 floats.*spans 120"):
            call(*args, ld=(16, 16, 16))


@pytest.mark.parametrize("entry", sorted(GEMM_ENTRIES))
def test_host_tensors_are_refused(entry):
    call = GEMM_ENTRIES[entry]
    t = _f32(64)
    with pytest.raises(ValueError, match="not on a GPU"):
        call(t, t, t)


def test_strided_views_are_refused():
    t = _f32(256)[::2]
    with pytest.raises(ValueError, match="contiguous"):
        g.sgemm(8, 8, 8, 1.0, t, 8, t, 8, 0.0, t, 8, stream=0)


def test_unread_operands_are_not_sized():
    # alpha == 0 (or K == 0): A and B are not read, so empty tensors pass the
    # extent check for them and the first complaint is about C
    e = _f32(0)
    for alpha, K in ((0.0, 8), (1.0, 0)):
        with pytest.raises(ValueError, match="C holds 10 floats"):
            g.sgemm(8, 8, K, alpha, e, 8, e, 8, 0.5, _f32(10), 8, stream=0)
    with pytest.raises(ValueError, match="A holds 0 floats"):
        g.sgemm(8, 8, 8, 1.0, e, 8, e, 8, 0.5, _f32(10), 8, stream=0)


def test_init_leaf_and_attention_checks():
    with pytest.raises(ValueError, match="C holds 10 floats"):
        g.sgemm_init_leaf(4, 4, 0.5, _f32(10), 4, stream=0)
    q = _f32(4 * 64)
    with pytest.raises(ValueError, match="O holds"):
        g.flash_attention(4, 4, 64, q, 64, q, 64, q, 64, _f32(100), 64, 0.1, stream=0)
    with pytest.raises(ValueError, match="float32"):
        g.flash_attention_supertiled(4, 4, 64, q, 64, q.double(), 64, q, 64, q, 64, 0.1, 2,
                                     stream=0)
    with pytest.raises(ValueError, match="not on a GPU"):
        g.flash_attention(4, 4, 64, q, 64, q, 64, q, 64, q, 64, 0.1, stream=0)


def test_host_resident_operands_are_checked():
    plan = g.sgemm_plan()
    a = np.zeros(64, np.float32)
    with pytest.raises(ValueError, match="float32"):
        g.sgemm_supertiled_host(8, 8, 8, 1.0, a.astype(np.float64), 8, a, 8, 0.0, a, 8, plan,
                                stream=0)
    with pytest.raises(ValueError, match="B holds 63 floats"):
        g.sgemm_supertiled_host(8, 8, 8, 1.0, a, 8, a[:63], 8, 0.0, a, 8, plan, stream=0)
    with pytest.raises(ValueError, match="C holds"):
        g.sgemm_supertiled_host(8, 8, 8, 1.0, a, 8, a, 8, 0.0, torch.zeros(10), 8, plan, stream=0)


def test_integer_addresses_pass_unchecked():
    # raw addresses are the C ABI's business: its own argument checks answer
    assert g.sgemm_raw(4, 4, 5, 1.0, 8, 4, 8, 4, 0.0, 8, 4, stream=0) == -6
    assert g.sgemm_raw(0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, stream=0) == 0


# ---------------------------------------------------------------------------
# dispatch log

def test_set_log_reports_and_switches(capfd):
    was = g.sgemm_set_log(True)
    try:
        assert g.sgemm_set_log(True) is True
        assert g.sgemm_raw(4, 4, 0, 1.0, None, 4, None, 4, 1.0, 8, 4, stream=0) == 0
        assert g.sgemm_supertiled_raw(0, 8, 8, 1.0, None, 8, None, 8, 1.0, None, 8, 4, 4, 4,
                                      stream=0) == 0
        err = capfd.readouterr().err.splitlines()
        assert err == [
            "phobos_sgemm: sgemm M=4 N=4 K=0 alpha=1: A and B not read, C <- beta*C",
            "phobos_sgemm: init_leaf M=4 N=4 beta=1: identity, nothing enqueued",
            "phobos_sgemm: sgemm_supertiled M=0 N=8: empty, nothing enqueued",
        ]
        assert g.sgemm_set_log(False) is True
        assert g.sgemm_raw(4, 4, 0, 1.0, None, 4, None, 4, 1.0, 8, 4, stream=0) == 0
        assert capfd.readouterr().err == ""
    finally:
        g.sgemm_set_log(was)


def test_environment_turns_the_log_on():
    code = ("import fp32_gemm_02_amd as g\n"
            "assert g.sgemm_supertiled_raw(8, 8, 8, 0.0, None, 8, None, 8, 1.0, 8, 8, 4, 4, 4,"
            " stream=0) == 0\n")
    for value, on in (("1", True), ("0", False), ("", False)):
        env = dict(os.environ, SGEMM_LOG=value, PYTHONPATH=ROOT)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                           text=True, cwd=ROOT, timeout=120)
        assert r.returncode == 0, r.stderr
        lines = [l for l in r.stderr.splitlines() if l.startswith("phobos_sgemm:")]
        if on:
            assert lines[0] == ("phobos_sgemm: sgemm_supertiled M=8 N=8 K=8 super-tiles 4x4x4: "
                                "grid 2x2, 0 K steps each (A and B not read: init leaf only), "
                                "0 step launches")
            assert len(lines) == 5 and all("identity" in l for l in lines[1:])
        else:
            assert lines == []


def test_tune_reports_the_runtime_error():
    """sgemm_tune passes the HIP runtime's own error on (1000 + e, e != 0):
    without a GPU its first allocation fails with 'no device'."""
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the tune would run")
    st = g.lib().sgemm_tune(8, 8, 8, 8, 8, 8, 2, None, None, None)
    assert st > g.SGEMM_ERR_HIP_BASE, st
    assert g.status_string(st) not in ("no error", "hipSuccess", "success")
