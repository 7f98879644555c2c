"""Compile the gfx950 SGEMM library in place (hipcc, no JIT, no torch extension).

    python -m fp32_gemm_02_amd.build

writes fp32_gemm_02_amd/libphobos_sgemm.so next to this file.  Each source is
compiled to an object of its own, in parallel, then the objects are linked.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libphobos_sgemm.so")
SOURCES = [os.path.join(HERE, "csrc", "sgemm_kernels.hip"),
           os.path.join(HERE, "csrc", "sgemm_tc.hip"),
           os.path.join(HERE, "csrc", "attention.hip"),
           os.path.join(HERE, "csrc", "sgemm_api.cpp"),
           os.path.join(HERE, "csrc", "sgemm_host.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 (v_pk_*_f32) instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# the host pass does not know the packed-fp32 feature name; that warning is noise
_NOISE = "is not a recognized feature for this target"


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in proc.stderr.splitlines() if _NOISE not in l)
    return proc.returncode, err


def build(extra_flags=(), out=LIB, verbose=False, jobs=None):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1), 8)
    with tempfile.TemporaryDirectory(prefix="phobos_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, *extra_flags, *inc, "-c", s, "-o", o]
                for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, err), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({rc}):\n{err}")
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        tmp = out + ".tmp"
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, err = _run(link)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
