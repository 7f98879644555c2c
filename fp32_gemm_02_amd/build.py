"""Compile the gfx950 SGEMM library in place (hipcc, no JIT, no torch extension).

    python -m fp32_gemm_02_amd.build

writes fp32_gemm_02_amd/libphobos_sgemm.so next to this file.
"""
import os
import subprocess
import sys

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
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 (v_pk_*_f32) instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(extra_flags=(), out=LIB, verbose=False):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name; that warning is noise
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
