"""Compile the gfx950 SGEMM library in place (hipcc, no JIT, no torch extension).

    python -m fp32_gemm_02_amd.build
    python -m fp32_gemm_02_amd.build --sanitize DIR

writes fp32_gemm_02_amd/libphobos_sgemm.so next to this file (or, with
--sanitize, DIR/libphobos_sgemm.so with AddressSanitizer and
UndefinedBehaviorSanitizer in its host code, for CPU-only checks).  Each source is
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
           os.path.join(HERE, "csrc", "sgemm_splitk.hip"),
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


# The CPU-only check of the host code: AddressSanitizer and
# UndefinedBehaviorSanitizer on the host pass only (the device code is built
# as usual), the sanitizer runtime shared, to be preloaded into the process.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-shared-libasan", "-g",
                  "-fno-omit-frame-pointer"]


def asan_runtime():
    """Path of the compiler's shared AddressSanitizer runtime (None if absent)."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                         "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build_sanitized(out_dir, verbose=False):
    """The library with sanitized host code, as out_dir/libphobos_sgemm.so;
    load it with asan_runtime() preloaded (LD_PRELOAD) and PHOBOS_SGEMM_LIB
    pointing at it.  For CPU-only runs: no GPU work is meant to go through it."""
    os.makedirs(out_dir, exist_ok=True)
    rt = asan_runtime()
    if rt is None:
        raise RuntimeError("no shared AddressSanitizer runtime next to the compiler")
    # linked against the runtime (found through the rpath), so that a plain C
    # program can link the library too
    return build(extra_flags=SANITIZE_FLAGS, out=os.path.join(out_dir, "libphobos_sgemm.so"),
                 verbose=verbose,
                 link_flags=SANITIZE_FLAGS + ["-Wl,-rpath," + os.path.dirname(rt)])


def build(extra_flags=(), out=LIB, verbose=False, jobs=None, link_flags=()):
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
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_flags, *objs, "-o",
                tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, err = _run(link)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[1] == "--sanitize":
        print(build_sanitized(sys.argv[2], verbose=True))
    else:
        print(build(verbose=True))
