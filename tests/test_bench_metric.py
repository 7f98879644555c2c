"""The benchmark's GFLOP/s convention against the figures the pages print."""
import os

import bench

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gflops_pages.txt")


def test_gflops_convention_matches_the_pages():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 4
    for name, M, N, K, ms, printed in rows:
        got = bench.gflops(int(M), int(N), int(K), float(ms))
        # times are printed to 0.01 ms: allow the rate that rounding implies
        assert abs(got - float(printed)) / float(printed) <= 0.005 / float(ms) + 1e-6, name


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert p.returncode == 2 and "one GPU" in p.stderr
