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


def test_step_stats():
    s = bench.step_stats([3.0, 1.0, 2.0, 4.0])
    assert s == {"median": 2.5, "mean": 2.5, "std": round(float((5 / 3) ** 0.5), 4), "min": 1.0,
                 "max": 4.0}
    assert bench.step_stats([7.0])["std"] == 0.0


class _Stream:
    def __init__(self):
        self.syncs = 0

    def synchronize(self):
        self.syncs += 1


def test_warm_up_runs_exactly_w_steps_when_given():
    n = []
    s = _Stream()
    assert bench.warm_up(lambda: n.append(1), 3, s) == 3
    assert len(n) == 3 and s.syncs == 1
    assert bench.warm_up(lambda: n.append(1), 0, s) == 0


def test_warm_up_default_runs_two_steps_and_the_minimum_time():
    import time
    n = []
    t0 = time.perf_counter()
    ran = bench.warm_up(lambda: (n.append(1), time.sleep(0.001)), None, _Stream())
    assert ran == len(n) >= 2
    assert time.perf_counter() - t0 >= bench.MIN_WARMUP_S
    slow = []
    assert bench.warm_up(lambda: (slow.append(1), time.sleep(0.6)), None, _Stream()) == 2


def test_traffic_only_for_the_counted_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("hbm_bytes_per_launch: 1234\nkernel_source_sha256_16: %s\n"
                 % bench.kernel_source_hash())
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(bench.DEFAULT_WORKLOAD) == 1234.0
    assert bench.measured_traffic("sgemm_256") is None
    assert bench.measured_traffic(bench.DEFAULT_WORKLOAD, "bf16") is None
    f.write_text("hbm_bytes_per_launch: 1234\nkernel_source_sha256_16: 0000000000000000\n")
    assert bench.measured_traffic(bench.DEFAULT_WORKLOAD) is None


def test_clock_sampler_reads_the_marked_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1900Mhz *\n2: 2400Mhz\n")
    c = bench.ClockSampler(period=0.01)
    c.paths = [str(f)]
    with c:
        import time
        time.sleep(0.05)
    s = c.summary()
    assert s["samples"] >= 1 and s["median_mhz"] == 1900.0 == s["min_mhz"] == s["max_mhz"]
    empty = bench.ClockSampler()
    empty.paths = []
    with empty:
        pass
    assert empty.summary() is None


def test_traffic_only_for_the_counted_tile(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("hbm_bytes_per_launch: 99\nkernel_config: 256x256x32x4x2\n"
                 "kernel_source_sha256_16: %s\n" % bench.kernel_source_hash())
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(bench.DEFAULT_WORKLOAD, config="256x256x32x4x2") == 99.0
    assert bench.measured_traffic(bench.DEFAULT_WORKLOAD, config="256x256x32x2x2") is None
    assert bench.measured_traffic(bench.DEFAULT_WORKLOAD) == 99.0
