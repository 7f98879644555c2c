"""Benchmark: super-tiled FP32 SGEMM, M = N = K = 16384, 4096^3 super-tiles, 1 GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--tune]

One step is one sgemm_supertiled call through the C ABI: argument checks,
the row-major walk over the 4 x 4 grid of output super-tiles, and per
super-tile the init leaf (a no-op launch-free identity at beta = 1) and four
step leaves of 4096^3 each (64 GEMM launches per step).  Inputs are seeded
synthetic uniform[-1, 1) matrices (the oracle's generators), resident in HBM
before the timed region.  Each timed step runs between its own pair of HIP
events, and before each step C is restored from a device copy of its initial
values, outside the events (beta = 1 would otherwise let it accumulate);
ms_per_step is the mean of the step times.  --warmup W runs exactly W
untimed steps first; without it, untimed steps run until at least 2 have run
and at least 1 s has passed (the count is reported).

Printed: one JSON line with the metric (GFLOP/s = 2*M*N*K / time per step),
the roofline of the dominant kernel (the step leaf; its duration per launch
from HIP events the library records on the launch stream during the timed
region, around one launch in 31) and the CPU oracle's rate on a bounded
slab of the same product.  The shader clock is sampled from the driver's
sysfs clock table by a host thread during the timed region.
The timed region records one more event after each step, so the config also
gives each step's median, mean, standard deviation, min and max (ms), and the
device with its HIP runtime; and the device's own FP32 matrix peak (compute units x
peak shader clock x 256 FLOP per clock per CU, from the HIP runtime) beside
the published 157.3 TFLOP/s.

Other options: --workload runs one of the other seeded workloads of
sgemm_workloads.py instead (one step = one sgemm call); --tune runs the tile
tuner on the step shape first (untimed) and times the winner;
--host-resident MIB keeps A, B and C in pinned host memory and times
sgemm_supertiled_host with the planner's plan for a device budget of MIB MiB
(a rate that includes every host<->device transfer; the workload's own
super-tile extents are replaced by the plan's); --tc f16|bf16 times the
matrix-core variant sgemm_tc (A and B rounded to that format, fp32
accumulation) as one monolithic call per step on the same inputs, its
cast pass included, with the roofline of its 16-bit GEMM kernel against the
16-bit matrix peak; --attention times the pages' second example, attention
over 16384 queries and keys with D = 64 (the pages' job), as one call of its
cluster form (super-tiles of 4096 query rows) per step.  For profiling
runs: --copy-calibration runs one plain device copy of 1 GiB first (a
known-size reference for the HBM byte counters); --skip-cpu-baseline leaves
the oracle leg out.
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_MFMA_TFLOPS = 157.3     # MI355X published dense FP32 matrix peak
FP32_MFMA_FLOP_PER_CLK_PER_CU = 256
# hipDeviceAttribute_t values of the HIP runtime's header
HIP_ATTR_CLOCK_RATE_KHZ = 5
HIP_ATTR_MULTIPROCESSOR_COUNT = 63
PEAK_HBM_GBS = 8000.0             # MI355X published HBM3E bandwidth
PEAK_F16_MFMA_TFLOPS = 2500.0     # MI355X published dense fp16 / bf16 matrix peak
DEFAULT_WORKLOAD = "supertiled_16384_t4096"
TRACE_EVERY = 31
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sgemm_step_4096_ld16384.txt")
TC_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tc16_gemm_f16_16384_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "fp32_gemm_02_amd", "csrc", f)
                  for f in ("sgemm_kernels.hip", "sgemm_device.h")]
TC_KERNEL_SOURCES = [os.path.join(ROOT, "fp32_gemm_02_amd", "csrc", f)
                     for f in ("sgemm_tc.hip", "sgemm_device.h")]


def gflops(M, N, K, ms):
    """The pages' convention: 2*M*N*K floating-point operations per product."""
    return 2.0 * M * N * K / (ms * 1e-3) / 1e9


def device_fp32_matrix_peak(device=0):
    """The FP32 matrix peak of this device from its own figures: compute units
    x peak shader clock x 256 FLOP per clock per CU, as the HIP runtime
    reports them; None if it cannot be asked."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    vals = []
    for attr in (HIP_ATTR_MULTIPROCESSOR_COUNT, HIP_ATTR_CLOCK_RATE_KHZ):
        v = ctypes.c_int()
        if hip.hipDeviceGetAttribute(ctypes.byref(v), ctypes.c_int(attr), ctypes.c_int(device)) != 0:
            return None
        vals.append(v.value)
    cus, khz = vals
    return {"cus": cus, "max_sclk_mhz": khz / 1e3,
            "tflops": round(cus * khz * 1e3 * FP32_MFMA_FLOP_PER_CLK_PER_CU / 1e12, 2)}


MIN_WARMUP_S = 1.0


def warm_up(step, warmup, stream):
    """Untimed steps before the timed region: exactly `warmup` when it is
    given; otherwise at least 2 steps and at least MIN_WARMUP_S seconds of them
    (each waited for).  The shader clock rises over hundreds of ms of load:
    after 0.15 s of the unaligned 5003x3001x2047 product the clock sampled
    during the timed steps was still about 2.0 GHz of its 2.4.
    Returns the number of steps run."""
    if warmup is not None:
        for _ in range(warmup):
            step()
        stream.synchronize()
        return warmup
    n, t0 = 0, time.perf_counter()
    while n < 2 or (time.perf_counter() - t0 < MIN_WARMUP_S and n < 100000):
        step()
        stream.synchronize()
        n += 1
    return n


def timed_steps(step, steps, stream, restore=None):
    """Run `steps` steps, each between a HIP event pair of its own on
    `stream`; `restore` (when given) runs before every step, outside the
    pairs, to put C back to its initial values.  Returns the sum of the step
    times (ms), each step's time (ms) and the host wall time of the whole
    loop (s)."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if restore is not None:
            restore()
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [starts[i].elapsed_time(ends[i]) for i in range(steps)]
    return float(sum(per_step)), per_step, wall


class ClockSampler:
    """The shader clock during the timed region, sampled by a host thread from
    the driver's sysfs table of shader clock levels (the line marked '*' is
    the level the GPU runs at) every `period` seconds.  Reading a sysfs file
    puts no work on the GPU.  summary() is None when the table is absent."""

    def __init__(self, period=0.05):
        import glob
        import threading
        self.period = period
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for path in self.paths:
            try:
                for line in open(path):
                    if "*" in line:
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        if m:
                            return int(m.group(1))
            except OSError:
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.paths:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        import numpy as np
        v = np.asarray(self.samples, dtype=np.float64)
        return {"source": "sysfs pp_dpm_sclk, current level", "samples": int(v.size),
                "median_mhz": float(np.median(v)), "min_mhz": float(v.min()),
                "max_mhz": float(v.max())}


def step_stats(per_step):
    """Median, mean, standard deviation, min and max of the per-step times (ms)."""
    import numpy as np
    v = np.asarray(per_step, dtype=np.float64)
    return {"median": round(float(np.median(v)), 4), "mean": round(float(v.mean()), 4),
            "std": round(float(v.std(ddof=1)) if v.size > 1 else 0.0, 4),
            "min": round(float(v.min()), 4), "max": round(float(v.max()), 4)}


def device_info(device=0):
    import torch
    props = torch.cuda.get_device_properties(device)
    return {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
            "hip_runtime": torch.version.hip}


def kernel_source_hash(sources=None):
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, tc=None, config=None):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel source for this workload
    (the fp32 step leaf of the default workload, or the fp16 GEMM of the
    matrix-core variant) and, when `config` (e.g. "256x256x32x4x2") is given
    and the summary names its tile, on that tile; else None."""
    if workload != DEFAULT_WORKLOAD:
        return None
    if tc is None:
        path, sources = TRAFFIC_FILE, KERNEL_SOURCES
    elif tc == "f16":
        path, sources = TC_TRAFFIC_FILE, TC_KERNEL_SOURCES
    else:
        return None
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"^kernel_source_sha256_16:\s*(\S+)", text, re.M)
    m_bytes = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    m_cfg = re.search(r"^kernel_config:\s*(\S+)", text, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(sources):
        return None
    if config is not None and m_cfg is not None and m_cfg.group(1) != config:
        return None
    return float(m_bytes.group(1))


def cpu_baseline(x, w, target_s=15.0, fmt=None):
    """The oracle as it stands, on a slab of rows of the same product (fmt:
    the oracle of the matrix-core variant)."""
    import oracle

    orc = oracle.default()
    threads = orc.max_threads()

    def run(rows):
        t0 = time.perf_counter()
        orc.sgemm(rows, w.N, w.K, w.alpha, x.A, x.B, w.beta, x.C, lda=w.lda, ldb=w.ldb,
                  ldc=w.ldc, fmt=fmt)
        return time.perf_counter() - t0

    # two probes give the per-row time and any fixed cost (the variant's
    # oracle rounds all of B first); the sample is sized from both
    r1 = max(8, threads)
    t1 = run(r1)
    r2 = min(w.M, 4 * r1)
    t2 = run(r2)
    per_row = max((t2 - t1) / max(r2 - r1, 1), 1e-6)
    fixed = max(t1 - per_row * r1, 0.0)
    rows = int(min(w.M, max(r1, (target_s - fixed) / per_row)))
    rows = max(threads, rows - rows % max(1, threads))
    t = run(rows)
    return {
        "value": round(gflops(rows, w.N, w.K, t * 1e3), 3),
        "unit": "GFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of the {w.M}x{w.N}x{w.K} product "
                  f"({rows}x{w.N}x{w.K}, {t:.1f} s, fp64 accumulation and bound"
                  + (", inputs rounded to the 16-bit format" if fmt else "") + ")",
    }


def attention_flops(Nq, Nk, D):
    """Two products of 2*Nq*Nk*D flops each (the softmax is not counted)."""
    return 4.0 * Nq * Nk * D


def cpu_baseline_attention(x, w, target_s=15.0):
    """The attention oracle as it stands, on a block of query rows."""
    import numpy as np

    import oracle

    orc = oracle.default()
    threads = orc.max_threads()

    def run(rows):
        t0 = time.perf_counter()
        orc.attention(w.Nq, w.Nk, w.D, x.Q, x.K, x.V, w.scale, rows=np.arange(rows),
                      ldq=w.ldq, ldk=w.ldk, ldv=w.ldv)
        return time.perf_counter() - t0

    r1 = max(8, threads)
    t1 = run(r1)
    rows = int(min(w.Nq, max(r1, r1 * target_s / max(t1, 1e-3))))
    rows = max(threads, rows - rows % max(1, threads))
    t = run(rows)
    return {
        "value": round(attention_flops(rows, w.Nk, w.D) / t / 1e9, 3),
        "unit": "GFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"query rows 0..{rows - 1} of the {w.Nq}x{w.Nk}, D={w.D} attention "
                  f"({t:.1f} s, fp64, bound included)",
    }


def main_attention(args):
    import numpy as np
    import torch

    import fp32_gemm_02_amd as g
    import sgemm_workloads as wl

    w = wl.ATTN_16384
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    x = wl.make_attn_inputs(w)
    with torch.cuda.stream(stream):
        dQ, dK, dV, dO = (torch.from_numpy(b).to(dev) for b in (x.Q, x.K, x.V, x.O))
    stream.synchronize()

    def step():
        g.flash_attention_supertiled(w.Nq, w.Nk, w.D, dQ, w.ldq, dK, w.ldk, dV, w.ldv, dO, w.ldo,
                                     w.scale, w.BR, stream=stream)

    args.warmup = warm_up(step, args.warmup, stream)
    g.sgemm_trace_begin(args.steps + 16)
    with ClockSampler() as clock:
        ms_total, per_step, _ = timed_steps(step, args.steps, stream)
    ms_kern, kinds, n = g.sgemm_trace_end(cap=args.steps + 16)
    launch_ms = float(np.mean([t for t, k in zip(ms_kern, kinds) if k == g.SGEMM_KIND_ATTENTION]))
    ms_per_step = ms_total / args.steps
    flops = attention_flops(w.Nq, w.Nk, w.D)
    value = flops / (ms_per_step * 1e-3) / 1e9
    achieved = flops / (launch_ms * 1e-3) / 1e12
    out = {
        "metric": "attention GFLOP/s (2 products of 2*Nq*Nk*D) at Nq = Nk = 16384, D = 64, 1 GPU",
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "entry": "flash_attention_supertiled", "Nq": w.Nq,
                   "Nk": w.Nk, "D": w.D, "scale": w.scale, "BR": w.BR,
                   "inputs": "Q/K/V %s/%s/%s, seed %d" % (*w.dists, w.seed),
                   "launches_per_step": 1,
                   "sclk_during_timed_region": clock.summary(),
                   "pct_of_fp32_matrix_peak": round(100.0 * value / 1e3 / PEAK_FP32_MFMA_TFLOPS, 2),
                   "step_ms": step_stats(per_step), "device": device_info()},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4), "traffic": None},
    }
    if not args.skip_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_attention(x, w)
    print(f"# timed {args.steps} steps: {ms_total:.2f} ms on the stream; {n} launches traced, "
          f"mean {launch_ms:.4f} ms", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: at least 2 and at least 1 s)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--tune", action="store_true")
    ap.add_argument("--host-resident", type=int, default=None, metavar="MIB")
    ap.add_argument("--tc", choices=("f16", "bf16"), default=None)
    ap.add_argument("--attention", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the super-tile grid of this workload is one "
              "GPU's share, and no multi-GPU path is built (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    if args.attention:
        main_attention(args)
        return

    import numpy as np
    import torch

    import fp32_gemm_02_amd as g
    import sgemm_workloads as wl

    if args.workload not in wl.BY_NAME:
        print(f"unknown workload {args.workload!r}; choose from {sorted(wl.BY_NAME)}",
              file=sys.stderr)
        sys.exit(2)
    w = wl.BY_NAME[args.workload]
    supertiled = w.entry == "sgemm_supertiled"
    host = args.host_resident is not None
    tc = {"f16": g.SGEMM_TC_F16, "bf16": g.SGEMM_TC_BF16}.get(args.tc)
    if tc is not None:
        if host:
            print("--tc and --host-resident do not combine", file=sys.stderr)
            sys.exit(2)
        supertiled = False   # one monolithic sgemm_tc call per step
    plan = None
    if host:
        if not supertiled:
            print("--host-resident needs a super-tiled workload", file=sys.stderr)
            sys.exit(2)
        plan = g.sgemm_plan_supertiles(w.M, w.N, w.K, w.beta, args.host_resident << 20)
        tiles = (min(plan.TM, w.M), min(plan.TN, w.N), min(plan.TK, w.K))
    else:
        tiles = (w.TM, w.TN, w.TK) if supertiled else None
    # the GEMM launches of one step: one per super-tile and K chunk, else one
    step_shape = tiles if supertiled else (w.M, w.N, w.K)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)

    x = wl.make_inputs(w)
    with torch.cuda.stream(stream):
        if host:
            # pinned host buffers (freshly allocated, then filled)
            dA, dB, dC = (torch.from_numpy(a).pin_memory() for a in (x.A, x.B, x.C))
        else:
            dA = torch.from_numpy(x.A).to(dev, non_blocking=False)
            dB = torch.from_numpy(x.B).to(dev, non_blocking=False)
            dC = torch.from_numpy(x.C).to(dev, non_blocking=False)
        if args.copy_calibration:
            src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
            dst = torch.empty_like(src)
            dst.copy_(src)
            del src, dst
    stream.synchronize()

    def step():
        if tc is not None:
            g.sgemm_tc(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc, fmt=tc,
                       stream=stream)
        elif host:
            g.sgemm_supertiled_host(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC,
                                    w.ldc, plan, stream=stream)
        elif supertiled:
            g.sgemm_supertiled(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC,
                               w.ldc, w.TM, w.TN, w.TK, stream=stream)
        else:
            g.sgemm(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc,
                    stream=stream)

    restore = None
    if w.beta != 0:
        # every timed step starts from the initial C (restored outside the
        # step's events); the copy lives on the device, or in host memory for
        # the host-resident form.  It is made before the warm-up: a step that
        # followed the 1 GiB allocation at once ran 2% slower than the rest.
        with torch.cuda.stream(stream):
            c0 = dC.clone()
        stream.synchronize()

        def restore():
            with torch.cuda.stream(stream):
                dC.copy_(c0, non_blocking=not host)

    tuned = None
    if args.tune and tc is None:
        tuned, _ = g.sgemm_tune(*step_shape, w.lda, w.ldb, w.ldc, reps=10, stream=stream)

    args.warmup = warm_up(step, args.warmup, stream)

    if supertiled:
        launches_per_step = (-(-w.M // tiles[0])) * (-(-w.N // tiles[1])) * (-(-w.K // tiles[2]))
    elif tc is not None:
        launches_per_step = 1 + g.sgemm_tc_get_config(tc, w.M, w.N, w.K).staged   # cast pass
    else:
        launches_per_step = 1
    # A pair of the library's trace events around a launch costs the stream
    # about 4.5 us (timing-only events, no system-scope fence); on the 64
    # launches of a super-tiled step, tracing each costs 0.5% of the step and
    # one in seven 0.1%.  The launches of such a step are all alike, so one in
    # TRACE_EVERY is traced (31, prime to the 4 K steps of a super-tile, so
    # every K position is sampled: 41 launches over 20 steps); steps of a few
    # unlike launches (the 16-bit form's cast pass and GEMM) trace all.
    every = TRACE_EVERY if launches_per_step >= 16 else 1
    # a step of one launch is timed by the step's own event pair, so the
    # library traces nothing then (a second pair per launch would only add
    # stream time)
    single = launches_per_step == 1 and tc is None and not host
    cap = args.steps * launches_per_step * 2 + 16
    if not single:
        g.sgemm_trace_begin(cap, every=every)
    with ClockSampler() as clock:
        ms_total, per_step, wall = timed_steps(step, args.steps, stream, restore)
    if not single:
        ms_kern, kinds, n = g.sgemm_trace_end(cap=cap)
    else:
        ms_kern, kinds = per_step, [g.SGEMM_KIND_GEMM] * len(per_step)
    ms_per_step = ms_total / args.steps
    value = gflops(w.M, w.N, w.K, ms_per_step)

    dominant = g.SGEMM_KIND_TC if tc is not None else g.SGEMM_KIND_GEMM
    step_ms = [t for t, k in zip(ms_kern, kinds) if k == dominant]
    cast_ms = [t for t, k in zip(ms_kern, kinds) if k == g.SGEMM_KIND_TC_CAST]
    avg_launch_ms = float(np.mean(step_ms))
    step_flops = 2.0 * step_shape[0] * step_shape[1] * step_shape[2]
    achieved_tflops = step_flops / (avg_launch_ms * 1e-3) / 1e12
    kcfg = (g.sgemm_tc_get_config(tc, w.M, w.N, w.K).as_tuple()[:5] if tc is not None else
            g.sgemm_get_config(*step_shape, w.lda, w.ldb, w.ldc).as_tuple())
    traffic = None if host else measured_traffic(args.workload, args.tc,
                                                 "x".join(str(v) for v in kcfg))
    peak = PEAK_FP32_MFMA_TFLOPS if tc is None else PEAK_F16_MFMA_TFLOPS

    dev_peak = device_fp32_matrix_peak() if tc is None else None
    out = {
        "metric": "SGEMM GFLOP/s and % of MI355X FP32 matrix peak at 16384^3, 1 GPU",
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": (f"tc_{args.tc}_{w.M}" if tc is not None else
                                w.name + ("_host_resident" if host else "")),
                   "entry": ("sgemm_tc" if tc is not None else
                             "sgemm_supertiled_host" if host else w.entry),
                   "M": w.M, "N": w.N, "K": w.K,
                   "lda": w.lda, "ldb": w.ldb, "ldc": w.ldc,
                   **(dict(zip(("TM", "TN", "TK"), tiles)) if supertiled else {}),
                   **({"device_budget_mib": args.host_resident,
                       "slots_a_b_c": [plan.a_slots, plan.b_slots, plan.c_slots],
                       "walk": {g.SGEMM_WALK_ROWS: "rows", g.SGEMM_WALK_SHELLS: "shells",
                                g.SGEMM_WALK_BLOCKS: "blocks"}[plan.walk],
                       "planned_transfer_bytes": plan.transfer_bytes,
                       "modeled_ms": round(plan.modeled_ms, 3),
                       "inputs_in": "pinned host memory (rate includes all transfers)"}
                      if host else {}),
                   "alpha": w.alpha, "beta": w.beta,
                   "inputs": "A/B/C %s/%s/%s, seed %d" % (*w.dists, w.seed),
                   "leaf_config": (
                       "bm=%d bn=%d bk=%d wm=%d wn=%d staged=%d" %
                       g.sgemm_tc_get_config(tc, w.M, w.N, w.K).as_tuple() if tc is not None else
                       "bm=%d bn=%d bk=%d wm=%d wn=%d" %
                       g.sgemm_get_config(*step_shape, w.lda, w.ldb, w.ldc).as_tuple()),
                   "tuned": tuned is not None,
                   "c_restored_each_step": restore is not None,
                   "traced_launches": ({"every": every, "count": len(step_ms)} if not single
                                       else "the step's own event pair (one launch per step)"),
                   "sclk_during_timed_region": clock.summary(),
                   "step_ms": step_stats(per_step),
                   "device": device_info(),
                   "launches_per_step": launches_per_step,
                   **({"cast_pass_ms": round(float(np.mean(cast_ms)), 4) if cast_ms else 0.0,
                       "gemm_ms": round(avg_launch_ms, 4),
                       "inputs_rounded_to": args.tc,
                       "pct_of_f16_matrix_peak": round(100.0 * value / 1e3 / PEAK_F16_MFMA_TFLOPS, 2)}
                      if tc is not None else
                      {"pct_of_fp32_matrix_peak": round(100.0 * value / 1e3 / PEAK_FP32_MFMA_TFLOPS, 2),
                       **({"device_fp32_matrix_peak": dev_peak,
                           "pct_of_device_fp32_matrix_peak":
                               round(100.0 * value / 1e3 / dev_peak["tflops"], 2)}
                          if dev_peak else {})})},
        "roofline": {"bound": "mfma", "achieved": round(achieved_tflops, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / peak, 4),
                     "traffic": traffic},
    }
    if tc is not None:
        out["metric"] = ("SGEMM GFLOP/s of the matrix-core variant (inputs rounded to %s, fp32 "
                         "accumulation) at %d^3, 1 GPU" % (args.tc, w.M))
        out["dtype"] = args.tc
    if not args.skip_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, w, fmt=tc)
    if tuned is not None:
        g.sgemm_set_config(None)
    traced = (f"{len(step_ms)} step-leaf launches traced (one in {every})" if not single else
              f"{len(step_ms)} launches timed by their step's events")
    print(f"# timed {args.steps} steps: {ms_total:.2f} ms on the stream ({wall * 1e3:.2f} ms "
          f"wall, C restores included); {traced}, mean {avg_launch_ms:.4f} ms", file=sys.stderr,
          flush=True)
    print("# step times (ms): " + " ".join(f"{t:.3f}" for t in per_step), file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
