"""Benchmark of the fused MXFP4 quant + a4w4 GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one gemm_a4w4_fused call (dynamic quantisation of A, the
block-scaled FP4 GEMM, bf16 store) on one batch of synthetic input; B is
quantised and packed once beforehand (offline, untimed). Inputs are resident in
HBM before the timed region.

By default the line's headline is the largest configuration the metric spans,
square M=N=4096 K=7168 (MFMA-bound: TFLOP/s against the dense MXFP4 peak), and
the other configurations (skinny, stress, tiny, grouped) ride on the same line
under "workloads", each timed the same way. --workload NAME times one workload.

Timing: W untimed warm-up steps; the K steps are captured once in a HIP graph,
replayed once untimed, and replayed again between two HIP events on the
launching stream. Cold runs (the default) rotate through enough distinct
operand sets (A, packed B, C) to exceed 512 MB, whatever K is, and read 512 MB
of another buffer just before the timed replay, so that no operand is left in
the 256 MB Infinity Cache by the untimed runs. Prints ONE JSON line.

The CPU oracle is timed beside it (the cpu_baseline leg) on a bounded sample of
the headline workload, its BLAS on the CPUs this process may use (capped by
OMP_NUM_THREADS when set).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
FP4_PEAK_TFLOPS = 10100.0   # MI355X dense MXFP4 matrix peak, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, TFLOP/s (the NVFP4 path's instruction)
METRIC = "µs/call, TFLOP/s and HBM GB/s (% of peak) for quant+a4w4 GEMM, M=16..4096"
ROTATE_BYTES = 512 << 20
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["mxfp4_block_scaled_02_amd/csrc/gemm.hip", "mxfp4_block_scaled_02_amd/csrc/mx_device.hpp",
                  "mxfp4_block_scaled_02_amd/csrc/host_common.hpp"]
RMS_SOURCES = ["mxfp4_block_scaled_02_amd/csrc/rmsnorm_quant.hip", "mxfp4_block_scaled_02_amd/csrc/mx_device.hpp",
               "mxfp4_block_scaled_02_amd/csrc/host_common.hpp"]
NV_SOURCES = ["mxfp4_block_scaled_02_amd/csrc/nvfp4.hip", "mxfp4_block_scaled_02_amd/csrc/host_common.hpp"]
COPY_BYTES = 256 << 20  # plain device copy used to calibrate the FETCH_SIZE / WRITE_SIZE counters


def alg_bytes(M, N, K):
    """A bf16 read once + B codes + B scales + C bf16 written once (the quantised A is never stored)."""
    return 2 * M * K + N * K // 2 + N * K // 32 + 2 * M * N


def alg_flops(M, N, K):
    return 2 * M * N * K


WORKLOADS = ["tiny", "skinny", "stress", "square", "grouped", "grouped_decode", "mid", "rmsnorm", "grouped_mnk",
             "skinny_shard8", "nvfp4_grouped"]
HEADLINE = "square"                       # the largest single-GPU configuration the metric spans
EXTRAS = ["skinny", "stress", "tiny", "grouped", "grouped_decode", "mid"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=None, choices=WORKLOADS,
                   help="time one workload only (default: the square headline plus skinny, stress, tiny, grouped, "
                        "grouped_decode and mid "
                        "as extra keys of the same line). rmsnorm times mxfp4_rmsnorm_quant at M4096 K7168; "
                        "grouped_mnk times grouped_gemm_a4w4_mnk on seeded groups with their own (M, N, K, L)")
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--sustained-steps", type=int, default=200,
                   help="default run: also time the headline over one replay of this many calls (the sustained "
                        "rate, after the power manager has settled; 0 skips it)")
    p.add_argument("--warm-cache", action="store_true", help="reuse one operand set (Infinity Cache resident)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="time an eager launch loop instead of a graph replay")
    p.add_argument("--unfused", action="store_true",
                   help="time the two-launch comparator instead: mxfp4_quant(A), then gemm_a4w4 on A_q")
    p.add_argument("--no-library", action="store_true",
                   help="default run: skip timing the library MXFP4 GEMM (torch._scaled_mm) on the headline")
    p.add_argument("--library", action="store_true",
                   help="with --workload (a single GEMM): also time the library MXFP4 GEMM on the same operands")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run plain device copies of a known size (counter calibration)")
    p.add_argument("--summarize-stats", metavar="DIR", help="print a summary of rocprofv3 --kernel-trace CSV output")
    p.add_argument("--select", default=None, metavar="A:B",
                   help="with --summarize-stats: only dispatches A..B-1 (in start order) of each kernel and grid; "
                        "a default bench run gives each workload's kernel W warm-up calls, the untimed replay of "
                        "K calls and the timed replay of K calls, so its timed calls are W+K:W+2K")
    p.add_argument("--summarize-pmc", nargs=3, metavar=("WORKLOAD_DIR", "COPY_DIR", "KERNEL"),
                   help="turn FETCH_SIZE/WRITE_SIZE runs into the traffic record for KERNEL")
    p.add_argument("--summarize-counters", nargs=2, metavar=("DIR", "KERNEL"),
                   help="per-dispatch averages of every counter collected for KERNEL, and the MFMA busy fraction")
    return p.parse_args()


def kernel_source_hash(sources=KERNEL_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def sources_for(name):
    """Source files whose hash keys the counter record of a workload or kernel name."""
    if "rmsnorm" in name:
        return RMS_SOURCES
    if "nvfp4" in name:
        return NV_SOURCES
    return KERNEL_SOURCES


def recorded_traffic(name):
    """HBM bytes per launch from the committed counter record, or None if the kernel changed since."""
    path = os.path.join(PROFILES, f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(sources_for(name)):
        return None
    return rec.get("bytes_per_launch")


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def summarize_stats(directory, select=None):
    """Per-kernel table from a rocprofv3 --kernel-trace run: one row per kernel and grid size (the split-K
    kernel serves tiny and skinny with one instance), with the calls, the mean, the 10th / 50th / 90th
    percentile, min and max of the per-dispatch durations, and the share of the total kernel time. With
    `select` ("A:B"), only dispatches A..B-1 (by start time) of each kernel and grid count."""
    durs = {}
    rows = sorted(_csv_rows(directory, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        wgs = 1
        for ax in "XYZ":
            wgs *= max(1, int(r[f"Grid_Size_{ax}"]) // max(1, int(r[f"Workgroup_Size_{ax}"])))
        durs.setdefault((r["Kernel_Name"], wgs), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if select:
        a, b = (int(x) if x else None for x in select.split(":"))
        durs = {k: d[a:b] for k, d in durs.items() if d[a:b]}
    total = sum(sum(d) for d in durs.values()) or 1.0
    print("| kernel | workgroups | calls | avg µs | p10 µs | median µs | p90 µs | min µs | max µs | share % |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for (name, wgs), d in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        p10, p50, p90 = np.percentile(d, [10, 50, 90])
        print(f"| {name[:90]} | {wgs} | {len(d)} | {np.mean(d):.3f} | {p10:.3f} | {p50:.3f} | {p90:.3f} | "
              f"{min(d):.3f} | {max(d):.3f} | {100 * sum(d) / total:.1f} |")


def summarize_pmc(workload_dir, copy_dir, kernel):
    """KiB per dispatch of FETCH_SIZE and WRITE_SIZE for KERNEL, scaled by the copy calibration."""
    def per_dispatch(directory, match):
        vals = {}
        for r in _csv_rows(directory, "counter_collection.csv"):
            if match in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}
    kv, kn = per_dispatch(workload_dir, kernel)
    cv, cn = per_dispatch(copy_dir, "copy")  # torch's device copy kernel
    expected_kib = COPY_BYTES / 1024
    out = {"kernel": kernel, "kernel_source_hash": kernel_source_hash(sources_for(kernel)),
           "copy_bytes": COPY_BYTES}
    total = 0.0
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        factor = expected_kib / cv[c] if cv.get(c) else None
        out[c] = {"kib_per_dispatch": kv.get(c), "dispatches": kn.get(c), "copy_kib": cv.get(c),
                  "copy_factor": factor}
        if kv.get(c) is not None and factor:
            total += kv[c] * factor * 1024
    out["bytes_per_launch"] = round(total)
    print(json.dumps(out, indent=1))


def summarize_counters(directory, kernel):
    """Per-dispatch averages of the counters of one rocprofv3 --pmc run. The MFMA busy
    fraction is SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs) over the kernel's
    cycles, GRBM_GUI_ACTIVE (summed over the 8 XCDs) / 8, times 1024."""
    vals = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if kernel in r["Kernel_Name"]:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = {k: {"per_dispatch": sum(v) / len(v), "dispatches": len(v)} for k, v in sorted(vals.items())}
    busy, active = vals.get("SQ_VALU_MFMA_BUSY_CYCLES"), vals.get("GRBM_GUI_ACTIVE")
    if busy and active:
        cycles = (sum(active) / len(active)) / 8
        out["mfma_busy_fraction"] = (sum(busy) / len(busy)) / (1024 * cycles)
        out["kernel_cycles"] = cycles
    print(json.dumps(out, indent=1))


def env_info():
    """What the run was on (best effort; a field that cannot be read is left out)."""
    import torch
    env = {}
    try:
        props = torch.cuda.get_device_properties(0)
        env.update(gpu=props.name, compute_units=props.multi_processor_count,
                   hbm_gib=round(props.total_memory / 2**30, 1))
    except Exception:
        pass
    env.update(torch=torch.__version__, hip=getattr(torch.version, "hip", None))
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        pass
    smi = smi_info()
    if smi:
        env["smi"] = smi
    return env


def smi_info():
    """Memory clock and package power cap of the GPU the run used, read from the amdgpu driver's sysfs files
    (plain file reads: no child process is started, since a child of a profiled process would inherit the
    profiler's preloaded library). The card is matched by PCI bus number. Best effort: None when the files
    are absent or no card matches. The shader clock read after the work would be the idle one and is not
    recorded."""
    import glob
    import torch
    try:
        bus = torch.cuda.get_device_properties(0).pci_bus_id
    except Exception:
        return None
    for dev in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        try:
            pci = os.path.basename(os.path.realpath(dev))  # e.g. 0000:a4:00.0
            if int(pci.split(":")[1], 16) != bus:
                continue
        except (ValueError, IndexError):
            continue
        out = {"card": os.path.basename(os.path.dirname(dev)), "pci": pci}
        try:
            with open(os.path.join(dev, "pp_dpm_mclk")) as f:
                for line in f:
                    if "*" in line:
                        out["mclk_mhz"] = float(line.split(":")[1].lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            pass
        for cap in glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_cap")):
            try:
                with open(cap) as f:
                    out["power_cap_w"] = int(f.read().strip()) / 1e6
            except (OSError, ValueError):
                pass
        return out
    return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def host_threads():
    """Threads for the oracle's BLAS: the CPUs this process may run on, capped by OMP_NUM_THREADS when the
    environment sets it (the share of a shared host this job is given). Returns (threads, affinity CPUs)."""
    aff = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    n = min(aff, int(cap)) if cap.isdigit() and int(cap) > 0 else aff
    return n, aff


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def time_oracle(fn, budget_s=12.0, max_runs=50):
    """Median wall time of fn() over at least 3 runs (1 if a run exceeds 60 s), within about budget_s,
    with the BLAS thread pool set to host_threads() (numpy's fp64 matmul is the only threaded step)."""
    from threadpoolctl import threadpool_limits
    n, aff = host_threads()
    times = []
    with threadpool_limits(limits=n):
        t_end = time.perf_counter() + budget_s
        while True:
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
            if times[-1] > 60 or (len(times) >= 3 and time.perf_counter() > t_end) or len(times) >= max_runs:
                break
    return float(np.median(times)), len(times), n, aff


def cpu_baseline(w, unit):
    """Time the oracle (untuned) on a bounded sample of the workload, scaled to the metric's unit."""
    import oracle
    from mxfp4_block_scaled_02_amd import synth
    name = w["name"]
    if name in synth.GROUPED:
        a, b = w["A"][0], w["B"][0]
    else:
        a, b = w["A"], w["B"]
    M, K = a.shape
    N = b.shape[0]
    bq, bs = oracle.quant_mx(b)  # B's quantisation is offline for the GPU too: excluded
    rows = np.arange(min(M, 64))
    t, runs, n, aff = time_oracle(lambda: oracle.gemm_ref(a[rows], bq, bs))
    m = len(rows)
    value = alg_flops(m, N, K) / t / 1e12 if unit == "TFLOP/s" else alg_bytes(m, N, K) / t / 1e9
    return dict(value=round(value, 6), unit=unit, cores=n, kind="oracle",
                sample=f"oracle gemm_ref (quant A, dequant A and B, fp64 matmul, bf16 round) on rows 0..{m - 1} of "
                       f"{'group 0' if name in synth.GROUPED else 'A'} against the full B (N={N}, K={K}); median of "
                       f"{runs} runs, {t * 1e3:.1f} ms each; numpy's BLAS on {n} threads, the rest single-threaded",
                affinity_cpus=aff, cpu_model=cpu_model())


_evict = None


def evict_infinity_cache():
    """Read 512 MB (twice the 256 MB Infinity Cache) so no operand stays cached from the untimed runs."""
    import torch
    global _evict
    if _evict is None:
        _evict = torch.ones(ROTATE_BYTES // 4, dtype=torch.int32, device="cuda")
    _evict.sum()


def n_sets(args, set_bytes):
    """Operand sets to rotate through: one (warm) or enough to exceed ROTATE_BYTES (never capped by --steps)."""
    return 1 if args.warm_cache else max(1, math.ceil(ROTATE_BYTES / set_bytes))


def cache_label(args, R, set_bytes):
    if R == 1:
        return "warm (1 operand set, reused)"
    return (f"cold ({R} rotated operand sets, {R * set_bytes / 1e6:.0f} MB; Infinity Cache evicted by a 512 MB "
            f"read before the timed replay)")


def timed_steps(step, args):
    """W untimed warm-up steps; the K steps captured in one HIP graph (an eager loop with --no-graph) and
    replayed once untimed; then (cold runs) the Infinity Cache evicted; then the K steps replayed between
    two HIP events on the launching stream. Returns ms per step."""
    import torch
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.no_graph:
        runner = lambda: [step(i) for i in range(args.steps)]  # noqa: E731
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.steps):
                step(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        runner = g.replay
    if not args.warm_cache:
        evict_infinity_cache()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    runner()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / args.steps


RMS_METRIC = "µs/call and HBM GB/s (% of peak) for RMSNorm fused with MXFP4 quantisation, M=4096 K=7168"
RMS_M, RMS_K, RMS_EPS = 4096, 7168, 1e-6


def rms_bytes(M, K):
    """x read once (2MK), the gain w (2K), codes (MK/2) and scale bytes (MK/32) written once."""
    return 2 * M * K + 2 * K + M * K // 2 + M * K // 32


def bench_rmsnorm(args):
    """One call of mxfp4_rmsnorm_quant per step, over rotated (cold) input sets."""
    import torch
    from mxfp4_block_scaled_02_amd import ops, synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seed = 101 if args.seed is None else args.seed
    M, K = RMS_M, RMS_K
    log(f"[bench] workload=rmsnorm seed={seed}: generating inputs")
    xb, wb = synth.make_a(M, K, seed), synth.make_norm_weight(K, seed)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x0, w = bf16(xb), bf16(wb)
    set_bytes = rms_bytes(M, K)
    R = n_sets(args, set_bytes)
    sets = [(x0.clone() if r else x0, torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
             torch.empty((M, K // 32), dtype=torch.uint8, device=dev)) for r in range(R)]

    def step(i):
        x, q, sc = sets[i % R]
        ops.rmsnorm_quant(x, w, RMS_EPS, out=(q, sc))

    ms_step = timed_steps(step, args)
    gbs = set_bytes / (ms_step * 1e-3) / 1e9
    out = dict(metric=RMS_METRIC, value=round(gbs, 3), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
               ms_per_step=round(ms_step, 6), higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="bf16 in, f64 sum of squares, f32 scale, mxfp4 out", data="synthetic",
               config=dict(workload="rmsnorm", seed=seed, M=M, K=K, eps=RMS_EPS,
                           cache=cache_label(args, R, set_bytes),
                           timing="hip graph replay" if not args.no_graph else "eager launch loop",
                           path="mxfp4_rmsnorm_quant"),
               us_per_call=round(ms_step * 1e3, 3), hbm_gbs=round(gbs, 2),
               roofline=dict(bound="hbm", achieved=round(gbs, 3), peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=round(gbs / HBM_PEAK_GBS, 4), traffic=recorded_traffic("rmsnorm"),
                             algorithmic_bytes=set_bytes))
    if not args.no_cpu_baseline:
        import oracle.rmsnorm as orn
        rows = 64
        t, runs, n, aff = time_oracle(lambda: orn.rmsnorm_quant(xb[:rows], wb, RMS_EPS))
        out["cpu_baseline"] = dict(value=round(rms_bytes(rows, K) / t / 1e9, 6), unit="GB/s", cores=n,
                                   kind="oracle", sample=f"oracle rmsnorm_quant on rows 0..{rows - 1} (K={K}); "
                                   f"median of {runs} runs, {t * 1e3:.1f} ms each; single-threaded numpy",
                                   affinity_cpus=aff, cpu_model=cpu_model())
    out["env"] = env_info()
    print(json.dumps(out), flush=True)


MNK_METRIC = "µs/call and TFLOP/s (% of peak) for grouped a4w4 GEMM with per-group (M, N, K) and batch L"


def mnk_problems(seed):
    """Seeded groups: M in {128..1024 step 64}, N in {1024, 2048, 4096}, K in {1024, 2048, 4096, 7168}, L in {1, 2, 3};
    six groups (at most 18 problems)."""
    g = np.random.default_rng([seed, 7])
    return [(int(128 + 64 * g.integers(0, 15)), int(g.choice([1024, 2048, 4096])),
             int(g.choice([1024, 2048, 4096, 7168])), int(g.integers(1, 4))) for _ in range(6)]


def bench_grouped_mnk(args):
    """One grouped_gemm_a4w4_mnk call per step over rotated (cold) operand sets."""
    import torch
    from mxfp4_block_scaled_02_amd import ops, synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seed = 102 if args.seed is None else args.seed
    shapes = mnk_problems(seed)
    log(f"[bench] workload=grouped_mnk seed={seed}: {shapes}")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    base = []
    for gi, (M, N, K, L) in enumerate(shapes):
        A = torch.stack([bf16(synth.make_a(M, K, seed, (gi, l))) for l in range(L)])
        Bp = torch.stack([ops.pack_B(*ops.quant(bf16(synth.make_b(N, K, seed, (gi, l))))) for l in range(L)])
        base.append((A, Bp, N))
    flops = sum(L * alg_flops(M, N, K) for M, N, K, L in shapes)
    nbytes = sum(L * alg_bytes(M, N, K) for M, N, K, L in shapes)
    set_bytes = sum(A.numel() * 2 + Bp.numel() for A, Bp, _ in base) + sum(L * 2 * M * N for M, N, K, L in shapes)
    R = n_sets(args, set_bytes)
    sets = []
    for r in range(R):
        probs = [(A.clone() if r else A, Bp.clone() if r else Bp, N) for A, Bp, N in base]
        outs = [torch.empty((A.shape[0], A.shape[1], N), dtype=torch.bfloat16, device=dev) for A, _, N in probs]
        sets.append((probs, outs))

    def step(i):
        probs, outs = sets[i % R]
        ops.grouped_gemm_mnk(probs, out_list=outs)

    ms_step = timed_steps(step, args)
    tflops = flops / (ms_step * 1e-3) / 1e12
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    if flops / (FP4_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9):
        bound, achieved, peak, unit = "mfma", tflops, FP4_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", gbs, HBM_PEAK_GBS, "GB/s"
    out = dict(metric=MNK_METRIC, value=round(achieved, 3), unit=unit, n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms_step, 6), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="mxfp4 (e2m1 x e8m0, fp32 accumulate, bf16 out)", data="synthetic",
               config=dict(workload="grouped_mnk", seed=seed, groups=[dict(M=M, N=N, K=K, L=L) for M, N, K, L in shapes],
                           cache=cache_label(args, R, set_bytes),
                           timing="hip graph replay" if not args.no_graph else "eager launch loop",
                           path="grouped_gemm_a4w4_mnk"),
               us_per_call=round(ms_step * 1e3, 3), tflops=round(tflops, 3), hbm_gbs=round(gbs, 2),
               roofline=dict(bound=bound, achieved=round(achieved, 3), peak=peak, unit=unit,
                             frac=round(achieved / peak, 4), traffic=recorded_traffic("grouped_mnk"),
                             algorithmic_bytes=nbytes,
                             algorithmic_flops=flops))
    if not args.no_cpu_baseline:
        import oracle
        M, N, K, L = shapes[0]
        a = synth.make_a(M, K, seed, (0, 0))
        bq, bs = oracle.quant_mx(synth.make_b(N, K, seed, (0, 0)))
        rows = min(M, 64)
        t, runs, n, aff = time_oracle(lambda: oracle.gemm_ref(a[:rows], bq, bs))
        val = alg_flops(rows, N, K) / t / 1e12 if unit == "TFLOP/s" else alg_bytes(rows, N, K) / t / 1e9
        out["cpu_baseline"] = dict(value=round(val, 6), unit=unit, cores=n, kind="oracle",
                                   sample=f"oracle gemm_ref on rows 0..{rows - 1} of the first problem (N={N}, K={K}); "
                                          f"median of {runs} runs, {t * 1e3:.1f} ms each; numpy's BLAS on {n} threads",
                                   affinity_cpus=aff, cpu_model=cpu_model())
    out["env"] = env_info()
    print(json.dumps(out), flush=True)


NV_METRIC = "µs/call and TFLOP/s (% of peak) for the NVFP4 group GEMM (E2M1, E4M3 per 16), per-group (M, N, K, L)"


def nv_bytes(M, N, K):
    """Algorithmic bytes of one NVFP4 problem: codes and scales of A and B read once, fp16 C written once."""
    return (M + N) * (K // 2 + K // 16) + 2 * M * N


def bench_nvfp4(args):
    """One grouped_gemm_nvfp4 call per step over rotated (cold) operand sets; the group
    shapes are those of the grouped_mnk workload (same seed)."""
    import torch
    from mxfp4_block_scaled_02_amd import ops, synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seed = 102 if args.seed is None else args.seed
    shapes = mnk_problems(seed)
    log(f"[bench] workload=nvfp4_grouped seed={seed}: {shapes}")
    u8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
    base = []
    for gi, (M, N, K, L) in enumerate(shapes):
        ops_ = [synth.make_nvfp4(M, K, seed, (gi, l)) + synth.make_nvfp4(N, K, seed, (gi, 100 + l)) for l in range(L)]
        base.append(tuple(torch.stack([u8(o[i]) for o in ops_]) for i in range(4)))
    flops = sum(L * alg_flops(M, N, K) for M, N, K, L in shapes)
    nbytes = sum(L * nv_bytes(M, N, K) for M, N, K, L in shapes)
    set_bytes = sum(sum(t.numel() for t in b) for b in base) + sum(L * 2 * M * N for M, N, K, L in shapes)
    R = n_sets(args, set_bytes)
    sets = []
    for r in range(R):
        probs = [tuple(t.clone() if r else t for t in b) for b in base]
        outs = [torch.empty((L, M, N), dtype=torch.float16, device=dev) for M, N, K, L in shapes]
        sets.append((probs, outs))

    def step(i):
        probs, outs = sets[i % R]
        ops.grouped_gemm_nvfp4(probs, out_list=outs)

    ms_step = timed_steps(step, args)
    tflops = flops / (ms_step * 1e-3) / 1e12
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    if flops / (BF16_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9):
        bound, achieved, peak, unit = "mfma", tflops, BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", gbs, HBM_PEAK_GBS, "GB/s"
    out = dict(metric=NV_METRIC, value=round(achieved, 3), unit=unit, n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms_step, 6), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="nvfp4 (e2m1 x e4m3 per 16; exact fp16 products, fp32 accumulate, fp16 out)",
               data="synthetic",
               config=dict(workload="nvfp4_grouped", seed=seed, groups=[dict(M=M, N=N, K=K, L=L) for M, N, K, L in shapes],
                           cache=cache_label(args, R, set_bytes),
                           timing="hip graph replay" if not args.no_graph else "eager launch loop",
                           path="grouped_gemm_nvfp4"),
               us_per_call=round(ms_step * 1e3, 3), tflops=round(tflops, 3), hbm_gbs=round(gbs, 2),
               roofline=dict(bound=bound, achieved=round(achieved, 3), peak=peak, unit=unit,
                             frac=round(achieved / peak, 4), traffic=recorded_traffic("nvfp4_grouped"),
                             algorithmic_bytes=nbytes,
                             algorithmic_flops=flops))
    if not args.no_cpu_baseline:
        import oracle
        M, N, K, L = shapes[0]
        aq, as_ = synth.make_nvfp4(M, K, seed, (0, 0))
        bq, bs = synth.make_nvfp4(N, K, seed, (0, 100))
        rows = min(M, 64)
        t, runs, n, aff = time_oracle(lambda: oracle.nvfp4.nvfp4_gemm_ref(aq[:rows], as_[:rows], bq, bs))
        val = alg_flops(rows, N, K) / t / 1e12 if unit == "TFLOP/s" else nv_bytes(rows, N, K) / t / 1e9
        out["cpu_baseline"] = dict(value=round(val, 6), unit=unit, cores=n, kind="oracle",
                                   sample=f"oracle nvfp4_gemm_ref on rows 0..{rows - 1} of the first problem "
                                          f"(N={N}, K={K}); median of {runs} runs, {t * 1e3:.1f} ms each; numpy's "
                                          f"BLAS on {n} threads", affinity_cpus=aff, cpu_model=cpu_model())
    out["env"] = env_info()
    print(json.dumps(out), flush=True)


def copy_calibration():
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": 5}))


def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.select)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library is a single-GPU kernel "
              "library with no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "rmsnorm":
        bench_rmsnorm(args)
        return
    if args.workload == "grouped_mnk":
        bench_grouped_mnk(args)
        return
    if args.workload == "nvfp4_grouped":
        bench_nvfp4(args)
        return
    if args.workload is not None:
        out, w, unit = bench_gemm(args.workload, args)
        if args.library:
            out["library"] = bench_library(args.workload, args)
        if not args.no_cpu_baseline:
            log("[bench] timing the CPU oracle on a bounded sample")
            out["cpu_baseline"] = cpu_baseline(w, unit)
        out["env"] = env_info()
        print(json.dumps(out), flush=True)
        return
    # Default: the headline (the largest configuration the metric spans) and the other configurations as
    # extra keys of the same line, each timed the same way.
    out, w, unit = bench_gemm(HEADLINE, args, sustained_steps=0 if args.no_graph else args.sustained_steps)
    del w
    extras = {}
    for name in EXTRAS:
        o, _, _ = bench_gemm(name, args)
        rf = o["roofline"]
        extras[name] = dict(config=o["config"], us_per_call=o["us_per_call"], tflops=o["tflops"], hbm_gbs=o["hbm_gbs"],
                            roofline=rf)
    out["workloads"] = extras
    if not args.no_library:
        out["library"] = bench_library(HEADLINE, args)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(synth_workload(HEADLINE, args), unit)
    out["env"] = env_info()
    print(json.dumps(out), flush=True)


def synth_workload(name, args):
    from mxfp4_block_scaled_02_amd import synth
    return synth.workload(name, synth.default_seed(name) if args.seed is None else args.seed)


def bench_gemm(name, args, sustained_steps=0):
    """One fused call (or, with --unfused, mxfp4_quant + gemm_a4w4) per step over rotated operand sets.
    With sustained_steps, the same calls are timed again over one replay of that many steps (a
    longer run, in which the shader clock settles lower under full load) and reported apart.
    Returns (the JSON record, the workload's inputs, the roofline unit)."""
    import torch
    from mxfp4_block_scaled_02_amd import ops, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth_workload(name, args)
    seed = w["seed"]
    log(f"[bench] workload={name} seed={seed}: generating inputs")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def prep_b(b_bits):
        bq, bs = ops.quant(bf16(b_bits))  # offline weight quantisation on the GPU (same kernel family)
        return ops.pack_B(bq, bs)

    if name in synth.GROUPED:
        Ms, N, K = w["Ms"], w["N"], w["K"]
        total_bytes = sum(alg_bytes(m, N, K) for m in Ms)
        total_flops = sum(alg_flops(m, N, K) for m in Ms)
        a0 = [bf16(x) for x in w["A"]]
        b0 = [prep_b(x) for x in w["B"]]
        set_bytes = sum(x.numel() * 2 for x in a0) + sum(x.numel() for x in b0) + sum(2 * m * N for m in Ms)
    else:
        M, N, K = w["M"], w["N"], w["K"]
        total_bytes, total_flops = alg_bytes(M, N, K), alg_flops(M, N, K)
        a0, b0 = bf16(w["A"]), prep_b(w["B"])
        set_bytes = a0.numel() * 2 + b0.numel() + 2 * M * N
    R = n_sets(args, set_bytes)
    log(f"[bench] operand set {set_bytes / 1e6:.2f} MB, rotating {R} sets")
    sets = []
    for r in range(R):
        if name in synth.GROUPED:
            a = [x.clone() for x in a0] if r else a0
            b = [x.clone() for x in b0] if r else b0
            c = [torch.empty((m, N), dtype=torch.bfloat16, device=dev) for m in Ms]
        else:
            a = a0.clone() if r else a0
            b = b0.clone() if r else b0
            c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        sets.append((a, b, c))
    if args.unfused:
        if name in synth.GROUPED:
            raise SystemExit("--unfused covers the single-GEMM workloads")
        aq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        asc = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)

    def step(i):
        a, b, c = sets[i % R]
        if name in synth.GROUPED:
            ops.grouped_gemm(a, b, N, out_list=c)
        elif args.unfused:
            ops.quant(a, out=(aq, asc))
            ops.gemm_a4w4(aq, asc, b, N, out=c)
        else:
            ops.gemm(a, b, N, out=c)

    ms_step = timed_steps(step, args)
    ms_sustained = None
    if sustained_steps > 0:
        import copy
        a2 = copy.copy(args)
        a2.steps, a2.warmup = sustained_steps, 0
        ms_sustained = timed_steps(step, a2)
    us = ms_step * 1e3
    gbs = total_bytes / (ms_step * 1e-3) / 1e9
    tflops = total_flops / (ms_step * 1e-3) / 1e12
    t_hbm, t_mfma = total_bytes / (HBM_PEAK_GBS * 1e9), total_flops / (FP4_PEAK_TFLOPS * 1e12)
    if t_mfma > t_hbm:
        bound, achieved, peak, unit = "mfma", tflops, FP4_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", gbs, HBM_PEAK_GBS, "GB/s"
    cfg = dict(workload=name, seed=seed, cache=cache_label(args, R, set_bytes),
               timing="hip graph replay" if not args.no_graph else "eager launch loop",
               path="unfused: mxfp4_quant + gemm_a4w4 (two launches)" if args.unfused else "fused: gemm_a4w4_fused"
               if name not in synth.GROUPED else "fused: grouped_gemm_a4w4 (one launch)")
    if name in synth.GROUPED:
        cfg.update(G=len(Ms), Ms=Ms, N=N, K=K)
    else:
        cfg.update(M=M, N=N, K=K)
    traffic = recorded_traffic(name + "_unfused" if args.unfused else name)
    roof = dict(bound=bound, achieved=round(achieved, 3), peak=peak, unit=unit, frac=round(achieved / peak, 4),
                traffic=traffic, algorithmic_bytes=total_bytes, algorithmic_flops=total_flops,
                traffic_ratio=round(traffic / total_bytes, 3) if traffic else None,
                frac_hbm=round(t_hbm / (ms_step * 1e-3), 4), frac_mfma=round(t_mfma / (ms_step * 1e-3), 4))
    out = dict(metric=METRIC, value=round(achieved, 3), unit=unit, n_gpus=1, steps=args.steps, warmup=args.warmup,
               ms_per_step=round(ms_step, 6), higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="mxfp4 (e2m1 x e8m0, fp32 accumulate, bf16 out)", data="synthetic", config=cfg,
               us_per_call=round(us, 3), tflops=round(tflops, 3), hbm_gbs=round(gbs, 2), roofline=roof)
    if ms_sustained is not None:
        rate = (total_flops / 1e12 if unit == "TFLOP/s" else total_bytes / 1e9) / (ms_sustained * 1e-3)
        out["sustained"] = dict(steps=sustained_steps, us_per_call=round(ms_sustained * 1e3, 3),
                                value=round(rate, 3), unit=unit, frac=round(rate / peak, 4))
    del sets, a0, b0
    torch.cuda.empty_cache()
    return out, w, unit


def bench_library(name, args):
    """The platform library's MXFP4 GEMM on the same workload, for comparison: torch._scaled_mm with
    float4_e2m1fn_x2 operands and float8_e8m0fnu block scales (hipBLASLt on ROCm). Its A and B are the
    codes and scale bytes of mxfp4_quant, made outside the timed region, so it times the GEMM alone
    (no quantisation of A), over rotated operand sets with the same protocol as bench_gemm. Its C is
    checked against gemm_a4w4 on the same codes (the same exact products; only the fp32 summation
    order may differ) with the tests' tolerance |d| <= 2^-7 |C| + 1e-3 max|C|."""
    import torch
    from mxfp4_block_scaled_02_amd import ops, synth
    path = "torch._scaled_mm (float4_e2m1fn_x2 x float8_e8m0fnu 1x32 scales, bf16 out; hipBLASLt)"
    if name in synth.GROUPED:
        return dict(path=path, error="single-GEMM workloads only")
    f4, e8 = getattr(torch, "float4_e2m1fn_x2", None), getattr(torch, "float8_e8m0fnu", None)
    if f4 is None or e8 is None:
        return dict(path=path, error="this torch has no float4_e2m1fn_x2 / float8_e8m0fnu")
    dev = torch.device("cuda:0")
    w = synth_workload(name, args)
    M, N, K = w["M"], w["N"], w["K"]

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    aq, asc = ops.quant(bf16(w["A"]))
    bq, bsc = ops.quant(bf16(w["B"]))
    set_bytes = aq.numel() + asc.numel() + bq.numel() + bsc.numel() + 2 * M * N
    R = n_sets(args, set_bytes)
    sets = [tuple(x.clone() if r else x for x in (aq, asc, bq, bsc)) + (torch.empty((M, N), dtype=torch.bfloat16,
                                                                                        device=dev),)
            for r in range(R)]

    def call(i):
        a, sa, b, sb, c = sets[i % R]
        c.copy_(torch._scaled_mm(a.view(f4), b.view(f4).t(), sa.view(e8), sb.view(e8), out_dtype=torch.bfloat16))

    def lib_step(i):
        a, sa, b, sb, _ = sets[i % R]
        torch._scaled_mm(a.view(f4), b.view(f4).t(), sa.view(e8), sb.view(e8), out_dtype=torch.bfloat16)

    try:
        call(0)
        ref = ops.gemm_a4w4(aq, asc, ops.pack_B(bq, bsc), N).float()
        got = sets[0][4].float()
        ok = bool(((got - ref).abs() <= 2.0 ** -7 * ref.abs() + 1e-3 * ref.abs().max()).all())
        ms = timed_steps(lib_step, args)
    except Exception as e:  # noqa: BLE001 - reported, never fatal to the bench line
        return dict(path=path, error=f"{type(e).__name__}: {e}"[:300])
    flops = alg_flops(M, N, K)
    tflops = flops / (ms * 1e-3) / 1e12
    out = dict(path=path, operands="A and B quantised by mxfp4_quant outside the timed region: the GEMM alone",
               us_per_call=round(ms * 1e3, 3), tflops=round(tflops, 3), frac_mfma=round(tflops / FP4_PEAK_TFLOPS, 4),
               agrees_with_gemm_a4w4=ok, cache=cache_label(args, R, set_bytes))
    del sets
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
