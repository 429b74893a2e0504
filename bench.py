#!/usr/bin/env python3
"""Benchmark of the MI355X bf16 GEMM library.

One step is one call of gemm_bf16 on the chosen workload (default: the
4096^3 square, A row-major, B and C column-major, N(0,1) seeded inputs,
alpha = 1, beta = 0), with inputs already resident in device memory.  The
protocol follows "Outperforming cuBLAS on H100: a worklog", section
"Experimental setup": W untimed warm-up launches, then the mean over K timed
launches, FLOPS = 2*M*N*K / time.  The K launches run back to back between
one pair of HIP events recorded on the stream the kernel runs on (synchronized
on both sides); their mean is `value` and the roofline's achieved rate.  A
second pass of K launches, each between its own event pair, gives the
per-launch spread (min / median / max); a per-launch pair also times the
command processor's dispatch of the kernel, a few microseconds that matter
for the short memory-bound launch.  Then the pages' own protocol (one
warm-up launch, the mean of 8 launches) is reported beside it.  When
beta != 0 C is in/out: every launch reads the previous launch's output as C0
(same bytes, same work).

Prints ONE JSON line (rank 0, one GPU).  With --all it prints one line per
workload instead.

    python bench.py [--gpus 1] [--steps 200] [--warmup 300] [--workload square_4096]

The roofline's "traffic" (HBM bytes per launch) comes from rocprofv3
FETCH_SIZE / WRITE_SIZE passes recorded in profiles/hbm_traffic.json, each
counter scaled by what it reads for a plain device copy of known size.  An
entry is used only if it was recorded for the same kernel, workload and
library source digest; otherwise traffic is null.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from bf16_gemm_fp32_amd import inputs  # noqa: E402

METRIC = "bf16 GEMM TFLOP/s at M=N=K=4096 and % of MI355X dense bf16 MFMA peak"
# MI355X published peaks: dense bf16 MFMA = 256 CU x 4096 flop/clk x 2.4 GHz,
# HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 5033.2  # dense fp8 MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0
EPI = {"none": 0, "gelu_tanh": 1, "relu": 2}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_threads():
    """Host threads for the CPU oracle: every core in this process's affinity
    mask, capped by the host's allotment for this GPU when one is set
    (OMP_NUM_THREADS; 16 cores per GPU on the MI355X boxes)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    allot = os.environ.get("OMP_NUM_THREADS", "")
    if allot.isdigit() and int(allot) > 0:
        n = min(n, int(allot))
    return max(1, n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, d, budget_cols=None):
    """Time the CPU oracle on a bounded sample of the workload: whole output
    columns (every row m of the first `cols` columns)."""
    import oracle
    nthreads = cpu_threads()
    M, N, K = w.M, w.N, w.K
    if budget_cols is None:
        # about 10-20 s on 16 host cores at ~0.37 GMAC/s per core
        target_macs = 4.0e9 * nthreads
        budget_cols = int(max(1, min(N, target_macs // max(1, M * K))))
    cols = budget_cols
    ms = np.tile(np.arange(M, dtype=np.int64), cols)
    ns = np.repeat(np.arange(cols, dtype=np.int64), M)
    t0 = time.perf_counter()
    if w.inp == "fp8":
        oracle.gemm_fp8_elems(M, N, K, d["A"], K, d["B"], K, ms, ns, d.get("C0"), M, w.alpha, w.beta,
                              d["scale_a"], d["scale_b"], d.get("bias"), w.epilogue, nthreads=nthreads)
    else:
        _, y = oracle.gemm_elems(M, N, K, d["A"], K, d["B"], K, ms, ns, d.get("C0"), M, w.alpha, w.beta,
                                 d.get("bias"), w.epilogue, nthreads=nthreads, return_pre=True)
        if w.out == "int8":
            oracle.quantize_i8_array(y, d["scale"][ms], w.zero_point)
    dt = time.perf_counter() - t0
    flops = 2.0 * M * cols * K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": f"{cols} whole columns of C ({M * cols} of {M * N} outputs, {flops:.3e} flop) "
                  f"in {dt:.2f} s on {cpu_model()}",
    }


def measured_record(workload, kernel):
    """The recorded counter passes for this kernel and workload (HBM bytes
    per launch, achieved clock, MFMA busy, ...), or None when no record
    matches this kernel, workload and library source digest."""
    from bf16_gemm_fp32_amd.build import source_digest
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    digest = source_digest()
    for e in rec.get("entries", []):
        if e.get("workload") == workload and e.get("kernel") == kernel and e.get("source_digest") == digest:
            return e
    return None


def device_info(torch):
    """Compute units and clocks of device 0 (HIP device attributes)."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "max_sclk_mhz": None}
    try:
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        # hipDeviceAttributeClockRate (kHz)
        attr = 5
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) == 0 and v.value > 0:
            info["max_sclk_mhz"] = v.value / 1000.0
    except OSError:
        pass
    return info


def run_workload(w, steps, warmup, cold, with_cpu):
    import torch
    import bf16_gemm_fp32_amd as gb

    gb.library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"[bench] workload {w.name}: M={w.M} N={w.N} K={w.K} building inputs")
    d = inputs.make_inputs(w)

    def dev_tensor(bits):
        if bits.dtype == np.uint8:
            return torch.from_numpy(bits).to(dev)
        return torch.from_numpy(bits.view(np.int16)).to(dev)

    # rotate distinct buffer sets (>= 512 MiB in all, twice the 256 MB
    # Infinity Cache) so the memory-bound workloads read B from HBM
    in_bytes = w.in_bytes * (w.M * w.K + w.K * w.N)
    copies = max(4, -(-512 * 2 ** 20 // max(in_bytes, 1))) if cold else 1
    q8 = w.out == "int8"
    A = [dev_tensor(d["A"]) for _ in range(copies)]
    B = [dev_tensor(d["B"]) for _ in range(copies)]
    C = [torch.empty(w.N * w.M, dtype=torch.int8 if q8 else torch.int16, device=dev) for _ in range(copies)]
    C0 = dev_tensor(d["C0"]) if "C0" in d else None
    bias = dev_tensor(d["bias"]) if "bias" in d else None
    scale = torch.from_numpy(d["scale"]).to(dev) if q8 else None
    fp8 = w.inp == "fp8"
    sa = torch.from_numpy(d["scale_a"]).to(dev) if fp8 else None
    sb = torch.from_numpy(d["scale_b"]).to(dev) if fp8 else None
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    bias_p = bias.data_ptr() if bias is not None else 0
    if fp8:
        kname = gb.gemm_fp8_kernel_name(w.M, w.N, w.K, A[0].data_ptr(), w.K, B[0].data_ptr(), w.K, C[0].data_ptr(),
                                        w.M, EPI[w.epilogue])
    elif q8:
        c0_p = C0.data_ptr() if C0 is not None else 0
        kname = gb.gemm_bf16_q8_kernel_name(w.M, w.N, w.K, A[0].data_ptr(), w.K, B[0].data_ptr(), w.K, c0_p, w.M,
                                            C[0].data_ptr(), w.M, w.beta, scale.data_ptr(), EPI[w.epilogue])
    else:
        kname = gb.gemm_bf16_kernel_name(w.M, w.N, w.K, A[0].data_ptr(), w.K, B[0].data_ptr(), w.K,
                                         C[0].data_ptr(), w.M, w.beta, bias_p, EPI[w.epilogue])
    log(f"[bench] kernel {kname}; warmup {warmup}, steps {steps}, cold={cold}")

    if C0 is not None and not q8:
        for c in C:
            c.copy_(C0)  # beta != 0: C starts as C0 and stays in/out

    def launch(i):
        return i % copies

    def call(j):
        if fp8:
            st = gb.gemm_fp8(w.M, w.N, w.K, A[j].data_ptr(), w.K, B[j].data_ptr(), w.K, C[j].data_ptr(), w.M,
                             w.alpha, w.beta, sa.data_ptr(), sb.data_ptr(), bias_p, EPI[w.epilogue], sp)
        elif q8:
            st = gb.gemm_bf16_q8(w.M, w.N, w.K, A[j].data_ptr(), w.K, B[j].data_ptr(), w.K, c0_p, w.M,
                                 C[j].data_ptr(), w.M, w.alpha, w.beta, bias_p, EPI[w.epilogue], scale.data_ptr(),
                                 w.zero_point, sp)
        else:
            st = gb.gemm_bf16(w.M, w.N, w.K, A[j].data_ptr(), w.K, B[j].data_ptr(), w.K, C[j].data_ptr(), w.M,
                              w.alpha, w.beta, bias_p, EPI[w.epilogue], sp)
        if st != 0:
            raise RuntimeError(f"gemm_bf16 status {st}: {gb.gemm_bf16_status_string(st)}")

    for i in range(warmup):
        call(launch(i))
    torch.cuda.synchronize()

    # timed region: K launches back to back between one event pair
    all0 = torch.cuda.Event(enable_timing=True)
    all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    all0.record(stream)
    for i in range(steps):
        call(launch(warmup + i))
    all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = all0.elapsed_time(all1)
    mean_ms = region_ms / steps
    tflops = w.flops / (mean_ms * 1e-3) / 1e12
    gbs = w.algorithmic_bytes / (mean_ms * 1e-3) / 1e9
    log(f"[bench] timed region: {steps} launches in {region_ms:.3f} ms -> {mean_ms * 1e3:.2f} us per launch, "
        f"{tflops:.1f} TFLOP/s, {gbs:.0f} GB/s algorithmic")

    # spread: the same K launches again, each between its own event pair
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        j = launch(warmup + steps + i)
        ev[i][0].record(stream)
        call(j)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]  # ms
    log(f"[bench] per-launch event pairs ms: mean {statistics.fmean(per):.4f} min {min(per):.4f} "
        f"median {statistics.median(per):.4f} max {max(per):.4f}")

    # The pages' own protocol, after the runs above: one warm-up launch, then
    # the mean of 8 launches, each between its own event pair.
    call(launch(warmup + 2 * steps))
    ev8 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(8)]
    for i in range(8):
        j = launch(warmup + 2 * steps + 1 + i)
        ev8[i][0].record(stream)
        call(j)
        ev8[i][1].record(stream)
    torch.cuda.synchronize()
    ms8 = statistics.fmean(a.elapsed_time(b) for a, b in ev8)

    rec = measured_record(w.name, kname)
    traffic = rec.get("hbm_bytes_per_launch") if rec else None
    if w.bound == "hbm":
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "traffic": traffic}
    else:
        peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                "frac": tflops / peak, "traffic": traffic}
    roof["traffic_unit"] = "bytes per launch (HBM, counter-measured)"
    roof["algorithmic_bytes"] = w.algorithmic_bytes
    roof["traffic_over_algorithmic"] = traffic / w.algorithmic_bytes if traffic else None
    out = {
        "metric": METRIC if w.name == "square_4096" else f"{'fp8' if fp8 else 'bf16'} GEMM TFLOP/s on {w.name}",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": mean_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
                   "bias": w.bias, "epilogue": w.epilogue, "layout": "A row-major, B/C column-major",
                   "kernel": kname, "inputs": "N(0,1) seeded (bias N(0,0.1))", "output": w.out,
                   "cache": f"cold ({copies} rotating buffer sets)" if cold else "warm"},
        "pct_of_peak": 100.0 * tflops / (PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS),
        "hbm_gbs_algorithmic": gbs,
        "per_launch_event_pairs_ms": {"mean": statistics.fmean(per), "min": min(per),
                                      "median": statistics.median(per), "max": max(per),
                                      "stdev": statistics.pstdev(per)},
        "pages_protocol": {"warmup": 1, "runs": 8, "ms_mean": ms8, "tflops": w.flops / (ms8 * 1e-3) / 1e12,
                           "note": "after the timed region: 1 warm-up launch, then the mean of 8 launches each "
                                   "timed by its own event pair"},
        "timed_region_wall_ms": wall * 1e3,
        "timed_region_event_ms": region_ms,
        "roofline": roof,
        "device": device_info(torch),
        # from the recorded counter passes of this kernel and workload at this
        # library build (null when none match): the achieved clock between
        # SQ_BUSY_CYCLES per shader engine and GRBM_GUI_ACTIVE per XCD over the
        # kernel time, MFMA busy cycles over the SIMD cycles, L2 hit rate and
        # LDS bank-conflict cycles per LDS instruction
        "profiled": ({k: rec.get(k) for k in ("sclk_mhz_lower", "sclk_mhz_upper", "mfma_busy", "mfma_busy_upper",
                                              "l2_hit", "lds_bank_conflict_per_lds_inst", "summary")}
                     if rec else None),
        "cpu_baseline": None,
    }
    if with_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, d)
    return out


def calibrate_copy(mib):
    """A plain device-to-device copy of `mib` MiB (torch's copy kernel): the
    reference for scaling the FETCH_SIZE / WRITE_SIZE counters, which should
    read `mib` MiB each for it."""
    import torch
    n = mib * 1024 * 1024 // 2
    src = torch.ones(n, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": 2 * n, "bytes_written": 2 * n}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # The part's clocks settle only after some 20-30 ms of sustained load
    # (the first ~200 launches at 4096^3 run ~20% slower, and again after an
    # idle second), so the default warm-up is 300 launches.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="square_4096", choices=list(inputs.WORKLOADS))
    ap.add_argument("--all", action="store_true", help="one JSON line per workload")
    ap.add_argument("--cold", choices=["auto", "yes", "no"], default="auto",
                    help="rotate 4 buffer sets (default: only for the memory-bound workload)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", type=int, metavar="MIB", default=0,
                    help="only run a plain MIB-MiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: gemm_bf16 is a single-GPU kernel library "
              "(multi-GPU sharding is described in the design notes, not implemented).", file=sys.stderr)
        sys.exit(2)

    names = list(inputs.WORKLOADS) if args.all else [args.workload]
    for name in names:
        w = inputs.WORKLOADS[name]
        cold = (w.bound == "hbm") if args.cold == "auto" else (args.cold == "yes")
        res = run_workload(w, args.steps, args.warmup, cold,
                           with_cpu=not args.no_cpu and (name == "square_4096" or not args.all))
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
