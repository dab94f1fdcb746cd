#!/usr/bin/env python3
"""Selective-scan forward benchmark on one MI355X.

A step is one call of the fused forward (every step of the method: softplus,
discretisation, the scan with its chunk carry, readout, final state) over one
batch of seeded synthetic input already resident in HBM.  The default workload
is the headline one: batch 8, L 4096, dim 1024, dstate 16, bf16 I/O with fp32
arithmetic.  Four copies of the inputs (over 512 MB together, twice the
256 MB Infinity Cache) are rotated so that x and delta of a step cannot be
served from a previous step's cache contents.

Prints one JSON line on stdout: throughput in state updates per second
(batch * L * dim * dstate per step, valid steps only for padded batches), the
algorithmic HBM GB/s, a roofline object for the kernel, and the CPU oracle
timed on this host on the same workload.

``--pass bwd`` measures the backward instead (gradients of every input for
seeded output gradients, from the chunk states of one untimed forward), with
its own roofline and the oracle's backward timed on the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

METRIC = "selective-scan state-updates/s (B·L·D·N) + HBM GB/s, B8 L4096 D1024 N16 bf16"

# MI355X figures used for the roofline.
CUS, SIMDS, LANES, CLOCK_HZ = 256, 4, 16, 2.4e9
FP32_VECTOR_PEAK_TFLOPS = 157.3   # published fp32 vector peak (128 FMA per CU per clock at 2.4 GHz)
HBM_PEAK_GBPS = 8000.0

# Algorithmic arithmetic in FMA-equivalent FLOPs: an fp32 add/mul/fma issue
# slot counts 2; v_exp_f32 and v_log_f32 occupy 4 FMA issue slots each
# (measured on gfx950: the transcendental rate is a quarter of the FMA rate
# and does not overlap with it), so they count 8.
#   per state update: exp(delta*A) 8 + mul delta*A, mul u*B, fma h, fma y 2 each = 16
#   per (b, t, d):    softplus (exp 8, log 8, mul, add, max, add, mul 2 each) 26
#                     + u = delta*x 2 + fma D*x 2 = 30
FLOPEQ_PER_UPDATE = 16.0
FLOPEQ_PER_ROW_STEP = 30.0
# Backward, per state update: exp(delta*A) 8; delta*A, u*B, h fma (recompute);
# g = C*dyp + mu, mu = Abar*g, sum g*B, da = g*h, da*Abar, sum da*Abar*A,
# dA += .*delta, dB += g*u, dC += dyp*h: 12 ops, 2 each = 32.  Per (b, t, d):
# softplus 26, sigmoid for its derivative (exp 8, rcp 8, add 2) 18, u = delta*x,
# dDelta fma, the clip/softplus factor, dx fma, dD fma (2 each) 10 = 54.
FLOPEQ_BWD_PER_UPDATE = 32.0
FLOPEQ_BWD_PER_ROW_STEP = 54.0

PROFILES = os.path.join(HERE, "profiles")
# Each pass's kernel sources and the build script that holds their compiler
# flags: a traffic record applies only to the build it was taken on.
_CSRC = os.path.join(HERE, "selective_state_space_scan_amd", "csrc")
_BUILD = os.path.join(HERE, "selective_state_space_scan_amd", "build.py")
KERNEL_SRCS = [os.path.join(_CSRC, f) for f in ("ssm_scan.hip", "ssm_internal.h")] + [_BUILD]
BWD_KERNEL_SRCS = [os.path.join(_CSRC, f) for f in ("ssm_scan_bwd.hip", "ssm_internal.h")] + [_BUILD]
TRAFFIC_RECORDS = {"fwd": ("ssm_fwd_kernel", KERNEL_SRCS), "bwd": ("ssm_bwd_kernel", BWD_KERNEL_SRCS)}


def kernel_source_hash(srcs=KERNEL_SRCS) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def algorithmic_bytes(w, e: int) -> int:
    """Bytes the method must move: x, delta read and y written ([B,L,D] each),
    B and C read ([B,L,N] each), A_log and D read, h_last written."""
    bld = w.batch * w.seqlen * w.dim
    bln = w.batch * w.seqlen * w.dstate
    return 3 * bld * e + 2 * bln * e + w.dim * w.dstate * 4 + w.dim * 4 + w.batch * w.dim * w.dstate * 4


def algorithmic_flops(w, valid_steps: int) -> float:
    """FMA-equivalent FLOPs of the method's arithmetic (see FLOPEQ_* above)."""
    return valid_steps * w.dim * (w.dstate * FLOPEQ_PER_UPDATE + FLOPEQ_PER_ROW_STEP)


def algorithmic_bytes_bwd(w, e: int, chunk_len: int) -> int:
    """Bytes the backward must move: x, delta, dy read and dx, ddelta written
    ([B,L,D] each, io dtype); B, C read (io) and dB, dC written (fp32)
    ([B,L,N] each); the chunk states read; A_log, D, dh_last read; dA_log, dD,
    dh0 written."""
    bld = w.batch * w.seqlen * w.dim
    bln = w.batch * w.seqlen * w.dstate
    n_chunks = (w.seqlen + chunk_len - 1) // chunk_len
    bdn = w.batch * w.dim * w.dstate
    return (5 * bld * e + 2 * bln * e + 2 * bln * 4 + (n_chunks - 1) * bdn * 4 + 2 * w.dim * w.dstate * 4
            + 2 * w.dim * 4 + 2 * bdn * 4)


def measured_traffic(w, kind: str = "fwd"):
    """HBM bytes per launch of the pass `kind` ("fwd" or "bwd", the backward
    counting its main and reduce kernels) measured with rocprofv3 (FETCH_SIZE +
    WRITE_SIZE, each scaled by the copy-kernel calibration) as recorded in
    profiles/, or None when there is no record for this workload or the
    kernel source has changed since it was taken."""
    kname, srcs = TRAFFIC_RECORDS[kind]
    path = os.path.join(PROFILES, f"traffic_{kname}_{w.name}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256") != kernel_source_hash(srcs):
        return None
    try:
        return int(float(rec["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def kernel_percentiles(kern_ms) -> dict:
    """p10 / median / p90 of the per-launch kernel times (ms)."""
    p = np.percentile(np.asarray(kern_ms, dtype=np.float64), [10, 50, 90])
    return {"kernel_ms_p10": round(float(p[0]), 5), "kernel_ms_p50": round(float(p[1]), 5),
            "kernel_ms_p90": round(float(p[2]), 5)}


TIMING_NOTES = {
    "kernel_avg_ms_from": "the timed region: K launches back to back between one pair of HIP events",
    "kernel_ms_percentiles_from": "a separate pass of K launches after the timed region, each between its own events",
}


def time_steps(step, steps: int, stream) -> float:
    """The timed region: `steps` launches back to back on `stream`, between one
    pair of HIP events, bracketed by synchronisations; ms per step.  No event
    is recorded between the launches: an event between two launches of the
    forward made the second one ~5 % slower on this GPU, so the per-launch
    average is the region's time over the launches (inter-launch gaps
    included)."""
    import torch
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(steps):
        step(k)
    t_end.record(stream)
    torch.cuda.synchronize()
    return t_start.elapsed_time(t_end) / steps


def per_launch_ms(step, steps: int, stream) -> list:
    """After the timed region, untimed: `steps` more launches, each between its
    own pair of events, for the spread of single launch times (ms)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record(stream)
        step(k)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def host_cpu() -> dict:
    """The host the CPU baseline ran on: processor model, logical CPUs, and
    the CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(inp, w, threads: int, min_seconds: float = 1.0) -> dict:
    """The fp64 oracle on the host, over the whole workload, repeated until at
    least `min_seconds` of wall time (so `threads` x that of CPU work)."""
    import oracle
    oracle.build()
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.selective_scan(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"],
                              valid_len=inp["valid_len"], delta_clamp=w.delta_clamp, nthreads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    steps = w.batch * w.seqlen if inp["valid_len"] is None else int(np.sum(inp["valid_len"]))
    upd = steps * w.dim * w.dstate * passes
    return {"value": upd / dt, "unit": "state-updates/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole {w.name} workload, {passes} passes ({upd} state updates, {dt:.2f} s wall, "
                      f"{threads} threads over (b, d) rows; fp64, gcc -O2)", "host": host_cpu()}


LDS_PATTERNS = ("read_b32 consecutive", "write_b32 consecutive", "read_b64 consecutive", "read_b128 consecutive",
                "write_b128 consecutive", "read_b32 broadcast", "read_b32 stride 2 (two lanes per bank)",
                "read_b128 16-lane rows broadcast, rows 80 words apart",
                "read2st64_b32 pair 256 words apart (same bank)", "read2_b32 pair 68 words apart (different banks)",
                "write2st64_b32 pair 256 words apart (same bank)")


def lds_probe(dev, blocks: int = 1024, iters: int = 4096) -> dict:
    """Launch each LDS access pattern of libssmpeaks.so once, in order (a
    profiler reads the LDS counters of each dispatch), and report their times."""
    import ctypes

    import torch

    from selective_state_space_scan_amd import build as B
    lib = ctypes.CDLL(B.PEAKS_LIB_PATH)
    lib.ssm_peak_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.ssm_peak_launch.restype = ctypes.c_int
    stream = torch.cuda.current_stream(dev)
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    res = {"lds_probe": {"blocks": blocks, "waves_per_block": 4, "accesses_per_wave": iters, "patterns": []}}
    for k, name in enumerate(LDS_PATTERNS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = lib.ssm_peak_launch(4, None, None, k, out.data_ptr(), blocks, iters, stream.cuda_stream)
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"ssm_peak_launch(4, pattern {k}) failed: {rc}")
        torch.cuda.synchronize()
        res["lds_probe"]["patterns"].append({"pattern": k, "name": name, "ms": round(e0.elapsed_time(e1), 4)})
    return res


def measure_peaks(dev) -> dict:
    """Peak rates of this GPU from the microbenchmarks in libssmpeaks.so
    (median of 10 timed launches after 3 warm-ups, HIP events on the
    launching stream): HBM read and copy bandwidth (GB/s, copy counting read
    plus write), the plain fp32 FMA rate (TFLOP/s, 2 per FMA) and the
    v_exp_f32 rate (T exp/s)."""
    import ctypes

    import torch

    from selective_state_space_scan_amd import build as B
    if not os.path.exists(B.PEAKS_LIB_PATH):
        raise FileNotFoundError(f"{B.PEAKS_LIB_PATH} is not built (python -m selective_state_space_scan_amd.build)")
    lib = ctypes.CDLL(B.PEAKS_LIB_PATH)
    lib.ssm_peak_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.ssm_peak_launch.restype = ctypes.c_int
    stream = torch.cuda.current_stream(dev)
    blocks = 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    big = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)  # 1 GiB
    dst = torch.empty((1 << 29) // 4, dtype=torch.float32, device=dev)  # 512 MiB

    def timed(which, a, b, n4, iters):
        ms = []
        for r in range(13):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.ssm_peak_launch(which, a, b, n4, out.data_ptr(), blocks, iters, stream.cuda_stream)
            e1.record(stream)
            if rc != 0:
                raise RuntimeError(f"ssm_peak_launch({which}) failed: {rc}")
            torch.cuda.synchronize()
            if r >= 3:
                ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    t_read = timed(0, big.data_ptr(), None, big.numel() // 4, 0)
    t_copy = timed(1, big.data_ptr(), dst.data_ptr(), dst.numel() // 4, 0)
    fma_iters, exp_iters = 2048, 512
    t_fma = timed(2, None, None, 0, fma_iters)
    t_exp = timed(3, None, None, 0, exp_iters)
    threads = blocks * 256
    del big, dst
    return {"hbm_read_gbps": round((1 << 30) / (t_read * 1e-3) / 1e9, 1),
            "hbm_copy_gbps": round(2 * (1 << 29) / (t_copy * 1e-3) / 1e9, 1),
            "fp32_fma_tflops": round(threads * fma_iters * 16 * 2 / (t_fma * 1e-3) / 1e12, 2),
            "exp_t_per_s": round(threads * exp_iters * 8 / (t_exp * 1e-3) / 1e12, 2)}


def add_measured_peak(roof: dict, peaks: dict) -> None:
    """The roofline's binding bound against the measured peak as well: plain
    FMA TFLOP/s for an ALU bound, HBM read GB/s for an HBM bound; and the
    algorithmic HBM rate against the measured copy rate (read + write bytes,
    like the algorithmic count)."""
    pm = peaks["fp32_fma_tflops"] if roof["bound"] == "alu" else peaks["hbm_read_gbps"]
    roof["peak_measured"] = pm
    roof["frac_measured"] = round(roof["achieved"] / pm, 4)
    if "hbm_gbps" in roof and peaks.get("hbm_copy_gbps"):
        roof["hbm_frac_measured_copy"] = round(roof["hbm_gbps"] / peaks["hbm_copy_gbps"], 4)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The GPU settles to its sustained clock over the first ~100 launches
    # (measured: 205 us average after 5 warm-up launches, 192 us after 200).
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=2, help="workload index (default: the headline one)")
    ap.add_argument("--rotate", type=int, default=4, help="input copies rotated between steps")
    ap.add_argument("--time-parts", type=int, default=0,
                    help="forward time split: parts to cut the sequence into (default 0: the library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the peak-rate microbenchmarks (roofline against the published peak only)")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (default: min(16, cpus))")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="measure the forward (default) or the backward")
    ap.add_argument("--combine", choices=("walk", "wave_scan"), default="walk",
                    help="how a tile's sub-chunks are joined: the serial walk (default) or the log-depth wave scan")
    ap.add_argument("--dstate", type=int, default=0,
                    help="override the workload's state count (16, 32 or 64; for the combine comparison)")
    ap.add_argument("--lds-probe", action="store_true",
                    help="instead of the benchmark, launch each LDS access pattern of libssmpeaks.so once "
                         "(reference readings for the LDS instruction and bank-conflict counters)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many MiB three times "
                         "(reference reading for the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import selective_state_space_scan_amd as ssm
    from selective_state_space_scan_amd import inputs as I

    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        return 1
    if args.lds_probe:
        print(json.dumps(lds_probe(torch.device("cuda:0"))))
        return 0
    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "repeats": 3}))
        return 0
    w = I.WORKLOADS[args.workload]
    if args.dstate and args.dstate != w.dstate:
        w = dataclasses.replace(w, dstate=args.dstate, name=f"{w.name}-as-n{args.dstate}")
    inp = I.make_inputs(w, I.seed_for(args.workload))
    if args.which == "bwd":
        return bench_bwd(args, w, inp)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if w.io == "bf16" else torch.float32
    sets = []
    base = {k: torch.from_numpy(inp[k]).to(dev).to(dt).contiguous() for k in ("x", "delta", "B", "C")}
    for r in range(max(1, args.rotate)):
        s = {k: (v if r == 0 else v.clone()) for k, v in base.items()}
        sets.append(s)
    A_log = torch.from_numpy(inp["A_log"]).to(dev)
    D = torch.from_numpy(inp["D"]).to(dev)
    vl = None if inp["valid_len"] is None else torch.from_numpy(inp["valid_len"]).to(dev)
    ys = [torch.empty_like(base["x"]) for _ in sets]
    hs = [torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev) for _ in sets]
    # The library's own time split (batches too small to fill the GPU): its
    # workspace is allocated here, outside the timed region.
    dims = ssm.ssm_scan_dims()
    dims.batch, dims.seqlen, dims.dim, dims.dstate = w.batch, w.seqlen, w.dim, w.dstate
    dims.io_dtype = ssm.SSM_IO_BF16 if w.io == "bf16" else ssm.SSM_IO_F32
    parts = args.time_parts or ssm.auto_time_parts(ssm._binding.handle_for(dev.index or 0), dims)
    ws_bytes = ssm.workspace_bytes(dims, parts)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step(k: int):
        s = sets[k % len(sets)]
        ssm.selective_scan_fwd(s["x"], s["delta"], A_log, s["B"], s["C"], D, vl, delta_clamp=w.delta_clamp,
                               y=ys[k % len(sets)], h_last=hs[k % len(sets)], time_parts=parts, workspace=ws,
                               combine=args.combine)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ms_per_step = time_steps(step, args.steps, stream)
    kern_avg_ms = ms_per_step
    kern_ms = per_launch_ms(step, args.steps, stream)

    steps_valid = w.batch * w.seqlen if inp["valid_len"] is None else int(np.sum(inp["valid_len"]))
    updates = steps_valid * w.dim * w.dstate
    e = 2 if w.io == "bf16" else 4
    nbytes = algorithmic_bytes(w, e)
    flops = algorithmic_flops(w, steps_valid)
    gbps = nbytes / (kern_avg_ms * 1e-3) / 1e9
    tflops = flops / (kern_avg_ms * 1e-3) / 1e12
    t_alu = flops / (FP32_VECTOR_PEAK_TFLOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9)
    traffic = measured_traffic(w)
    if t_alu >= t_hbm:
        roof = {"bound": "alu", "achieved": round(tflops, 3), "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / FP32_VECTOR_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}
    roof["kernel"] = ("ssm_fwd_kernel" if parts == 1 else
                      f"ssm_fwd_kernel: fold of {parts - 1} time parts, then the forward over {parts} parts")
    roof["kernel_avg_ms"] = round(kern_avg_ms, 5)
    roof.update(kernel_percentiles(kern_ms))
    roof.update(TIMING_NOTES)
    roof["hbm_gbps"] = round(gbps, 1)
    roof["hbm_frac"] = round(gbps / HBM_PEAK_GBPS, 4)
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_tflop"] = flops / 1e12
    roof["traffic_unit"] = "bytes per launch"

    peaks = None if args.no_peaks else measure_peaks(dev)
    if peaks is not None:
        add_measured_peak(roof, peaks)
    out = {
        "metric": METRIC,
        "value": updates / (ms_per_step * 1e-3),
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "hbm_gbps": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1),
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim, "dstate": w.dstate,
                   "io": w.io, "state_updates_per_step": updates, "input_copies_rotated": len(sets),
                   "time_parts": parts, "combine": args.combine},
        "roofline": roof,
    }
    if peaks is not None:
        out["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        out["cpu_baseline"] = cpu_baseline(inp, w, threads)
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline_bwd(inp, cot, w, threads: int, min_seconds: float = 2.0) -> dict:
    """The fp64 oracle's backward on the host, over the whole workload,
    repeated until at least `min_seconds` of wall time."""
    import oracle
    oracle.build()
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.selective_scan_bwd(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], cot["dy"],
                                  valid_len=inp["valid_len"], dh_last=cot["dh_last"], delta_clamp=w.delta_clamp,
                                  nthreads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    steps = w.batch * w.seqlen if inp["valid_len"] is None else int(np.sum(inp["valid_len"]))
    upd = steps * w.dim * w.dstate * passes
    used = min(threads, w.batch)  # the oracle's backward deals batch rows to threads
    return {"value": upd / dt, "unit": "state-updates/s", "cores": used, "kind": "oracle",
            "sample": f"the whole {w.name} workload, {passes} passes ({upd} state updates, {dt:.2f} s wall, "
                      f"{used} threads over batch rows; fp64, gcc -O2)", "host": host_cpu()}


def bench_bwd(args, w, inp) -> int:
    import torch

    import selective_state_space_scan_amd as ssm
    from selective_state_space_scan_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if w.io == "bf16" else torch.float32
    cot = I.make_cotangents(w, I.seed_for(args.workload) + 500)
    cl = ssm.bwd_chunk_len(w.dstate)
    A_log = torch.from_numpy(inp["A_log"]).to(dev)
    D = torch.from_numpy(inp["D"]).to(dev)
    vl = None if inp["valid_len"] is None else torch.from_numpy(inp["valid_len"]).to(dev)
    base = {k: torch.from_numpy(inp[k]).to(dev).to(dt).contiguous() for k in ("x", "delta", "B", "C")}
    base["dy"] = torch.from_numpy(cot["dy"]).to(dev).to(dt)
    dhl = torch.from_numpy(cot["dh_last"]).to(dev)
    sets = []
    for r in range(max(1, args.rotate)):
        s = {k: (v if r == 0 else v.clone()) for k, v in base.items()}
        # the forward (untimed) leaves the chunk states the backward recomputes from
        _, _, s["cs"] = ssm.selective_scan_fwd(s["x"], s["delta"], A_log, s["B"], s["C"], D, vl,
                                               delta_clamp=w.delta_clamp, return_chunk_states=True, chunk_len=cl)
        sets.append(s)
    dims = ssm.ssm_scan_dims()
    dims.batch, dims.seqlen, dims.dim, dims.dstate = w.batch, w.seqlen, w.dim, w.dstate
    dims.io_dtype = ssm.SSM_IO_BF16 if w.io == "bf16" else ssm.SSM_IO_F32
    ws = torch.empty(ssm.bwd_workspace_bytes(dims), dtype=torch.uint8, device=dev)

    def step(k: int):
        s = sets[k % len(sets)]
        ssm.selective_scan_bwd(s["x"], s["delta"], A_log, s["B"], s["C"], D, vl, s["dy"], s["cs"], dh_last=dhl,
                               delta_clamp=w.delta_clamp, workspace=ws)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ms_per_step = time_steps(step, args.steps, stream)
    kern_avg_ms = ms_per_step
    kern_ms = per_launch_ms(step, args.steps, stream)
    steps_valid = w.batch * w.seqlen if inp["valid_len"] is None else int(np.sum(inp["valid_len"]))
    updates = steps_valid * w.dim * w.dstate
    e = 2 if w.io == "bf16" else 4
    nbytes = algorithmic_bytes_bwd(w, e, cl)
    flops = steps_valid * w.dim * (w.dstate * FLOPEQ_BWD_PER_UPDATE + FLOPEQ_BWD_PER_ROW_STEP)
    gbps = nbytes / (kern_avg_ms * 1e-3) / 1e9
    tflops = flops / (kern_avg_ms * 1e-3) / 1e12
    traffic = measured_traffic(w, "bwd")
    if flops / (FP32_VECTOR_PEAK_TFLOPS * 1e12) >= nbytes / (HBM_PEAK_GBPS * 1e9):
        roof = {"bound": "alu", "achieved": round(tflops, 3), "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / FP32_VECTOR_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}
    roof.update({"kernel": "ssm_bwd_kernel + ssm_bwd_reduce_kernel", "kernel_avg_ms": round(kern_avg_ms, 5),
                 "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes": nbytes,
                 "algorithmic_tflop": flops / 1e12, "traffic_unit": "bytes per launch"})
    roof.update(kernel_percentiles(kern_ms))
    roof.update(TIMING_NOTES)
    peaks = None if args.no_peaks else measure_peaks(dev)
    if peaks is not None:
        add_measured_peak(roof, peaks)
    out = {
        "metric": "selective-scan backward state-updates/s (B·L·D·N) + HBM GB/s",
        "value": updates / (ms_per_step * 1e-3),
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "hbm_gbps": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1),
        "config": {"workload": w.name, "pass": "backward", "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                   "dstate": w.dstate, "io": w.io, "state_updates_per_step": updates, "chunk_len": cl,
                   "input_copies_rotated": len(sets)},
        "roofline": roof,
    }
    if peaks is not None:
        out["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        out["cpu_baseline"] = cpu_baseline_bwd(inp, cot, w, threads)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
