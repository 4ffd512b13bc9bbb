#!/usr/bin/env python3
"""Bench of libsgemm: SGEMM TFLOP/s and % of the MI355X FP32 peak on one GPU.

One step = one call of the library's ``sgemm`` on the whole workload (inputs
resident in HBM before the timed region).  Default workload: M = N = K = 4096,
A, B ~ U[-1, 1), alpha = 1, beta = 0.  Prints ONE JSON line on stdout.

    python bench.py [--gpus 1] [--steps 200] [--warmup 100] [--preroll 1.0] [--workload square4096]
                    [--variant ID] [--op NN|NT|TN|TT] [--no-cpu-baseline] [--cpu-full]
                    [--cpu-threads N] [--cold | --cold-dirty] [--shard-rows G] [--smi]

Order of the GPU work: one call whose output is checked against the oracle; the pre-roll
(``--preroll`` seconds of back-to-back steps, reported in the line as ``preroll``: the engine
clock ramps up over the first tens of milliseconds of sustained load, and a run measured from a
cold start times that ramp rather than the kernel); the warmup steps; an engine-clock probe; the
timed region; a second probe (``sclk_mhz``: the clock right before and right after the timed
region, read on the GPU on the same stream); single launches for the spread; and the launch
floor (``launch_floor``: an empty kernel with the dispatched variant's grid, timed the same way).

``--op`` other than NN stores A as K x M and/or B as N x K and times
``sgemm_op`` (op(A) * op(B)) on the same logical product.

CPU figures (unless --no-cpu-baseline): ``cpu_baseline`` times the float64 oracle on a
bounded sample of the workload (and checks the GPU's first output against it);
``cpu_blocked`` times a cache-blocked fp32 CPU SGEMM (cpu_blocked/) on the whole
workload, the fairer CPU comparison.

Roofline: ``roofline`` prices the mean launch against the FP32 MFMA peak (TFLOP/s); for the
tall-skinny workload, which is reported against HBM, it gives the algorithmic bytes per launch
over the same duration against the 8 TB/s HBM peak instead, with the compute figure beside it in
``roofline_compute``.  With ``--cold`` the mean launch is that of launches timed one by one after
a cache flush.

FLOP count: 2*M*N*K per call (one multiply and one add per (i, j, k); the
count "SGEMM CUDA kernel (First Half)", "Part 4", gives as 2MNK, and with which
"1D Register Tiling: One Thread, TM Outputs" turns 10.506 ms at 4096^3 into
13081.8 GFLOP/s).  The epilogue's alpha/beta operations are not counted.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from fp32_gemm_05_amd.roofline import (FP32_PEAK_TFLOPS, FP32_VALU_PEAK_TFLOPS, HBM_PEAK_GBS,  # noqa: E402
                                       algorithmic_bytes, gemm_flops)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def stored_traffic(workload: str, variant: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they match this kernel build."""
    path = os.path.join(ROOT, "profiles", f"traffic_{variant}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from fp32_gemm_05_amd.profiling import kernel_source_hash
    if rec.get("kernel_source_hash") != kernel_source_hash(variant):
        return None
    return rec.get("hbm_bytes_per_launch")


def resolve_variant(sg, spec: str) -> int:
    """A --variant argument as a variant id: an id, a variant name, or -1 (dispatch)."""
    spec = str(spec).strip()
    if spec.lstrip("-").isdigit():
        return int(spec)
    for i in range(sg.sgemm_num_variants()):
        if sg.sgemm_variant_name(i) == spec:
            return i
    raise SystemExit(f"bench.py: no kernel variant named {spec!r}")


def host_cpu_model() -> str | None:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def preroll(step, record_event, step_ms: float, seconds: float, smi: bool = False, settle_s: float = 1.5,
            n_samples: int = 3, spacing_s: float = 1.0):
    """Back-to-back steps for at least `seconds` (about two 20 ms batches kept queued), so that the
    timed region starts at the engine clock this workload sustains.  With smi, amd-smi's per-XCD
    gfx clocks are also read n_samples times, spacing_s apart, after settle_s of load (the reading
    is a snapshot the driver refreshes about once a second), and the pre-roll lasts as long as that
    takes.  Returns (steps launched, seconds, median over samples of the XCD mean in MHz or None)."""
    import shutil
    import subprocess
    import threading

    vals, done = [], threading.Event()
    exe = shutil.which("amd-smi") if smi else None

    def poll():
        try:
            time.sleep(settle_s)
            for i in range(n_samples):
                if i:
                    time.sleep(spacing_s)
                r = subprocess.run([exe, "metric", "-g", "0", "-c", "--json"], capture_output=True, text=True,
                                   timeout=8)
                d = json.loads(r.stdout)
                gpu = d["gpu_data"][0] if isinstance(d, dict) else d[0]
                xs = [v["clk"]["value"] for k, v in gpu["clock"].items()
                      if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                      and isinstance(v["clk"].get("value"), (int, float))]
                if xs:
                    vals.append(sum(xs) / len(xs))
        except (OSError, ValueError, KeyError, IndexError, TypeError, subprocess.SubprocessError):
            pass
        finally:
            done.set()

    if seconds <= 0 and exe is None:
        return 0, 0.0, None
    batch = max(1, int(20.0 / max(step_ms, 1e-3)))
    th = None
    if exe is not None:
        th = threading.Thread(target=poll, daemon=True)
        th.start()
    prev = None
    n = 0
    t0 = time.perf_counter()
    cap = max(seconds, 15.0 if exe is not None else 0.0)
    while time.perf_counter() - t0 < cap:
        if time.perf_counter() - t0 >= seconds and (th is None or done.is_set()):
            break
        for _ in range(batch):
            step()
        n += batch
        ev = record_event()
        if prev is not None:
            prev.synchronize()
        prev = ev
    if prev is not None:
        prev.synchronize()
    dt = time.perf_counter() - t0
    if th is not None:
        th.join(timeout=1.0)
    vals.sort()
    return n, dt, (vals[len(vals) // 2] if vals else None)


def cpu_baseline(A, B, C0, w, out_gpu, target_s: float = 15.0, full: bool = False, threads: int = 0):
    """Time the float64 oracle on a bounded sample of the same workload (leading rows of C), or on
    the whole workload with full=True; threads <= 0 means all host threads.

    The oracle's values on those rows also check the GPU output of the first call.
    Returns (record for the JSON line, parity summary).
    """
    import numpy as np

    import oracle

    threads = threads if threads > 0 else len(os.sched_getaffinity(0))
    flops_per_row = 2.0 * w.N * w.K
    probe = min(w.M, 16)
    t0 = time.perf_counter()
    oracle.ref_rows(A, B, C0, w.alpha, w.beta, rows=(0, probe), nthreads=threads)
    t_probe = max(time.perf_counter() - t0, 1e-6)
    rate = probe * flops_per_row / t_probe
    rows = w.M if full else int(min(w.M, max(probe, rate * target_s / flops_per_row)))
    # in blocks of about 10 s, each logged, so that a long full-workload run shows progress
    chunk = max(1, int(rate * 10.0 / flops_per_row))
    parts_ref, parts_bound = [], []
    t0 = time.perf_counter()
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        rr, bb = oracle.ref_rows(A, B, C0, w.alpha, w.beta, rows=(r0, r1), nthreads=threads)
        parts_ref.append(rr)
        parts_bound.append(bb)
        if rows > chunk:
            log(f"oracle: rows {r1}/{rows} after {time.perf_counter() - t0:.1f} s")
    dt = time.perf_counter() - t0
    ref = np.concatenate(parts_ref) if parts_ref else np.zeros((0, w.N))
    bound = np.concatenate(parts_bound) if parts_bound else np.zeros((0, w.N))
    used = min(threads, oracle.max_threads())
    got = out_gpu[:rows].astype(np.float64)
    err_ratio = np.abs(got - ref) / bound
    parity = {
        "rows_checked": rows,
        "max_err_over_bound": float(err_ratio.max()) if rows else 0.0,
        "pass": bool(np.isfinite(got).all() and (err_ratio <= 1.0).all()),
    }
    rec = {
        "value": rows * flops_per_row / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": used,
        "kind": "oracle",
        "sample": f"rows 0..{rows} of C ({rows}x{w.N} outputs, K={w.K}), float64 i-j-k loop, "
                  f"{dt:.1f} s wall",
        "seconds": dt,
    }
    return rec, parity


def cpu_blocked_baseline(A, B, C0, w, reps: int = 3):
    """Time the cache-blocked CPU SGEMM (cpu_blocked/) on the whole workload, on all host threads:
    one untimed call, then the best of `reps` timed calls."""
    import cpu_blocked

    threads = len(os.sched_getaffinity(0))
    C = C0.copy()
    cpu_blocked.gemm(A, B, C, w.alpha, w.beta, nthreads=threads)
    best = float("inf")
    for _ in range(reps):
        C[...] = C0
        t0 = time.perf_counter()
        cpu_blocked.gemm(A, B, C, w.alpha, w.beta, nthreads=threads)
        best = min(best, time.perf_counter() - t0)
    return {
        "value": round(2.0 * w.M * w.N * w.K / best / 1e12, 4),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "blocked",
        "isa": cpu_blocked.isa(),
        "sample": f"the whole {w.M}x{w.N}x{w.K} workload, fp32 cache-blocked with packed panels, best of "
                  f"{reps} ({best:.3f} s)",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--smi", action="store_true",
                    help="also read amd-smi's gfx clocks during the pre-roll (which then lasts about 4 s)")
    ap.add_argument("--no-sclk", action="store_true", help="no amd-smi reading (the default; kept for old commands)")
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    # the engine clock ramps up over the first tens of milliseconds of sustained MFMA work
    ap.add_argument("--preroll", type=float, default=1.0, metavar="SECONDS",
                    help="seconds of back-to-back steps before the warmup (reported in the line; 0: none)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--variant", default="-1", help="force a kernel variant, by id or name (default: dispatch)")
    ap.add_argument("--op", default="NN", choices=["NN", "NT", "TN", "TT"],
                    help="storage of A and B: op(A) op(B), T = stored transposed (sgemm_op)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle on the whole workload instead of a bounded sample of rows")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (default: all host threads)")
    ap.add_argument("--cold", action="store_true",
                    help="read a 512 MiB buffer before every timed launch (evicts the operands from the L2s "
                         "and the Infinity Cache, leaving clean lines, so the operands come from HBM); each "
                         "launch is then timed between its own two events")
    ap.add_argument("--shard-rows", type=int, default=1, metavar="G",
                    help="time one GPU's share of the workload split by rows over G GPUs (the first "
                         "ceil(M/G) rows of A and C, all of B) on this GPU; no collective is run")
    ap.add_argument("--cold-dirty", action="store_true",
                    help="as --cold, but overwrite the 512 MiB buffer instead: the caches then hold dirty lines "
                         "whose write-back competes with the timed launch")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): libsgemm is a single-GPU "
              f"library and no multi-GPU path is built.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import fp32_gemm_05_amd as sg
    from fp32_gemm_05_amd.build import build, is_stale
    from fp32_gemm_05_amd.workloads import HEADLINE, WORKLOADS, make_inputs

    if not os.path.exists(sg.library_path()) or is_stale():
        log("libsgemm.so missing or stale: building")
        build()
    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1

    w = WORKLOADS[args.workload or HEADLINE]
    if args.shard_rows > 1:
        from dataclasses import replace
        w = replace(w, name=f"{w.name}_rows1of{args.shard_rows}", M=-(-w.M // args.shard_rows))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload: {w.describe()}")
    A, B, C0 = make_inputs(w)
    ta, tb = args.op[0], args.op[1]
    # the stored operands: A^T is K x M, B^T is N x K
    As = np.ascontiguousarray(A.T) if ta == "T" else A
    Bs = np.ascontiguousarray(B.T) if tb == "T" else B
    lda, ldb = As.shape[1], Bs.shape[1]
    dA = torch.from_numpy(As).to(dev)
    dB = torch.from_numpy(Bs).to(dev)
    dC = torch.from_numpy(C0).to(dev)
    forced = resolve_variant(sg, args.variant)
    vid = forced if forced >= 0 else sg.sgemm_op_select_variant(ta, tb, w.M, w.N, w.K, dA, lda, dB, ldb, dC, w.N)
    vname = sg.sgemm_variant_name(vid)
    info = sg.sgemm_variant_info(vid)
    log(f"variant: {vname} {info}")
    stream = torch.cuda.current_stream()

    if args.op == "NN":
        def step():
            sg.sgemm_ex(w.M, w.N, w.K, w.alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb, w.beta,
                        dC.data_ptr(), w.N, stream=stream.cuda_stream, variant=forced)
    else:
        def step():
            sg.sgemm_op_ex(ta, tb, w.M, w.N, w.K, w.alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb, w.beta,
                           dC.data_ptr(), w.N, stream=stream.cuda_stream, variant=forced)

    from fp32_gemm_05_amd.profiling import SclkProbe, launch_floor_ms

    def record_event():
        ev = torch.cuda.Event()
        ev.record(stream)
        return ev

    # everything the measurement needs is set up before the pre-roll: a pause of tens of
    # milliseconds between the pre-roll and the timed region (loading a library, allocating) lets
    # the engine clock drop again, and the timed region would then re-time its ramp
    probe_before, probe_after = SclkProbe(), SclkProbe()
    floor_grid = -(-w.M // info["BM"]) * -(-w.N // info["BN"])
    launch_floor_ms(floor_grid, info["threads"], info["lds_bytes"], 1, stream, warmup=1)

    # first call: its output is the one checked against the oracle
    step()
    torch.cuda.synchronize()
    out_first = dC.cpu().numpy()

    # a rough step time for the pre-roll's batching
    t0 = time.perf_counter()
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    rough_ms = (time.perf_counter() - t0) * 1e3 / 3
    pre_steps, pre_s, smi_mhz = preroll(step, record_event, rough_ms, args.preroll, smi=args.smi and not args.no_sclk)
    # straight on into the warmup (the pre-roll returns as soon as its queue has drained)
    for _ in range(args.warmup):
        step()
    log(f"pre-roll: {pre_steps} steps in {pre_s:.2f} s")
    n_spread = 0
    cold = args.cold or args.cold_dirty
    if cold:
        # 512 MiB > the 256 MB Infinity Cache and every L2: the flush before each launch evicts the
        # operands.  Launch i is timed between its own events (the flush is outside them).
        flush = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device=dev)
        flush_out = torch.empty((), dtype=torch.float32, device=dev)
        ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        probe_before.launch(stream)
        for i in range(args.steps):
            if args.cold_dirty:
                flush.fill_(float(i))
            else:
                torch.sum(flush, dim=0, out=flush_out)
            ev_s[i].record(stream)
            step()
            ev_e[i].record(stream)
        probe_after.launch(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        per_launch = np.array([a.elapsed_time(b) for a, b in zip(ev_s, ev_e)])
        total_ms = float(per_launch.sum())
        del flush, flush_out
    else:
        # Two events on the kernels' stream bracket the K back-to-back launches; the mean launch
        # duration is the timed region over K (events between launches would add their own gaps).
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        probe_before.launch(stream)
        ev0.record(stream)
        for i in range(args.steps):
            step()
        ev1.record(stream)
        probe_after.launch(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = ev0.elapsed_time(ev1)
        # the spread of single launches, from a separate pass after the timed region
        n_spread = min(args.steps, 50)
        ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread)]
        ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread)]
        for i in range(n_spread):
            ev_s[i].record(stream)
            step()
            ev_e[i].record(stream)
        torch.cuda.synchronize()
        per_launch = np.array([a.elapsed_time(b) for a, b in zip(ev_s, ev_e)])
    ms_per_step = total_ms / args.steps
    sclk_before, sclk_after = probe_before.mhz(), probe_after.mhz()
    log(f"engine clock (on-GPU probe): {sclk_before} MHz right before the timed region, {sclk_after} MHz right after")
    # the launch floor: an empty kernel with this variant's grid, workgroup size and LDS
    floor_ms = launch_floor_ms(floor_grid, info["threads"], info["lds_bytes"], args.steps, stream)
    log(f"dispatch plan: first=1 rough=3 preroll={pre_steps} warmup={args.warmup} timed={args.steps} "
        f"single={n_spread} floor={args.steps + 20}")
    log(f"launch floor: empty kernel, {floor_grid} workgroups of {info['threads']} threads, "
        f"{info['lds_bytes']} B LDS: {floor_ms * 1e3:.2f} us per launch")
    flops = gemm_flops(w.M, w.N, w.K)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    # cold: the mean of the individually timed launches (the flushes between them are excluded);
    # warm: the timed region over K
    avg_launch_ms = float(per_launch.mean()) if cold else ms_per_step
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    log(f"timed {args.steps} steps{' (cold)' if cold else ''}: {total_ms:.3f} ms events, "
        f"{wall * 1e3:.3f} ms wall; mean launch {avg_launch_ms:.4f} ms; {len(per_launch)} single launches: "
        f"median {float(np.median(per_launch)):.4f}, min {per_launch.min():.4f}, max {per_launch.max():.4f}")

    is_mfma = info["kind"] == "mfma"
    peak = FP32_PEAK_TFLOPS if is_mfma else FP32_VALU_PEAK_TFLOPS
    traffic = stored_traffic(w.name, vname)
    alg_bytes = algorithmic_bytes(w.M, w.N, w.K, w.beta)
    compute_roof = {
        "bound": "mfma" if is_mfma else "alu",
        "achieved": round(achieved, 3),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
    }
    if w.roofline == "hbm":
        # algorithmic bytes per launch over the same mean launch duration, against HBM
        gbps = alg_bytes / (avg_launch_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbps / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        roofline = compute_roof
    line = {
        "metric": "SGEMM TFLOP/s and % of FP32 peak at M=N=K=4096 on 1 MI355X",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"sgemm{'' if args.op == 'NN' else '_op ' + args.op} {w.M}x{w.N}x{w.K} "
                         f"alpha={w.alpha:g} beta={w.beta:g} {w.dist} seed={w.seed}"
                         + (f" (one GPU's row share of a {args.shard_rows}-GPU split)" if args.shard_rows > 1 else "")),
            "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
            "op": args.op, "variant": vname,
        },
        "pct_fp32_peak": round(100.0 * tflops / FP32_PEAK_TFLOPS, 2),
        "launch_median_ms": round(float(np.median(per_launch)), 5),
        "launch_min_ms": round(float(per_launch.min()), 5),
        "cold": "dirty" if args.cold_dirty else bool(args.cold),
        "alg_GBps": round(alg_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "pct_hbm_peak_alg": round(100.0 * alg_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "roofline": roofline,
        "preroll": {"seconds": round(pre_s, 3), "steps": pre_steps},
        # the engine clock right before and right after the timed region, read on the GPU on the
        # kernels' stream (shader cycles over real-time ticks of a probe kernel), and the share of
        # the FP32 peak at their mean (the 157.3 figure assumes 2.4 GHz)
        "sclk_mhz": {"before": round(sclk_before, 1) if sclk_before else None,
                     "after": round(sclk_after, 1) if sclk_after else None},
        "pct_fp32_peak_at_sclk": round(100.0 * achieved / (FP32_PEAK_TFLOPS * (sclk_before + sclk_after) / 2
                                                           / 2400.0), 2) if sclk_before and sclk_after else None,
        "launch_floor": {"us": round(floor_ms * 1e3, 3), "workgroups": floor_grid, "threads": info["threads"],
                         "lds_bytes": info["lds_bytes"], "floor_over_launch": round(floor_ms / avg_launch_ms, 4)},
        "host_cpu": host_cpu_model(),
    }
    if smi_mhz is not None:
        line["sclk_mhz_smi_preroll"] = round(smi_mhz, 1)
    if roofline is not compute_roof:
        line["roofline_compute"] = compute_roof
    if not args.no_cpu_baseline:
        rec, parity = cpu_baseline(A, B, C0, w, out_first, full=args.cpu_full, threads=args.cpu_threads)
        line["cpu_baseline"] = {k: rec[k] for k in ("value", "unit", "cores", "kind", "sample")}
        line["cpu_baseline"]["value"] = round(rec["value"], 6)
        line["parity"] = parity
        log(f"oracle: {rec['sample']} on {rec['cores']} threads; parity {parity}")
        if not parity["pass"]:
            log("PARITY FAILURE: the timed kernel's output is outside the oracle bound")
        # a second, fairer CPU figure: the blocked fp32 SGEMM on the same workload
        line["cpu_blocked"] = cpu_blocked_baseline(A, B, C0, w)
        log(f"blocked CPU SGEMM: {line['cpu_blocked']}")
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0 if line.get("parity", {"pass": True})["pass"] else 3


if __name__ == "__main__":
    sys.exit(main())
