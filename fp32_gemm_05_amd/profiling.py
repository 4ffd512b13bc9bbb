"""rocprofv3 helpers for libsgemm's measurements.

    python -m fp32_gemm_05_amd.profiling copy --mib 1024 --reps 3
        a plain device-to-device copy of known size; run under `rocprofv3 --pmc FETCH_SIZE`
        (then WRITE_SIZE) it calibrates how many bytes one KiB of each counter stands for.
    python -m fp32_gemm_05_amd.profiling read --mib 256 [--mode warm|cold|cold-dirty]
        a streaming read of known size (a hand-written read kernel, libhbm_read.so), warm or after
        evicting the caches: the read bandwidth an HBM-bound kernel can expect under the same protocol.
    python -m fp32_gemm_05_amd.profiling stats <kernel_stats.csv> --command "..." --out X.md
        short text summary of a `rocprofv3 --kernel-trace --stats` run.
    python -m fp32_gemm_05_amd.profiling traffic --kernel SUBSTR --fetch F.csv --write W.csv
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --workload NAME --variant NAME --out X.json
        HBM bytes per launch of one kernel from two --pmc runs, each scaled by the copy calibration.
    python -m fp32_gemm_05_amd.profiling counters <counter_collection.csv> --kernel SUBSTR --out X.md
        per-dispatch means of any collected counters for one kernel.
    python -m fp32_gemm_05_amd.profiling series <kernel_trace.csv> --log BENCH_STDERR --command "..." --out X.md
        per-phase durations of a traced bench run (first call, pre-roll, warmup, timed region, ...).
    python -m fp32_gemm_05_amd.profiling collect --dir D --workload W [--warmup N] [--out-dir profiles]
        runs every rocprofv3 pass below (each as a child process with its own time limit) and then
        `report`: the one command behind each committed summary.
    python -m fp32_gemm_05_amd.profiling report --dir D --workload W --out-dir profiles
        one summary per (kernel, workload) from the runs the profiling commands below leave in D:
          D/trace_W   rocprofv3 --kernel-trace --stats ... -- python bench.py --workload W --no-cpu-baseline --no-sclk
          D/fetch_W   rocprofv3 --pmc FETCH_SIZE ...        -- python bench.py --workload W --steps 3 --warmup 1 --no-cpu-baseline --no-sclk
          D/write_W   rocprofv3 --pmc WRITE_SIZE ...        (same bench command)
          D/rdreq_W   rocprofv3 --pmc TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum ...
          D/sq_W      rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT
                      SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVES SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE ...
          D/copy_fetch, D/copy_write, D/copy_rdreq: the same counters over `profiling copy --mib 1024 --reps 3`

No arithmetic of the GEMM lives here; this is measurement plumbing only.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

from .roofline import FP32_PEAK_TFLOPS, algorithmic_bytes, gemm_flops, panel_read_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# The files that fix what runs on the GPU for a given variant: the shared kernel pieces, the
# variant's kernel family, and how each variant is launched.  The dispatch (which variant a call
# gets) is not included: the counter summaries are per variant, so a retuned table leaves them
# valid, and so does a change to another kernel family.
KERNEL_COMMON = ("kernel_common.hpp", "sgemm_launch.hpp")
# kernel family of a variant, by its name's prefix
KERNEL_FAMILIES = (("mfma32p_", "kernel_pipe.hpp"), ("mfma32d_", "kernel_deep.hpp"), ("mfma32k", "kernel_splitk.hpp"),
                   ("mfma32r_", "kernel_direct.hpp"), ("mfma32l_", "kernel_dl.hpp"), ("mfma32_", "kernel_mfma.hpp"),
                   ("valu_", "kernel_valu.hpp"))


def kernel_sources(variant: str):
    """The source files whose text determines the code a variant runs."""
    fam = next((f for prefix, f in KERNEL_FAMILIES if variant.startswith(prefix)), None)
    return KERNEL_COMMON + ((fam,) if fam else ())


def _strip_variant_table(text: bytes) -> bytes:
    """The launch source without its variant table (the row macros and the rows, from the table's
    header comment to the end of the array): adding or editing other variants' rows leaves every
    kernel's own code, and so its counters, unchanged; a row's name spells out its configuration
    and is hashed separately."""
    start = text.find(b"// ---- The variant table:")
    if start < 0:
        start = text.find(b"const Variant kVariants[] = {")
    if start < 0:
        return text
    end = text.find(b"\n};", text.find(b"const Variant kVariants[] = {", start))
    return text[:start] + text[end:] if end >= 0 else text


def kernel_source_hash(variant: str) -> str:
    """Hash of the kernel code a variant runs: the shared kernel pieces and its family's kernel
    template, the launch code (without the variant table) and the variant's name, which spells out
    its template configuration."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp32_gemm_05_amd", "csrc")
    for name in kernel_sources(variant):
        with open(os.path.join(csrc, name), "rb") as f:
            text = f.read()
        if name == "sgemm_launch.hpp":
            text = _strip_variant_table(text)
        h.update(name.encode() + b"\0" + text)
    h.update(b"variant\0" + variant.encode())
    return h.hexdigest()[:16]


def run_copy(mib: int, reps: int) -> None:
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy: {reps} x {mib} MiB device-to-device ({2 * mib} MiB of traffic each)", flush=True)


def _hbm_read_lib():
    import ctypes
    from .build import HBM_READ_LIB, build_hbm_read
    if not os.path.exists(HBM_READ_LIB):
        build_hbm_read()
    lib = ctypes.CDLL(HBM_READ_LIB)
    lib.hbm_read_workgroups.restype = ctypes.c_long
    lib.hbm_read_workgroups.argtypes = [ctypes.c_long, ctypes.c_int]
    lib.hbm_read.restype = ctypes.c_int
    lib.hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def launch_refs_lib():
    """liblaunch_refs.so: the empty kernel of the launch floor and the engine-clock probe."""
    import ctypes
    from .build import LAUNCH_REFS_LIB, build_launch_refs
    if not os.path.exists(LAUNCH_REFS_LIB):
        build_launch_refs()
    lib = ctypes.CDLL(LAUNCH_REFS_LIB)
    lib.launch_floor.restype = ctypes.c_int
    lib.launch_floor.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.sclk_probe.restype = ctypes.c_int
    lib.sclk_probe.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p]
    lib.wall_clock_khz.restype = ctypes.c_int
    lib.wall_clock_khz.argtypes = []
    return lib


class SclkProbe:
    """The engine clock at one point of a stream: a probe kernel of one workgroup per XCD spins for
    `ticks` ticks of the constant-rate real-time counter and counts shader cycles meanwhile.
    launch() enqueues it (no host synchronisation); mhz() reads the result afterwards: the mean
    over the workgroups of cycles / ticks x the real-time counter's rate."""

    def __init__(self, nblocks: int = 8, ticks: int = 2000):
        import torch
        self.lib = launch_refs_lib()
        self.nblocks, self.ticks = nblocks, ticks
        self.buf = torch.zeros(2 * nblocks, dtype=torch.int64, device="cuda")
        self.khz = self.lib.wall_clock_khz()

    def launch(self, stream) -> None:
        rc = self.lib.sclk_probe(self.nblocks, self.ticks, self.buf.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"sclk_probe returned {rc}")

    def mhz(self):
        v = self.buf.cpu().tolist()
        ratios = [c / t for c, t in zip(v[0::2], v[1::2]) if t > 0]
        if not ratios or self.khz <= 0:
            return None
        return sum(ratios) / len(ratios) * self.khz / 1000.0


def launch_floor_ms(nwg: int, threads: int, lds_bytes: int, steps: int, stream, warmup: int = 20) -> float:
    """Mean time per launch of an empty kernel with the given grid, workgroup size and LDS, timed
    as the bench times a GEMM: `steps` back-to-back launches between two events on `stream`."""
    import torch
    lib = launch_refs_lib()

    def go():
        rc = lib.launch_floor(nwg, threads, lds_bytes, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"launch_floor returned {rc}")

    for _ in range(warmup):
        go()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        go()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def run_read(mib: int, reps: int, mode: str, chunk_kib: int = 1024) -> None:
    """Read-bandwidth reference: a hand-written streaming read (csrc/hbm_read.hip: each workgroup
    reads one contiguous chunk with eight 128-bit loads in flight per thread) over `mib` MiB, each
    read timed between its own events.  mode: "warm" (back-to-back), "cold" (a 512 MiB buffer is
    read before every timed read: the operands leave the L2s and the Infinity Cache, which then
    hold clean lines) or "cold-dirty" (the 512 MiB buffer is overwritten instead: dirty lines are
    written back while the timed read runs) -- the protocols of bench.py, --cold and --cold-dirty."""
    import torch
    lib = _hbm_read_lib()
    nbytes = mib * 1024 * 1024
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    nwg = lib.hbm_read_workgroups(nbytes, chunk_kib)
    out = torch.empty(nwg * 256, dtype=torch.float32, device="cuda")
    flush = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device="cuda") if mode != "warm" else None
    fout = torch.empty(lib.hbm_read_workgroups(flush.numel() * 4, chunk_kib) * 256, dtype=torch.float32,
                       device="cuda") if flush is not None else None
    stream = torch.cuda.current_stream()

    def read(buf, o):
        rc = lib.hbm_read(buf.data_ptr(), buf.numel() * 4, chunk_kib, o.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hbm_read returned {rc}")

    for _ in range(200):  # the engine clock ramps up under sustained load
        read(x, out)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (e0, e1) in enumerate(evs):
        if mode == "cold":
            read(flush, fout)
        elif mode == "cold-dirty":
            flush.fill_(float(i))
        e0.record(stream)
        read(x, out)
        e1.record(stream)
    torch.cuda.synchronize()
    times = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    med = times[len(times) // 2]
    print(f"read: {mib} MiB {mode}, median {med * 1e3:.1f} us (min {times[0] * 1e3:.1f}) over {reps} -> "
          f"{nbytes / (med * 1e-3) / 1e12:.2f} TB/s", flush=True)


def _read_counters(path: str, kernel_substr: str):
    """{counter: [value per dispatch]} for dispatches whose kernel name contains kernel_substr."""
    per = defaultdict(dict)
    with open(path) as f:
        for row in csv.DictReader(f):
            if kernel_substr not in row["Kernel_Name"]:
                continue
            per[row["Dispatch_Id"]][row["Counter_Name"]] = float(row["Counter_Value"])
    out = defaultdict(list)
    for d in per.values():
        for k, v in d.items():
            out[k].append(v)
    return out


def _dispatches(path: str, kernel_substr: str):
    """[(counters dict, duration ns)] per dispatch of the matching kernel, in dispatch order."""
    per = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if kernel_substr not in row["Kernel_Name"]:
                continue
            d = per.setdefault(int(row["Dispatch_Id"]), [{}, 0])
            d[0][row["Counter_Name"]] = float(row["Counter_Value"])
            d[1] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    return [tuple(per[k]) for k in sorted(per)]


def _mean(xs):
    return sum(xs) / len(xs) if xs else float("nan")


def cmd_stats(args) -> None:
    with open(args.csv) as f:
        rows = list(csv.DictReader(f))
    lines = [f"# rocprofv3 kernel trace: {args.title}", "", "Command:", "", "```", args.command, "```", "",
             "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} % |")
    if args.note:
        lines += ["", args.note]
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


def cmd_traffic(args) -> None:
    fetch = _mean(_read_counters(args.fetch, args.kernel)["FETCH_SIZE"])
    write = _mean(_read_counters(args.write, args.kernel)["WRITE_SIZE"])
    cfetch = _mean(_read_counters(args.copy_fetch, args.copy_kernel)["FETCH_SIZE"])
    cwrite = _mean(_read_counters(args.copy_write, args.copy_kernel)["WRITE_SIZE"])
    # the copy reads copy_bytes and writes copy_bytes
    f_scale = args.copy_bytes / (cfetch * 1024.0)
    w_scale = args.copy_bytes / (cwrite * 1024.0)
    hbm = fetch * 1024.0 * f_scale + write * 1024.0 * w_scale
    rec = {
        "workload": args.workload, "variant": args.variant, "kernel_match": args.kernel,
        "FETCH_SIZE_KiB_per_launch": fetch, "WRITE_SIZE_KiB_per_launch": write,
        "copy_bytes": args.copy_bytes, "copy_FETCH_SIZE_KiB": cfetch, "copy_WRITE_SIZE_KiB": cwrite,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": args.alg_bytes,
        "kernel_source_hash": kernel_source_hash(args.variant), "commands": args.commands,
    }
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def cmd_counters(args) -> None:
    c = _read_counters(args.csv, args.kernel)
    lines = [f"# rocprofv3 counters: {args.title}", "", "Command:", "", "```", args.command, "```", "",
             f"Kernel match: `{args.kernel}`; dispatches: {max((len(v) for v in c.values()), default=0)}", "",
             "| Counter | Mean per dispatch |", "|---|---|"]
    for k in sorted(c):
        lines.append(f"| {k} | {_mean(c[k]):.6g} |")
    if args.note:
        lines += ["", args.note]
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


def cmd_series(args) -> None:
    """Per-phase durations of a traced bench run: the GEMM kernel's dispatches in order, split by
    the bench's "dispatch plan" line (first call, step-time probe, pre-roll, warmup, timed region,
    single launches), with the duration of every dispatch of the first and last phases shown."""
    import re
    with open(args.log) as f:
        plan = next((l for l in f if l.startswith("dispatch plan:")), None)
    if plan is None:
        raise SystemExit(f"no 'dispatch plan' line in {args.log}")
    phases = [(k, int(v)) for k, v in re.findall(r"(\w+)=(\d+)", plan) if k != "floor"]
    with open(args.csv) as f:
        rows = [r for r in csv.DictReader(f) if args.kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    starts = [int(r["Start_Timestamp"]) for r in rows]
    expect = sum(n for _, n in phases)
    lines = [f"# Dispatch series: {args.title}", "", "Command:", "", "```", args.command, "```", "",
             f"Kernel match: `{args.kernel}`; {len(dur)} dispatches traced, {expect} in the bench's plan "
             f"({plan.strip()[len('dispatch plan: '):]}).", "",
             "| Phase | Dispatches | Mean (us) | Min (us) | Max (us) | First (us) | Last (us) | Span incl. gaps (ms) |",
             "|---|---|---|---|---|---|---|---|"]
    i = 0
    for name, n in phases:
        seg = dur[i:i + n]
        if seg:
            span = (starts[i + n - 1] - starts[i]) / 1e6 + seg[-1] / 1e3
            lines.append(f"| {name} | {n} | {_mean(seg):.1f} | {min(seg):.1f} | {max(seg):.1f} | {seg[0]:.1f} | "
                         f"{seg[-1]:.1f} | {span:.3f} |")
        i += n
    if args.show:
        lines += ["", f"Durations (us) of the first {args.show} dispatches, in order:", "",
                  ", ".join(f"{x:.0f}" for x in dur[:args.show])]
    if args.note:
        lines += ["", args.note]
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


N_XCD, N_CU, N_SIMD = 8, 256, 1024  # MI355X


def _stats_rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _mean_counter(path, substr, name):
    return _mean(_read_counters(path, substr).get(name, []))


def _workload_figures(workload):
    from fp32_gemm_05_amd.workloads import WORKLOADS
    w = WORKLOADS[workload]
    return w, gemm_flops(w.M, w.N, w.K), algorithmic_bytes(w.M, w.N, w.K, w.beta)


def _variant_tile(name):
    """(BM, BN) of the named kernel variant in the built library, or None."""
    from . import _binding as sg
    for i in range(sg.sgemm_num_variants()):
        if sg.sgemm_variant_name(i) == name:
            info = sg.sgemm_variant_info(i)
            return info["BM"], info["BN"]
    return None


def cmd_report(args) -> None:
    d, W = args.dir, args.workload
    w, flops, alg_bytes = _workload_figures(W)
    rows = _stats_rows(os.path.join(d, f"trace_{W}", "run_kernel_stats.csv"))
    kern = [r for r in rows if "sgemm" in r["Name"]]
    if len(kern) != 1:
        raise SystemExit(f"expected one sgemm kernel in the trace of {W}, found {len(kern)}")
    k = kern[0]
    name = k["Name"]
    avg_ns = float(k["AverageNs"])
    # the bench's launches: the first call, the warmup, the timed region (`steps` back-to-back
    # launches) and a pass of min(steps, 50) individually timed launches
    with open(os.path.join(d, f"trace_{W}", "run_kernel_trace.csv")) as f:
        disp = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in csv.DictReader(f)
                if r["Kernel_Name"] == name]
    spread = min(args.steps, 50)
    timed = disp[-(args.steps + spread):-spread]
    timed_ns = _mean(timed)
    # variant name from the kernel signature is not unique; take it from the bench log
    variant = args.variant
    sq = {c: _mean(v) for c, v in _read_counters(os.path.join(d, f"sq_{W}", "run_counter_collection.csv"), "sgemm").items()}
    fetch = _mean_counter(os.path.join(d, f"fetch_{W}", "run_counter_collection.csv"), "sgemm", "FETCH_SIZE")
    write = _mean_counter(os.path.join(d, f"write_{W}", "run_counter_collection.csv"), "sgemm", "WRITE_SIZE")
    rd = {c: _mean(v) for c, v in _read_counters(os.path.join(d, f"rdreq_{W}", "run_counter_collection.csv"), "sgemm").items()}
    cfetch = _mean_counter(os.path.join(d, "copy_fetch", "run_counter_collection.csv"), "copyBuffer", "FETCH_SIZE")
    cwrite = _mean_counter(os.path.join(d, "copy_write", "run_counter_collection.csv"), "copyBuffer", "WRITE_SIZE")
    copy_bytes = 1024.0 ** 3
    f_scale = copy_bytes / (cfetch * 1024.0)
    w_scale = copy_bytes / (cwrite * 1024.0)
    hbm = fetch * 1024.0 * f_scale + write * 1024.0 * w_scale
    rd_bytes = 32 * rd.get("TCC_EA0_RDREQ_32B_sum", 0.0) + 64 * rd.get("TCC_EA0_RDREQ_64B_sum", 0.0) + \
        128 * rd.get("TCC_EA0_RDREQ_128B_sum", 0.0)
    gui = sq.get("GRBM_GUI_ACTIVE", float("nan")) / N_XCD
    mfma_util = sq.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (N_SIMD * gui)
    # the last dispatch of the counter run (after its warmup): engine clock = active cycles per XCD
    # over the dispatch's duration, and that dispatch's MFMA busy fraction
    last_c, last_ns = _dispatches(os.path.join(d, f"sq_{W}", "run_counter_collection.csv"), "sgemm")[-1]
    last_gui = last_c.get("GRBM_GUI_ACTIVE", float("nan")) / N_XCD
    sclk_last = last_gui / last_ns if last_ns > 0 else float("nan")  # cycles per ns = GHz
    mfma_last = last_c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (N_SIMD * last_gui)
    lds_conf = sq.get("SQ_LDS_BANK_CONFLICT", float("nan")) / (N_CU * gui)
    expect_mfma = w.M * w.N * w.K / 2048.0  # 32x32x2 MFMAs of the exact problem (no tile padding)
    tflops = flops / (avg_ns * 1e-9) / 1e12
    tflops_timed = flops / (timed_ns * 1e-9) / 1e12
    tile = _variant_tile(variant)
    panel = panel_read_bytes(w.M, w.N, w.K, *tile) if tile else float("nan")
    bench = "python -u bench.py --workload %s" % W
    trace_opt = f"--trace-args='{args.trace_args}' " if args.trace_args else ""
    sq_warm = args.sq_warmup
    cmds = [
        f"python -m fp32_gemm_05_amd.profiling collect --dir <dir> --workload {W} "
        f"{'--warmup ' + args.trace_args.split()[-1] + ' ' if args.trace_args.startswith('--warmup') else ''}"
        f"(runs all of the following)",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace_{W} -o run -- {bench} "
        f"{args.trace_args + ' ' if args.trace_args else ''}--no-cpu-baseline --no-sclk",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch_{W} -o run -- {bench} --steps 3 --warmup 1 --no-cpu-baseline --no-sclk",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write_{W} -o run -- {bench} --steps 3 --warmup 1 --no-cpu-baseline --no-sclk",
        f"rocprofv3 --pmc TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum --output-format csv -d <dir>/rdreq_{W} -o run -- {bench} --steps 3 --warmup 1 --no-cpu-baseline --no-sclk",
        f"rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVES SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE --output-format csv -d <dir>/sq_{W} -o run -- {bench} --steps 3 --warmup {sq_warm} --no-cpu-baseline --no-sclk",
        "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE, then the three TCC_EA0_RDREQ_*_sum) --output-format csv -d <dir>/copy_fetch (copy_write, copy_rdreq) -o run -- python -u -m fp32_gemm_05_amd.profiling copy --mib 1024 --reps 3",
        f"python -m fp32_gemm_05_amd.profiling report --dir <dir> --workload {W} --variant {variant} "
        f"{trace_opt}--out-dir profiles",
    ]
    lines = [
        f"# `{variant}` on {W}", "",
        f"Workload: {w.describe()}; {flops / 1e9:.2f} GFLOP and {alg_bytes / 1e6:.1f} MB of algorithmic traffic per call.",
        f"Kernel: `{name}`", "",
        "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
        f"| Dispatches | Mean duration | TFLOP/s | % of {FP32_PEAK_TFLOPS} |", "|---|---|---|---|",
        f"| all {k['Calls']} (first call, warmup, timed region, 50 single launches; the --stats average) | {avg_ns / 1e3:.1f} us | "
        f"{tflops:.1f} | {100 * tflops / FP32_PEAK_TFLOPS:.1f} % |",
        f"| the {len(timed)} of the bench's timed region | {timed_ns / 1e3:.1f} us | {tflops_timed:.1f} | "
        f"{100 * tflops_timed / FP32_PEAK_TFLOPS:.1f} % |", "",
        f"Min {float(k['MinNs']) / 1e3:.1f} us, max {float(k['MaxNs']) / 1e3:.1f} us over all dispatches.", "",
        "## Counters (means per dispatch)", "",
        "| Counter | Value |", "|---|---|",
    ]
    for c in sorted(sq):
        lines.append(f"| {c} | {sq[c]:.6g} |")
    lines += [
        f"| FETCH_SIZE (KiB) | {fetch:.6g} |", f"| WRITE_SIZE (KiB) | {write:.6g} |",
    ]
    for c in sorted(rd):
        lines.append(f"| {c} | {rd[c]:.6g} |")
    lines += [
        "", "## Derived", "",
        f"* MFMA instructions: {sq.get('SQ_INSTS_MFMA', float('nan')):.6g} (the problem needs M*N*K/2048 = "
        f"{expect_mfma:.6g} v_mfma_f32_32x32x2_f32; the rest is tile padding at ragged edges)",
        f"* MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs) = {100 * mfma_util:.1f} % "
        f"(mean over the counter run's dispatches); {100 * mfma_last:.1f} % in its last dispatch",
        (f"* Engine clock in the counter run's last dispatch: GRBM_GUI_ACTIVE / 8 XCDs / duration = "
         f"{sclk_last:.2f} GHz ({last_ns / 1e3:.1f} us under counter collection)" if last_ns >= 150_000 else
         f"* Engine clock: not derived (a {last_ns / 1e3:.1f} us dispatch is too short: GRBM_GUI_ACTIVE also "
         f"counts cycles of the counter collection around it, which also lowers the MFMA busy figure)"),
        f"* LDS bank-conflict cycles per CU-cycle: SQ_LDS_BANK_CONFLICT / (256 CUs x GRBM_GUI_ACTIVE / 8) = "
        f"{100 * lds_conf:.2f} %",
        f"* Copy calibration: a {copy_bytes / 2**20:.0f} MiB device copy reads FETCH_SIZE {cfetch:.6g} KiB "
        f"(scale {f_scale:.4f}) and writes WRITE_SIZE {cwrite:.6g} KiB (scale {w_scale:.4f})",
        f"* HBM-side traffic per launch (copy-calibrated FETCH_SIZE + WRITE_SIZE): {hbm / 1e6:.1f} MB "
        f"= {hbm / alg_bytes:.2f} x the algorithmic {alg_bytes / 1e6:.1f} MB",
        f"* L2 read requests by size: {rd_bytes / 1e6:.1f} MB read (32/64/128 B requests counted at their size)",
        (f"* Panel reads of the {tile[0]}x{tile[1]} tiling, K*(1/BM + 1/BN) values per output: {panel / 1e6:.1f} MB "
         f"per launch; the L2 serves all but the L2->fabric traffic above" if tile else
         "* Panel reads: variant not found in the library"),
        "", "## Commands", "", "```", *cmds, "```", "",
    ]
    if args.note:
        lines += [args.note, ""]
    os.makedirs(args.out_dir, exist_ok=True)
    base = f"{variant}__{W}"
    with open(os.path.join(args.out_dir, base + ".md"), "w") as f:
        f.write("\n".join(lines))
    rec = {"workload": W, "variant": variant, "kernel": name, "avg_ns_all_dispatches": avg_ns,
           "avg_ns_timed_region": timed_ns,
           "FETCH_SIZE_KiB_per_launch": fetch, "WRITE_SIZE_KiB_per_launch": write,
           "fetch_scale": f_scale, "write_scale": w_scale, "hbm_bytes_per_launch": hbm,
           "l2_read_bytes_by_request_size": rd_bytes, "algorithmic_bytes_per_launch": alg_bytes,
           "mfma_busy": mfma_util, "mfma_busy_last_dispatch": mfma_last, "sclk_ghz_last_dispatch": sclk_last if last_ns >= 150_000 else None,
           "lds_bank_conflict_per_cu_cycle": lds_conf,
           "kernel_source_hash": kernel_source_hash(variant), "commands": cmds}
    with open(os.path.join(args.out_dir, f"traffic_{variant}_{W}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print("\n".join(lines))


# Counter passes of one summary: each rocprofv3 --pmc run stays within one pass's limits
# (at most 8 SQ counters and 4 TCC counters; FETCH_SIZE alone takes 3 TCC counters).
PMC_PASSES = [
    ("fetch", ["FETCH_SIZE"]),
    ("write", ["WRITE_SIZE"]),
    ("rdreq", ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum"]),
    ("sq", ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_VALU_MFMA_BUSY_CYCLES",
            "SQ_BUSY_CYCLES", "SQ_WAVES", "SQ_INSTS_VALU_MFMA_MOPS_F32", "GRBM_GUI_ACTIVE"]),
]


def _run(cmd, log, timeout):
    """Run one profiler command as a child process (this process never touches the GPU)."""
    import subprocess
    print("+ " + " ".join(cmd), flush=True)
    with open(log, "w") as f:
        res = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, timeout=timeout)
    if res.returncode != 0:
        raise SystemExit(f"command failed ({res.returncode}), see {log}: {' '.join(cmd)}")


def cmd_collect(args) -> None:
    """All the runs one summary needs, then the summary: the copy calibration (once per directory),
    the kernel trace of the bench (with --warmup so that the clock has ramped up), the four counter
    passes, and `report`.  Each profiler run is a child process with its own time limit."""
    d, W = args.dir, args.workload
    os.makedirs(d, exist_ok=True)
    py = sys.executable
    rp = ["rocprofv3", "--output-format", "csv"]
    copy = [py, "-u", "-m", "fp32_gemm_05_amd.profiling", "copy", "--mib", "1024", "--reps", "3"]
    for tag, counters in (("copy_fetch", ["FETCH_SIZE"]), ("copy_write", ["WRITE_SIZE"]),
                          ("copy_rdreq", PMC_PASSES[2][1])):
        if not os.path.isdir(os.path.join(d, tag)):
            _run(rp + ["--pmc", *counters, "-d", os.path.join(d, tag), "-o", "run", "--", *copy],
                 os.path.join(d, tag + ".log"), 120)
    bench = [py, "-u", os.path.join(ROOT, "bench.py"), "--workload", W]
    _run(rp + ["--kernel-trace", "--stats", "-d", os.path.join(d, f"trace_{W}"), "-o", "run", "--", *bench,
               "--warmup", str(args.warmup), "--no-cpu-baseline", "--no-sclk"], os.path.join(d, f"trace_{W}.log"), 300)
    variant = None
    with open(os.path.join(d, f"trace_{W}.log")) as f:
        for line in f:
            if line.startswith("variant: "):
                variant = line.split()[1]
    if variant is None:
        raise SystemExit("the bench did not report its variant")
    for tag, counters in PMC_PASSES:
        _run(rp + ["--pmc", *counters, "-d", os.path.join(d, f"{tag}_{W}"), "-o", "run", "--", *bench,
                   "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-sclk"], os.path.join(d, f"{tag}_{W}.log"), 120)
    report = argparse.Namespace(dir=d, workload=W, variant=variant, steps=200, sq_warmup=1,
                                trace_args=f"--warmup {args.warmup}", out_dir=args.out_dir, note="")
    cmd_report(report)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    p = sub.add_parser("copy")
    p.add_argument("--mib", type=int, default=1024)
    p.add_argument("--reps", type=int, default=3)
    p = sub.add_parser("read")
    p.add_argument("--mib", type=int, default=256)
    p.add_argument("--reps", type=int, default=50)
    p.add_argument("--mode", default="warm", choices=["warm", "cold", "cold-dirty"])
    p.add_argument("--chunk-kib", type=int, default=1024)
    p = sub.add_parser("stats")
    p.add_argument("csv")
    p.add_argument("--title", default="")
    p.add_argument("--command", required=True)
    p.add_argument("--note", default="")
    p.add_argument("--out", required=True)
    p = sub.add_parser("traffic")
    p.add_argument("--kernel", required=True)
    p.add_argument("--copy-kernel", default="copy")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--copy-fetch", required=True)
    p.add_argument("--copy-write", required=True)
    p.add_argument("--copy-bytes", type=float, required=True)
    p.add_argument("--alg-bytes", type=float, default=None)
    p.add_argument("--workload", required=True)
    p.add_argument("--variant", required=True)
    p.add_argument("--commands", nargs="*", default=[])
    p.add_argument("--out", required=True)
    p = sub.add_parser("counters")
    p.add_argument("csv")
    p.add_argument("--kernel", required=True)
    p.add_argument("--title", default="")
    p.add_argument("--command", required=True)
    p.add_argument("--note", default="")
    p.add_argument("--out", required=True)
    p = sub.add_parser("series", help="per-phase dispatch durations of a traced bench run")
    p.add_argument("csv", help="run_kernel_trace.csv of `rocprofv3 --kernel-trace` over bench.py")
    p.add_argument("--log", required=True, help="the bench's stderr (holds its dispatch plan)")
    p.add_argument("--kernel", default="sgemm")
    p.add_argument("--title", default="")
    p.add_argument("--command", required=True)
    p.add_argument("--show", type=int, default=40)
    p.add_argument("--note", default="")
    p.add_argument("--out", required=True)
    p = sub.add_parser("collect", help="run every profiler pass of one workload and write its summary")
    p.add_argument("--dir", required=True, help="where the raw rocprofv3 output goes")
    p.add_argument("--workload", required=True)
    p.add_argument("--warmup", type=int, default=100, help="bench warmup of the traced run")
    p.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    p = sub.add_parser("report")
    p.add_argument("--dir", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--variant", required=True)
    p.add_argument("--steps", type=int, default=200, help="timed steps of the traced bench run")
    p.add_argument("--sq-warmup", type=int, default=1, help="bench warmup of the SQ counter run")
    p.add_argument("--trace-args", default="", help="extra bench.py arguments of the traced run (e.g. a longer "
                   "warmup, so that short kernels are traced at the ramped-up engine clock)")
    p.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    p.add_argument("--note", default="")
    args = ap.parse_args(argv)
    if args.cmd == "report":
        cmd_report(args)
    elif args.cmd == "collect":
        cmd_collect(args)
    elif args.cmd == "copy":
        run_copy(args.mib, args.reps)
    elif args.cmd == "read":
        run_read(args.mib, args.reps, args.mode, args.chunk_kib)
    elif args.cmd == "stats":
        cmd_stats(args)
    elif args.cmd == "traffic":
        cmd_traffic(args)
    elif args.cmd == "counters":
        cmd_counters(args)
    elif args.cmd == "series":
        cmd_series(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
