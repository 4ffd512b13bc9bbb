"""rocprofv3 helpers for libsgemm's measurements.

    python -m fp32_gemm_05_amd.profiling copy --mib 1024 --reps 3
        a plain device-to-device copy of known size; run under `rocprofv3 --pmc FETCH_SIZE`
        (then WRITE_SIZE) it calibrates how many bytes one KiB of each counter stands for.
    python -m fp32_gemm_05_amd.profiling read --mib 256 [--mode warm|cold|cold-dirty]
        a streaming read of known size (a hand-written read kernel, libhbm_read.so), warm or after
        evicting the caches: the read bandwidth an HBM-bound kernel can expect under the same protocol.
    python -m fp32_gemm_05_amd.profiling write --m 8192 --n 8192
        a matrix written in 64x64 tiles in the MFMA epilogue's store order (plain and nontemporal
        stores) and by torch's fill_: the write bandwidth a store-heavy shape can expect.
    python -m fp32_gemm_05_amd.profiling stats <kernel_stats.csv> --command "..." --out X.md
        short text summary of a `rocprofv3 --kernel-trace --stats` run.
    python -m fp32_gemm_05_amd.profiling traffic --kernel SUBSTR --fetch F.csv --write W.csv
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --workload NAME --variant NAME --out X.json
        HBM bytes per launch of one kernel from two --pmc runs, each scaled by the copy calibration.
    python -m fp32_gemm_05_amd.profiling counters <counter_collection.csv> --kernel SUBSTR --out X.md
        per-dispatch means of any collected counters for one kernel.
    python -m fp32_gemm_05_amd.profiling series <kernel_trace.csv> --log BENCH_STDERR --command "..." --out X.md
        per-phase durations of a traced bench run (first call, pre-roll, warmup, timed region, ...).
    python -m fp32_gemm_05_amd.profiling phases --workload W [--variant NAME]
        per-wave prologue / K loop / epilogue cycles of one launch from the phase-stamp build
        (libsgemm_stamps.so), next to the back-to-back launch time, the launch floor and the K
        loop's MFMA ideal (runs on the GPU itself, not under a profiler).
    python -m fp32_gemm_05_amd.profiling lds-probe   (under rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS)
    python -m fp32_gemm_05_amd.profiling lds-passes <counter_collection.csv> --out X.md
        which lanes of one 32-, 64- or 128-bit LDS access share a pass, from lane-pair patterns.
    python -m fp32_gemm_05_amd.profiling collect --dir D --workload W [--variant NAME] [--warmup N] [--out-dir profiles]
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
                   ("mfma32r_", "kernel_direct.hpp"), ("mfma32l_", "kernel_dl.hpp"), ("mfma16l_", "kernel_dl.hpp"),
                   ("mfma32_", "kernel_mfma.hpp"),
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
    lib.hbm_write_tiles.restype = ctypes.c_int
    lib.hbm_write_tiles.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
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
    lib.lds_probe.restype = ctypes.c_int
    lib.lds_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mfma_chain.restype = ctypes.c_int
    lib.mfma_chain.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p]
    return lib


def mfma_cycles(kind: int, stream, ilp: int = 4, n: int = 4096, nblocks: int = 256):
    """Shader cycles per MFMA of shape kind (32: 32x32x2, 16: 16x16x4 f32) at one wave per SIMD,
    issued as `ilp` interleaved dependent chains (ilp = 4: the issue rate, with no wait for a
    previous result): (median, min, max) over the waves of the chain kernel."""
    import torch
    lib = launch_refs_lib()
    cyc = torch.zeros(4 * nblocks, dtype=torch.int64, device="cuda")
    sink = torch.empty(256 * nblocks, dtype=torch.float32, device="cuda")
    for _ in range(3):  # the last launch's cycles are kept
        rc = lib.mfma_chain(nblocks, n, kind, ilp, cyc.data_ptr(), sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"mfma_chain returned {rc}")
    torch.cuda.synchronize()
    c = sorted(x / n for x in cyc.cpu().tolist())
    return c[len(c) // 2], c[0], c[-1]


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


def run_write(m: int, n: int, reps: int) -> None:
    """Write-bandwidth reference: an m x n matrix written in 64x64 tiles in the MFMA epilogue's
    store order (csrc/hbm_read.hip, hbm_write_tiles), with plain and with nontemporal stores, next
    to torch's fill_ of the same buffer; medians of back-to-back writes, each between its own
    events, after 200 untimed ones."""
    import torch
    lib = _hbm_read_lib()
    buf = torch.empty(m * n, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    nbytes = m * n * 4

    def tiles(nt):
        rc = lib.hbm_write_tiles(buf.data_ptr(), m, n, n, nt, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hbm_write_tiles returned {rc}")

    for label, go in (("tile order, plain stores", lambda: tiles(0)),
                      ("tile order, nontemporal stores", lambda: tiles(1)),
                      ("torch fill_", lambda: buf.fill_(2.0))):
        for _ in range(200):
            go()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(stream)
            go()
            e1.record(stream)
        torch.cuda.synchronize()
        times = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        med = times[len(times) // 2]
        print(f"write {m}x{n} ({nbytes / 2**20:.0f} MiB), {label}: median {med * 1e3:.1f} us "
              f"(min {times[0] * 1e3:.1f}) over {reps} -> {nbytes / (med * 1e-3) / 1e12:.2f} TB/s", flush=True)
    if float(buf[-1]) != 2.0:
        raise RuntimeError("fill_ did not write the buffer")


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


def _variant_info(name):
    """sgemm_variant_info of the named kernel variant in the built library, or None."""
    from . import _binding as sg
    for i in range(sg.sgemm_num_variants()):
        if sg.sgemm_variant_name(i) == name:
            return sg.sgemm_variant_info(i)
    return None


def cmd_report(args) -> None:
    d, W = args.dir, args.workload
    tag = getattr(args, "run_tag", None) or W  # raw-output directory suffix (workload[__variant])
    forced = f" --variant {args.variant}" if tag != W else ""
    w, flops, alg_bytes = _workload_figures(W)
    rows = _stats_rows(os.path.join(d, f"trace_{tag}", "run_kernel_stats.csv"))
    kern = [r for r in rows if "sgemm" in r["Name"]]
    if len(kern) != 1:
        raise SystemExit(f"expected one sgemm kernel in the trace of {W}, found {len(kern)}")
    k = kern[0]
    name = k["Name"]
    avg_ns = float(k["AverageNs"])
    # the bench's launches: the first call, the warmup, the timed region (`steps` back-to-back
    # launches) and a pass of min(steps, 50) individually timed launches
    with open(os.path.join(d, f"trace_{tag}", "run_kernel_trace.csv")) as f:
        disp = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in csv.DictReader(f)
                if r["Kernel_Name"] == name]
    spread = min(args.steps, 50)
    timed = disp[-(args.steps + spread):-spread]
    timed_ns = _mean(timed)
    # variant name from the kernel signature is not unique; take it from the bench log
    variant = args.variant
    sq = {c: _mean(v) for c, v in _read_counters(os.path.join(d, f"sq_{tag}", "run_counter_collection.csv"), "sgemm").items()}
    fetch = _mean_counter(os.path.join(d, f"fetch_{tag}", "run_counter_collection.csv"), "sgemm", "FETCH_SIZE")
    write = _mean_counter(os.path.join(d, f"write_{tag}", "run_counter_collection.csv"), "sgemm", "WRITE_SIZE")
    rd = {c: _mean(v) for c, v in _read_counters(os.path.join(d, f"rdreq_{tag}", "run_counter_collection.csv"), "sgemm").items()}
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
    last_c, last_ns = _dispatches(os.path.join(d, f"sq_{tag}", "run_counter_collection.csv"), "sgemm")[-1]
    last_gui = last_c.get("GRBM_GUI_ACTIVE", float("nan")) / N_XCD
    sclk_last = last_gui / last_ns if last_ns > 0 else float("nan")  # cycles per ns = GHz
    mfma_last = last_c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (N_SIMD * last_gui)
    lds_conf = sq.get("SQ_LDS_BANK_CONFLICT", float("nan")) / (N_CU * gui)
    info = _variant_info(variant)
    mb = info.get("mfma_block", 32) if info else 32
    # MFMAs of the exact problem (no tile padding): 32x32x2 = 2048 and 16x16x4 = 1024 multiply-adds each
    expect_mfma = w.M * w.N * w.K / (2048.0 if mb == 32 else 1024.0) if mb else 0.0
    mfma_desc = {32: "v_mfma_f32_32x32x2_f32", 16: "v_mfma_f32_16x16x4_f32"}.get(mb, "(a vector-FMA kernel: none)")
    tflops = flops / (avg_ns * 1e-9) / 1e12
    tflops_timed = flops / (timed_ns * 1e-9) / 1e12
    tile = (info["BM"], info["BN"]) if info else None
    panel = panel_read_bytes(w.M, w.N, w.K, *tile) if tile else float("nan")
    bench = "python -u bench.py --workload %s%s" % (W, forced)
    trace_opt = f"--trace-args='{args.trace_args}' " if args.trace_args else ""
    sq_warm = args.sq_warmup
    cmds = [
        f"python -m fp32_gemm_05_amd.profiling collect --dir <dir> --workload {W}{forced} "
        f"{'--warmup ' + args.trace_args.split()[1] + ' ' if args.trace_args.startswith('--warmup') else ''}"
        f"(runs all of the following)",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace_{tag} -o run -- python -u bench.py "
        f"--workload {W} {args.trace_args + ' ' if args.trace_args else ''}--no-cpu-baseline --no-sclk",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch_{tag} -o run -- {bench} --steps 3 --warmup 1 --no-cpu-baseline --no-sclk",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write_{tag} -o run -- {bench} --steps 3 --warmup 1 --no-cpu-baseline --no-sclk",
        f"rocprofv3 --pmc TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum --output-format csv -d <dir>/rdreq_{tag} -o run -- {bench} --steps 3 --warmup 1 --no-cpu-baseline --no-sclk",
        f"rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVES SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE --output-format csv -d <dir>/sq_{tag} -o run -- {bench} --steps 3 --warmup {sq_warm} --no-cpu-baseline --no-sclk",
        "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE, then the three TCC_EA0_RDREQ_*_sum) --output-format csv -d <dir>/copy_fetch (copy_write, copy_rdreq) -o run -- python -u -m fp32_gemm_05_amd.profiling copy --mib 1024 --reps 3",
        f"python -m fp32_gemm_05_amd.profiling report --dir <dir> --workload {W} --variant {variant} "
        f"{'--run-tag ' + tag + ' ' if tag != W else ''}{trace_opt}--out-dir profiles",
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
        f"* MFMA instructions: {sq.get('SQ_INSTS_MFMA', float('nan')):.6g} (the problem needs "
        f"{expect_mfma:.6g} {mfma_desc}; the rest is tile padding at ragged edges)",
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


def cmd_phases(args) -> None:
    """Where one launch's time goes, per wave, from the phase-stamp build of libsgemm: the cycles of
    the prologue (kernel start until the first slab has landed), the K loop and the epilogue, each
    wave's start and end on the real-time clock, and the engine clock over the wave.  Next to them:
    the same variant's time per launch back to back (libsgemm.so, after a clock pre-roll), the
    launch floor of its grid, and the K loop's ideal -- the wave's MFMAs at the cycles one MFMA
    takes in a dependent chain (mfma_chain).  Runs on the GPU in this process."""
    import ctypes

    import numpy as np
    import torch
    from . import _binding as sg
    from . import build as hb
    from .workloads import WORKLOADS, make_inputs

    for path in (hb.LIB, hb.STAMPS_LIB):
        if not os.path.exists(path):
            raise SystemExit(f"{path} is not built (__graft_entry__.build())")
    prod = sg.load_library()
    st = sg.load_library(hb.STAMPS_LIB)
    st.sgemm_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_uint]
    st.sgemm_phase_stamps.restype = ctypes.c_int
    refs = launch_refs_lib()
    W = args.workload
    w = WORKLOADS[W]
    A, B, C0 = make_inputs(w)
    dev = torch.device("cuda:0")
    dA, dB, dC = (torch.from_numpy(x).to(dev) for x in (A, B, C0))
    stream = torch.cuda.current_stream()
    if args.variant:
        vid = next((i for i in range(sg.sgemm_num_variants()) if sg.sgemm_variant_name(i) == args.variant), -1)
        if vid < 0:
            raise SystemExit(f"no variant named {args.variant}")
    else:
        vid = prod.sgemm_select_variant(w.M, w.N, w.K, dA.data_ptr(), w.K, dB.data_ptr(), w.N, dC.data_ptr(), w.N)
    name = sg.sgemm_variant_name(vid)
    if st.sgemm_variant_name(vid).decode() != name:
        raise SystemExit("libsgemm.so and libsgemm_stamps.so were built from different sources")
    info = sg.sgemm_variant_info(vid)
    print(f"[phases] {W}: variant {name}", flush=True)

    def call(lib):
        rc = lib.sgemm_ex(w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.K, dB.data_ptr(), w.N, w.beta, dC.data_ptr(),
                          w.N, stream.cuda_stream, vid)
        if rc != 0:
            raise RuntimeError(f"sgemm_ex returned {rc}")

    def preroll(lib, seconds):
        import time
        t0 = time.time()
        while time.time() - t0 < seconds:
            for _ in range(50):
                call(lib)
            torch.cuda.synchronize()

    # cold: a 512 MiB read (more than the Infinity Cache and every L2) before a launch evicts its
    # operands, as the bench's --cold does
    flush = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device=dev) if args.cold else None
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def evict():
        if flush is not None:
            torch.sum(flush, dim=0, out=flush_out)

    # back to back, as the bench times it (cold: each launch between its own events, after a flush)
    preroll(prod, args.preroll)
    if args.cold:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            evict()
            a.record(stream)
            call(prod)
            b.record(stream)
        torch.cuda.synchronize()
        b2b_us = sum(a.elapsed_time(b) for a, b in evs) / args.steps * 1e3
    else:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            call(prod)
        e1.record(stream)
        torch.cuda.synchronize()
        b2b_us = e0.elapsed_time(e1) / args.steps * 1e3
    tiles = -(-w.M // info["BM"]) * -(-w.N // info["BN"])
    floor_us = launch_floor_ms(tiles, info["threads"], info["lds_bytes"], args.steps, stream) * 1e3
    print(f"[phases] back to back {b2b_us:.2f} us per launch; launch floor {floor_us:.2f} us", flush=True)

    # the stamped launches
    wpg = info["threads"] // 64
    waves = tiles * wpg
    buf = torch.zeros(waves * 10, dtype=torch.int64, device=dev)
    preroll(st, args.preroll / 2)
    if st.sgemm_phase_stamps(buf.data_ptr(), waves) != 0:
        raise RuntimeError("sgemm_phase_stamps failed")
    for _ in range(3):
        evict()
        call(st)
    torch.cuda.synchronize()
    st.sgemm_phase_stamps(None, 0)
    x = buf.cpu().numpy().reshape(waves, 5, 2).astype(np.int64)
    if (x[:, :4, 0] == 0).any():
        raise SystemExit(f"{name}: its kernel family records no phase stamps (the direct-to-LDS, plain and "
                         f"deep MFMA kernels do)")
    c, r, hw = x[:, :4, 0], x[:, :4, 1], x[:, 4, 0]
    pro, loop, epi = c[:, 1] - c[:, 0], c[:, 2] - c[:, 1], c[:, 3] - c[:, 2]
    rate_mhz = refs.wall_clock_khz() / 1000.0
    mhz = (c[:, 3] - c[:, 0]) / np.maximum(r[:, 3] - r[:, 0], 1) * rate_mhz
    start_us = (r[:, 0] - r[:, 0].min()) / rate_mhz
    end_us = (r[:, 3] - r[:, 0].min()) / rate_mhz
    span_us = float(end_us.max())
    mb = info.get("mfma_block") or 32
    nslab = -(-w.K // info["BK"])
    fm, fn = info["WM_or_TM"] // mb, info["WN_or_TN"] // mb
    mfmas = nslab * fm * fn * info["BK"] * mb // 64  # per wave: BK*MB/64 MFMAs per block and slab
    issue = mfma_cycles(mb, stream, ilp=4)  # the issue rate (independent chains)
    dep = mfma_cycles(mb, stream, ilp=1)    # one dependent chain
    cyc = issue[0]
    ideal = mfmas * cyc
    clk = float(np.median(mhz))
    # waves per SIMD: HW_ID holds SIMD_ID [5:4], CU_ID [11:8], SH_ID [12], SE_ID [15:13]; workgroup g
    # runs on XCD g % 8 (round-robin dispatch over the XCDs)
    wg = np.arange(waves) // wpg
    key = ((wg % 8) << 16) | (((hw >> 13) & 7) << 8) | (((hw >> 12) & 1) << 7) | (((hw >> 8) & 15) << 2) | ((hw >> 4) & 3)
    simd_busy, simd_waves = [], []
    for k in np.unique(key):
        sel = key == k
        window_us = (r[sel, 3].max() - r[sel, 0].min()) / rate_mhz
        simd_waves.append(int(sel.sum()))
        simd_busy.append(sel.sum() * ideal / max(window_us * clk, 1e-9))
    nsimd = len(simd_busy)
    total_ideal_us = waves * ideal / clk / 1024.0  # all the MFMAs spread over the chip's 1024 SIMDs

    def q(a, us=False):
        a = np.asarray(a, dtype=np.float64)
        f = (lambda v: f"{v:.0f} ({v / clk:.2f} us)") if us else (lambda v: f"{v:.2f}")
        return f"{f(np.median(a))} | {f(a.min())} | {f(a.max())}"

    def pct(a):
        a = 100 * np.asarray(a, dtype=np.float64)
        return f"{np.median(a):.1f} % | {a.min():.1f} % | {a.max():.1f} %"

    shape = {32: "v_mfma_f32_32x32x2_f32", 16: "v_mfma_f32_16x16x4_f32"}[mb]
    lines = [
        f"# Phase stamps: `{name}` on {W}{' (cold caches)' if args.cold else ''}", "",
        f"Workload: {w.describe()}.  Grid: {tiles} workgroups of {info['threads']} threads ({waves} waves), "
        f"{mfmas} {shape} per wave.", "",
        "| Per launch | us |", "|---|---|",
        (f"| cold: mean of {args.steps} launches each timed alone after a 512 MiB flush (libsgemm.so) | {b2b_us:.2f} |"
         if args.cold else
         f"| back to back (libsgemm.so, {args.steps} launches after a {args.preroll:.1f} s pre-roll) | {b2b_us:.2f} |"),
        f"| launch floor of the grid (empty kernel, same grid, timed the same way) | {floor_us:.2f} |",
        f"| wave span of one stamped launch (first wave start to last wave end) | {span_us:.2f} |",
        f"| {'launch time' if args.cold else 'back to back'} - span: launch gap and the grid's ramp-up | "
        f"{b2b_us - span_us:.2f} |",
        f"| every MFMA of the launch at the issue rate, spread evenly over 1024 SIMDs | {total_ideal_us:.2f} |", "",
        f"MFMA issue cost (mfma_chain at one wave per SIMD): {cyc:.1f} cycles with four interleaved "
        f"chains (min {issue[1]:.1f}, max {issue[2]:.1f}), {dep[0]:.1f} cycles in one dependent chain.", "",
        "| Per wave (stamped launch) | median | min | max |", "|---|---|---|---|",
        f"| engine clock (MHz) | {q(mhz)} |",
        f"| prologue cycles (start to first slab landed) | {q(pro, True)} |",
        f"| K loop cycles | {q(loop, True)} |",
        f"| epilogue cycles | {q(epi, True)} |",
        f"| start after the first wave (us) | {q(start_us)} |",
        f"| end after the first wave's start (us) | {q(end_us)} |",
        f"| K loop at the issue rate: ideal {ideal:.0f} cycles / loop cycles (one wave per SIMD only) | "
        f"{pct(ideal / loop)} |", "",
        f"| Per SIMD ({nsimd} SIMDs ran waves) | median | min | max |", "|---|---|---|---|",
        f"| waves | {q(simd_waves)} |",
        f"| matrix-pipe busy: its waves' MFMAs at the issue rate / (last wave end - first wave start) | "
        f"{pct(simd_busy)} |", "",
        "## Command", "", "```",
        f"python -m fp32_gemm_05_amd.profiling phases --workload {W}"
        f"{' --variant ' + args.variant if args.variant else ''}{' --cold' if args.cold else ''} --steps {args.steps} "
        f"--preroll {args.preroll}",
        "```", "",
    ]
    if args.note:
        lines += [args.note, ""]
    os.makedirs(args.out_dir, exist_ok=True)
    out = os.path.join(args.out_dir, f"phases_{name}__{W}{'_cold' if args.cold else ''}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines), flush=True)


# Lane-pair patterns of the LDS pass probe: lanes i and j read two different words of the same
# banks (float offsets 0 and 64, 256 bytes apart) and every other lane one broadcast word in other
# banks (float 32), so a dispatch has bank-conflict cycles exactly when i and j share a pass.
LDS_PROBE_WIDTHS = (16, 8, 4)
LDS_PROBE_LANES = (0, 8, 16, 32)


def lds_probe_plan():
    plan = []
    for width in LDS_PROBE_WIDTHS:
        for i in LDS_PROBE_LANES:
            for j in range(64):
                if j != i:
                    idx = [32] * 64
                    idx[i], idx[j] = 0, 64
                    plan.append((width, i, j, idx))
    return plan


def cmd_lds_probe(args) -> None:
    """Launch every lane-pair pattern once (one wave, `reps` reads each); run it under
    `rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS`.  The dispatches follow lds_probe_plan()."""
    import torch
    lib = launch_refs_lib()
    plan = lds_probe_plan()
    tabs = torch.tensor([p[3] for p in plan], dtype=torch.int32, device="cuda")
    out = torch.zeros(64, device="cuda")
    stream = torch.cuda.current_stream()
    for n, (width, i, j, idx) in enumerate(plan):
        rc = lib.lds_probe(tabs[n].data_ptr(), width, args.reps, out.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"lds_probe returned {rc}")
    torch.cuda.synchronize()
    print(f"lds-probe: {len(plan)} dispatches of {args.reps} reads", flush=True)


def cmd_lds_passes(args) -> None:
    """The LDS pass grouping from a counter run of `lds-probe`: for each access width and probe
    lane i, the lanes j whose pattern has bank-conflict cycles."""
    per = defaultdict(dict)
    with open(args.csv) as f:
        for row in csv.DictReader(f):
            if "lds_probe" in row["Kernel_Name"]:
                per[int(row["Dispatch_Id"])][row["Counter_Name"]] = float(row["Counter_Value"])
    plan = lds_probe_plan()
    ids = sorted(per)
    if len(ids) != len(plan):
        raise SystemExit(f"expected {len(plan)} probe dispatches, found {len(ids)}")
    shared = defaultdict(list)
    cycles = defaultdict(set)
    for d, (width, i, j, _) in zip(ids, plan):
        c = per[d].get("SQ_LDS_BANK_CONFLICT", 0.0)
        if c > 0:
            shared[(width, i)].append(j)
        cycles[width].add(c)

    def ranges(xs):
        xs, out = sorted(xs), []
        for x in xs:
            if out and x == out[-1][1] + 1:
                out[-1][1] = x
            else:
                out.append([x, x])
        return ", ".join(f"{a}-{b}" if a != b else f"{a}" for a, b in out) or "none"

    lines = ["# LDS passes: which lanes of one access share a pass (MI355X)", "",
             "Lanes i and j read two different words of the same four banks, every other lane one "
             "broadcast word in other banks; the dispatch counts SQ_LDS_BANK_CONFLICT cycles exactly "
             f"when i and j go through the LDS in the same pass ({args.reps} reads per dispatch).", "",
             "| Access | Lane i | Lanes j sharing its pass |", "|---|---|---|"]
    for width in LDS_PROBE_WIDTHS:
        for i in LDS_PROBE_LANES:
            lines.append(f"| {width * 8}-bit | {i} | {ranges(shared[(width, i)])} |")
    lines += ["", "Conflict-cycle values seen per dispatch: " +
              "; ".join(f"{w * 8}-bit {sorted(v)}" for w, v in cycles.items()), "",
              "## Commands", "", "```",
              f"rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS --output-format csv -d <dir> -o run -- "
              f"python -u -m fp32_gemm_05_amd.profiling lds-probe --reps {args.reps}",
              "python -m fp32_gemm_05_amd.profiling lds-passes <dir>/run_counter_collection.csv --out profiles/lds_passes.md",
              "```", ""]
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines), flush=True)


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
    if args.variant:
        bench += ["--variant", args.variant]  # a forced variant instead of the dispatched one
    tag_w = f"{W}__{args.variant}" if args.variant else W  # raw-output directories of this run
    _run(rp + ["--kernel-trace", "--stats", "-d", os.path.join(d, f"trace_{tag_w}"), "-o", "run", "--", *bench,
               "--warmup", str(args.warmup), "--no-cpu-baseline", "--no-sclk"], os.path.join(d, f"trace_{tag_w}.log"), 300)
    variant = None
    with open(os.path.join(d, f"trace_{tag_w}.log")) as f:
        for line in f:
            if line.startswith("variant: "):
                variant = line.split()[1]
    if variant is None:
        raise SystemExit("the bench did not report its variant")
    for tag, counters in PMC_PASSES:
        _run(rp + ["--pmc", *counters, "-d", os.path.join(d, f"{tag}_{tag_w}"), "-o", "run", "--", *bench,
                   "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-sclk"],
             os.path.join(d, f"{tag}_{tag_w}.log"), 120)
    extra = f"--warmup {args.warmup}" + (f" --variant {args.variant}" if args.variant else "")
    report = argparse.Namespace(dir=d, workload=W, variant=variant, steps=200, sq_warmup=1, trace_args=extra,
                                out_dir=args.out_dir, note="", run_tag=tag_w)
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
    p = sub.add_parser("write")
    p.add_argument("--m", type=int, default=8192)
    p.add_argument("--n", type=int, default=8192)
    p.add_argument("--reps", type=int, default=50)
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
    p.add_argument("--variant", default=None, help="profile this variant (by name) instead of the dispatched one")
    p.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    p = sub.add_parser("phases", help="per-wave phase breakdown from the phase-stamp build (runs on the GPU)")
    p.add_argument("--workload", required=True)
    p.add_argument("--variant", default=None, help="a variant by name (default: the dispatched one)")
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--preroll", type=float, default=1.0, help="seconds of launches before timing")
    p.add_argument("--cold", action="store_true", help="evict the caches before every timed and stamped launch")
    p.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    p.add_argument("--note", default="")
    p = sub.add_parser("lds-probe", help="launch the LDS lane-pair patterns (run under rocprofv3 --pmc)")
    p.add_argument("--reps", type=int, default=64)
    p = sub.add_parser("lds-passes", help="the LDS pass grouping from a counter run of lds-probe")
    p.add_argument("csv")
    p.add_argument("--reps", type=int, default=64)
    p.add_argument("--out", required=True)
    p = sub.add_parser("report")
    p.add_argument("--dir", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--variant", required=True)
    p.add_argument("--steps", type=int, default=200, help="timed steps of the traced bench run")
    p.add_argument("--sq-warmup", type=int, default=1, help="bench warmup of the SQ counter run")
    p.add_argument("--trace-args", default="", help="extra bench.py arguments of the traced run (e.g. a longer "
                   "warmup, so that short kernels are traced at the ramped-up engine clock)")
    p.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    p.add_argument("--run-tag", default=None, help="directory suffix of a collect run with a forced variant "
                   "(<workload>__<variant>)")
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
    elif args.cmd == "write":
        if args.m % 64 or args.n % 64 or args.m <= 0 or args.n <= 0:
            raise SystemExit("write: --m and --n must be positive multiples of 64")
        run_write(args.m, args.n, args.reps)
    elif args.cmd == "stats":
        cmd_stats(args)
    elif args.cmd == "traffic":
        cmd_traffic(args)
    elif args.cmd == "counters":
        cmd_counters(args)
    elif args.cmd == "series":
        cmd_series(args)
    elif args.cmd == "phases":
        cmd_phases(args)
    elif args.cmd == "lds-probe":
        cmd_lds_probe(args)
    elif args.cmd == "lds-passes":
        cmd_lds_passes(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
