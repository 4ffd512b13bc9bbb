"""rocprofv3 helpers for libsgemm's measurements.

    python -m fp32_gemm_05_amd.profiling copy --mib 1024 --reps 3
        a plain device-to-device copy of known size; run under `rocprofv3 --pmc FETCH_SIZE`
        (then WRITE_SIZE) it calibrates how many bytes one KiB of each counter stands for.
    python -m fp32_gemm_05_amd.profiling stats <kernel_stats.csv> --command "..." --out X.md
        short text summary of a `rocprofv3 --kernel-trace --stats` run.
    python -m fp32_gemm_05_amd.profiling traffic --kernel SUBSTR --fetch F.csv --write W.csv
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --workload NAME --variant NAME --out X.json
        HBM bytes per launch of one kernel from two --pmc runs, each scaled by the copy calibration.
    python -m fp32_gemm_05_amd.profiling counters <counter_collection.csv> --kernel SUBSTR --out X.md
        per-dispatch means of any collected counters for one kernel.

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

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp32_gemm_05_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
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
        "kernel_source_hash": kernel_source_hash(), "commands": args.commands,
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


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    p = sub.add_parser("copy")
    p.add_argument("--mib", type=int, default=1024)
    p.add_argument("--reps", type=int, default=3)
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
    args = ap.parse_args(argv)
    if args.cmd == "copy":
        run_copy(args.mib, args.reps)
    elif args.cmd == "stats":
        cmd_stats(args)
    elif args.cmd == "traffic":
        cmd_traffic(args)
    elif args.cmd == "counters":
        cmd_counters(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
