#!/usr/bin/env python3
"""Tile-parameter autotuner of libsgemm: sweep every kernel variant over each shape
class, gate each candidate on the float64 oracle, time it, and write the dispatch
table (fp32_gemm_05_amd/csrc/tuned_table.inc) from the winners.

    python tests/autotune.py [--out results.json] [--write-table] [--classes large,small,skinny]

The tile parameters (BM, BN, BK, wave tile WM x WN or microtile TM x TN, and an
occupancy target) are compile-time template arguments, as in the pages' kernels
("Optimizing Matrix Multiplication in CUDA", sections on 2D thread tiling and
warp tiling, where they are template parameters tuned by hand); each compiled
instance is one variant of the library, and the sweep runs over all of them.

Selection: within a (shape class, vector-load class) pair, a variant must pass
the oracle check on every representative workload; the winner minimises the
geometric mean of (time / best time) over those workloads, and replaces the
table's current entry only when it beats it by more than --keep-margin (1 %).  This file imports
the oracle, so it lives with the tests; the library never runs it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TABLE = os.path.join(ROOT, "fp32_gemm_05_amd", "csrc", "tuned_table.inc")

# (label, shape class, workload name or None, M, N, K, dist, alpha, beta, vector-load eligible)
CASES = [
    ("square4096", "large", "square4096", None, None, None, None, None, None, True),
    ("square8192", "huge", "square8192", None, None, None, None, None, None, True),
    ("square6144", "huge", "square4096", 6144, 6144, 6144, None, None, None, True),
    ("ragged8191x8190x2047", "huge", "ragged3001x5003x777", 8191, 8190, 2047, None, None, None, False),
    ("square4096_odd_ld", "large", "square4096", 4096, 4095, 4095, "uniform", 1.0, 0.0, False),
    ("ragged3001x5003x2047", "large", "ragged3001x5003x777", 3001, 5003, 2047, None, None, None, False),
    ("ragged3001x5003x777", "shallow", "ragged3001x5003x777", None, None, None, None, None, None, False),
    ("ragged2500x3500x1000", "shallow", "ragged3001x5003x777", 2500, 3500, 1000, None, None, None, False),
    ("shallow4096x4096x512", "shallow", "square4096", 4096, 4096, 512, None, None, None, True),
    ("shallow3072x3072x768", "shallow", "square1024_beta", 3072, 3072, 768, None, None, None, True),
    ("shallow2560x3584x320", "shallow_shortk", "square256", 2560, 3584, 320, None, None, None, True),
    ("shallow2048x2048x896", "shallow", "square1024_beta", 2048, 2048, 896, None, None, None, True),
    ("shallow2880x3776x272", "shallow_shortk", "square256", 2880, 3776, 272, None, None, None, True),
    ("shallow5632x2432x224", "shallow_shortk", "square256", 5632, 2432, 224, None, None, None, True),
    ("shallow2048x2560x640", "shallow", "square1024_beta", 2048, 2560, 640, None, None, None, True),
    ("shallow5001x2301x251", "shallow_shortk", "ragged3001x5003x777", 5001, 2301, 251, None, None, None, False),
    ("shallow3001x4001x301", "shallow_shortk", "ragged3001x5003x777", 3001, 4001, 301, None, None, None, False),
    ("shallow2501x2999x449", "shallow_shortk", "ragged3001x5003x777", 2501, 2999, 449, None, None, None, False),
    ("shallow4401x2901x263", "shallow_shortk", "ragged3001x5003x777", 4401, 2901, 263, None, None, None, False),
    ("medium2585x6716x2000", "medium", "square4096", 2585, 6716, 2000, None, None, None, True),
    ("medium3000x3000x3000", "medium", "square4096", 3000, 3000, 3000, None, None, None, True),
    ("shard1024x4096x4096", "medium", "square4096", 1024, 4096, 4096, None, None, None, True),
    ("shard2048x4096x4096", "long_k", "square4096", 2048, 4096, 4096, None, None, None, True),
    ("shard1024x8192x8192", "long_k", "square8192", 1024, 8192, 8192, None, None, None, True),
    ("longk2047x4095x4097", "long_k", "ragged3001x5003x777", 2047, 4095, 4097, None, None, None, False),
    ("longk1500x6000x6000", "long_k", "ragged3001x5003x777", 1500, 6000, 6001, None, None, None, False),
    ("medium2062x3171x3921", "medium", "ragged3001x5003x777", 2062, 3171, 3921, None, None, None, False),
    ("medium5000x2001x2501", "medium", "ragged3001x5003x777", 5000, 2001, 2501, None, None, None, False),
    ("medium2301x2703x2101", "medium", "ragged3001x5003x777", 2301, 2703, 2101, None, None, None, False),
    ("medium4201x5999x1603", "medium", "ragged3001x5003x777", 4201, 5999, 1603, None, None, None, False),
    ("medium901x4801x1201", "medium", "ragged3001x5003x777", 901, 4801, 1201, None, None, None, False),
    ("medium6001x401x2301", "medium", "ragged3001x5003x777", 6001, 401, 2301, None, None, None, False),
    ("tinyk5555x1124x68", "tiny_k", "square4096", 5555, 1124, 68, None, None, None, True),
    ("tinyk1953x2052x72", "tiny_k", "square4096", 1953, 2052, 72, None, None, None, True),
    ("tinyk8192x8192x32", "tiny_k", "square4096", 8192, 8192, 32, None, None, None, True),
    ("tinyk3001x4001x101", "tiny_k", "ragged3001x5003x777", 3001, 4001, 101, None, None, None, False),
    ("tinyk2048x2047x33", "tiny_k", "ragged3001x5003x777", 2048, 2047, 33, None, None, None, False),
    ("longk1024x1024x4096", "small_longk", "square1024_beta", 1024, 1024, 4096, None, None, None, True),
    ("shard512x4096x4096", "medium", "square4096", 512, 4096, 4096, None, None, None, True),
    ("longk1089x728x5752", "small_longk", "square4096", 1089, 728, 5752, None, None, None, True),
    ("longk1751x907x5323", "medium", "ragged3001x5003x777", 1751, 907, 5323, None, None, None, False),
    ("longk777x1501x3001", "small_full", "ragged3001x5003x777", 777, 1501, 3001, None, None, None, False),
    ("longk1199x587x3229", "small_longk", "ragged3001x5003x777", 1199, 587, 3229, None, None, None, False),
    ("longk1003x777x2503", "small_longk", "ragged3001x5003x777", 1003, 777, 2503, None, None, None, False),
    ("square256", "tiny_shortk", "square256", None, None, None, None, None, None, True),
    ("shortk822x124x88", "tiny_shortk", "square256", 822, 124, 88, None, None, None, True),
    ("shortk2664x180x284", "tiny_shortk", "square256", 2664, 180, 284, None, None, None, True),
    ("shortk700x100x333", "tiny_shortk", "ragged3001x5003x777", 700, 100, 333, None, None, None, False),
    ("shortk2048x1536x384", "small_shortk", "square1024_beta", 2048, 1536, 384, None, None, None, True),
    ("shortk1536x1024x256", "small_shortk", "square256", 1536, 1024, 256, None, None, None, True),
    ("shortk3600x284x148", "small_shortk", "square256", 3600, 284, 148, None, None, None, True),
    ("shortk7195x426x167", "small_shortk", "ragged3001x5003x777", 7195, 426, 167, None, None, None, False),
    ("shortk516x1306x236", "small_shortk", "ragged3001x5003x777", 516, 1306, 236, None, None, None, False),
    ("tiny1554x64x5093", "tiny", "ragged3001x5003x777", 1554, 64, 5093, None, None, None, False),
    ("square1024_beta", "small", "square1024_beta", None, None, None, None, None, None, True),
    ("ragged1001x1003x777", "small", "ragged3001x5003x777", 1001, 1003, 777, None, None, None, False),
    ("full1111x1113x1001", "small_full", "ragged3001x5003x777", 1111, 1113, 1001, None, None, None, False),
    ("full900x1500x833", "small_full", "ragged3001x5003x777", 900, 1500, 833, None, None, None, False),
    ("full1200x1300x700", "small_multi", "square1024_beta", 1200, 1300, 700, None, None, None, True),
    ("full1400x1000x1400", "small_full", "square256", 1400, 1000, 1400, None, None, None, True),
    ("full1100x1100x1000", "small_full", "square1024_beta", 1100, 1100, 1000, None, None, None, True),
    ("multi763x2487x641", "small_multi", "ragged3001x5003x777", 763, 2487, 641, None, None, None, False),
    ("multi1531x1527x1101", "small_multi", "ragged3001x5003x777", 1531, 1527, 1101, None, None, None, False),
    ("multi1915x1783x1901", "small_multi", "ragged3001x5003x777", 1915, 1783, 1901, None, None, None, False),
    ("multi635x5111x701", "small_multi", "ragged3001x5003x777", 635, 5111, 701, None, None, None, False),
    ("multi764x2484x640", "small_multi", "square1024_beta", 764, 2484, 640, None, None, None, True),
    ("multi1532x1524x1100", "small_multi", "square1024_beta", 1532, 1524, 1100, None, None, None, True),
    ("multi1916x1780x1900", "small_multi", "square1024_beta", 1916, 1780, 1900, None, None, None, True),
    ("small892x1083x609", "small", "ragged3001x5003x777", 892, 1083, 609, None, None, None, False),
    ("small1000x800x1000", "small", "square1024_beta", 1000, 800, 1000, None, None, None, True),
    ("small512x512x512", "tiny", "square256", 512, 512, 512, None, None, None, True),
    ("tiny333x555x777", "tiny", "ragged3001x5003x777", 333, 555, 777, None, None, None, False),
    ("tiny600x200x1000", "tiny", "ragged3001x5003x777", 600, 200, 1000, None, None, None, False),
    ("tiny640x384x1536", "tiny", "square1024_beta", 640, 384, 1536, None, None, None, True),
    ("small768x1280x1024", "small", "square1024_beta", 768, 1280, 1024, None, None, None, True),
    ("small2048x512x1536", "small", "square256", 2048, 512, 1536, None, None, None, True),
    ("ragged700x900x1301", "small", "ragged3001x5003x777", 700, 900, 1301, None, None, None, False),
    ("skinny65536x64x1024", "skinny", "skinny65536x64x1024", None, None, None, None, None, None, True),
    ("skinny65536x61x1021", "skinny", "skinny65536x64x1024", 65536, 61, 1021, None, None, None, False),
    ("skinny100003x47x777", "skinny", "ragged3001x5003x777", 100003, 47, 777, None, None, None, False),
    ("narrow262144x32x512", "narrow", "skinny65536x64x1024", 262144, 32, 512, None, None, None, True),
    ("narrow131072x16x1024", "narrow", "skinny65536x64x1024", 131072, 16, 1024, None, None, None, True),
    ("narrow65536x24x2048", "narrow", "skinny65536x64x1024", 65536, 24, 2048, None, None, None, True),
    ("narrow100003x29x777", "narrow", "ragged3001x5003x777", 100003, 29, 777, None, None, None, False),
    ("narrow200003x7x333", "narrow", "ragged3001x5003x777", 200003, 7, 333, None, None, None, False),
]
# Classes timed in three cache states, each state scored as a case of its own: "warm"
# (back-to-back launches), "cold" (each timed launch follows a read of a 512 MiB buffer, which
# evicts the operands from the L2s and the 256 MB Infinity Cache and leaves clean lines) and
# "dirty" (the 512 MiB buffer is overwritten instead, so dirty lines are written back while the
# launch runs).  The skinny class streams A from HBM: warm launches alone would time it partly
# out of the Infinity Cache, and cold ones alone would miss what evicting dirty lines costs.
COLD_CLASSES = {"skinny", "narrow"}
STATES = ("warm", "cold", "dirty")
CLASS_IDS = {"skinny": "kSkinny", "small": "kSmall", "large": "kLarge", "huge": "kHuge", "shallow": "kShallow",
             "medium": "kMedium", "small_longk": "kSmallLongK", "tiny_k": "kTinyK", "tiny": "kTiny",
             "small_shortk": "kSmallShortK", "long_k": "kLongK", "small_full": "kSmallFull",
             "narrow": "kNarrow", "tiny_shortk": "kTinyShortK",
             "shallow_shortk": "kShallowShortK", "small_multi": "kSmallMulti"}


def log(msg):
    print(msg, flush=True)


def read_table():
    """Existing (class, vec) -> (variant, score) entries of the dispatch table."""
    import re
    out = {}
    if os.path.exists(TABLE):
        ids = {v: k for k, v in CLASS_IDS.items()}
        for m in re.finditer(r'\{(k\w+), (\d), "([\w]+)"\},\s*//[^\n]*?best ([\d.]+)[^\n]*$', open(TABLE).read(), re.M):
            out[(ids[m.group(1)], int(m.group(2)))] = (m.group(3), float(m.group(4)))
    return out


def shape_class(M, N, K):
    """The shape class the library gives an M x N x K product (shape_class in csrc/sgemm.hip,
    restated; tests/test_autotune_cpu.py checks the two agree)."""
    def cd(a, b):
        return -(-a // b)
    t64 = cd(M, 64) * cd(N, 64)
    if N <= 32 and t64 >= 128:
        return "narrow"
    if N <= 64 and t64 >= 128:
        return "skinny"
    t = cd(M, 128) * cd(N, 128)
    if t < 256:
        if cd(M, 32) * cd(N, 64) <= 256:
            return "tiny_shortk" if K < 512 else "tiny"
        if K < 512:
            return "small_shortk"
        if K >= 2048 and t64 >= 384:
            return "medium"
        if t64 <= 256:
            return "small_longk" if K >= 2048 else "small"
        return "small_full" if t64 <= 384 else "small_multi"
    if K < 128:
        return "tiny_k"
    if t >= 2048:
        return "huge"
    if K <= 1024:
        return "shallow_shortk" if K < 512 else "shallow"
    if t * 100 >= cd(t, 1024) * 1024 * 85:
        return "large"
    return "long_k" if t >= 512 and K >= 4096 else "medium"


def load_results(paths):
    """The records of one or more saved runs (tuning sweeps or regret runs), a later file's record
    of a (case, variant) replacing an earlier one's, each labelled with the shape class the library
    gives its shape (a regret run labels its shapes "random"; an older sweep may predate a class
    boundary); records of transposed operand forms are left out."""
    merged = {}
    for path in paths:
        with open(path) as f:
            for r in json.load(f)["results"]:
                if r.get("op", "NN") != "NN":
                    continue  # transposed forms are dispatched by their own rules, not by the table
                merged[(r["case"], r["variant"])] = dict(r, **{"class": shape_class(r["M"], r["N"], r["K"])})
    return list(merged.values())


def choose_winners(results, keep_margin):
    """Per (class, vector-load class): the variant with the smallest geometric-mean slowdown
    against the per-case best, among those that ran and passed parity on every case.  The table's
    current entry is kept unless it is slower than that winner by more than keep_margin (run-to-run
    variation of these scores is about 1 %)."""
    incumbent = read_table()
    winners = {}
    for cls in sorted({r["class"] for r in results}):
        for vclass in (0, 1):
            recs = [r for r in results if r["class"] == cls and r["vec_class"] == vclass]
            if not recs:
                continue
            cases = sorted({r["case"] for r in recs})
            best = {c: min(r["ms_median"] for r in recs if r["case"] == c and r["parity"]) for c in cases}
            score = {}
            for name in sorted({r["variant"] for r in recs}):
                rs = {r["case"]: r for r in recs if r["variant"] == name}
                if set(rs) != set(cases) or not all(r["parity"] for r in rs.values()):
                    continue
                # a vector-load class may also be served by a scalar-load variant, never the reverse
                score[name] = math.exp(sum(math.log(rs[c]["ms_median"] / best[c]) for c in cases) / len(cases))
            if not score:
                continue
            win = min(score, key=score.get)
            old = incumbent.get((cls, vclass), (None, 0.0))[0]
            if old in score and old != win and score[old] <= score[win] * (1.0 + keep_margin):
                log(f"keep {cls}/{'vec' if vclass else 'scalar'}: {old} ({score[old]:.3f}; "
                    f"{win} {score[win]:.3f} is within the margin)")
                win = old
            winners[(cls, vclass)] = (win, score[win])
            log(f"winner {cls}/{'vec' if vclass else 'scalar'}: {win} (geo-mean slowdown {score[win]:.3f})")
    return winners


def write_table(winners):
    """Write the table: the new winners replace the entries of their classes, others are kept."""
    merged = read_table()
    merged.update(winners)
    winners = merged
    lines = ["// Dispatch table: (shape class, vector-load eligibility) -> variant name.",
             "// Written by tests/autotune.py from timed, oracle-checked runs on MI355X",
             f"// ({time.strftime('%Y-%m-%d')}); each entry names the geometric-mean-fastest variant",
             "// over that class's representative workloads.",
             "const TableEntry kTunedTable[] = {"]
    for (cls, vclass), (win, sc) in sorted(winners.items()):
        states = " (warm, cold, dirty)" if cls in COLD_CLASSES else ""
        lines.append(f'    {{{CLASS_IDS[cls]}, {vclass}, "{win}"}},  // slowdown vs per-case best {sc:.3f}{states}')
    lines.append("};")
    with open(TABLE, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"wrote {TABLE}")


def parse_shapes(text):
    """"[OP:]MxNxK,...": explicit shapes for the regret mode, OP one of NN (the default), NT, TN,
    TT (128-bit loads when every stored row length -- N and K, and M for a transposed A -- is a
    multiple of 4; beta 0).  Returns (M, N, K, aligned, beta, op) tuples."""
    out = []
    for item in text.split(","):
        op, _, dims = item.rpartition(":")
        op = (op or "NN").upper()
        if op not in ("NN", "NT", "TN", "TT"):
            raise ValueError(f"bad operand form in {item!r}")
        M, N, K = (int(x) for x in dims.lower().split("x"))
        if min(M, N, K) <= 0:
            raise ValueError(f"bad shape {item!r}")
        aligned = N % 4 == 0 and K % 4 == 0 and (op[0] == "N" or M % 4 == 0)
        out.append((M, N, K, aligned, 0.0, op))
    return out


def regret_mode(args, sg, sweep) -> int:
    """Dispatch regret on random shapes (or on the shapes given with --shapes): for each, every
    variant is timed and the dispatched one compared with the fastest (time of the dispatched
    variant / best time)."""
    import numpy as np

    rng = np.random.default_rng(args.regret_seed)
    records, summary = [], []
    shapes = parse_shapes(args.shapes) if args.shapes else []
    for c in range(len(shapes) if shapes else args.regret):
        op = "NN"
        if shapes:
            M, N, K, aligned, beta, op = shapes[c]
            rng = np.random.default_rng(args.regret_seed + c)
        else:
            M = int(np.exp(rng.uniform(np.log(256), np.log(8192))))
            N = int(np.exp(rng.uniform(np.log(64), np.log(8192))))
            K = int(np.exp(rng.uniform(np.log(64), np.log(8192))))
            aligned = bool(rng.integers(0, 2))
            if aligned:
                N, K = max(4, N - N % 4), max(4, K - K % 4)
            elif N % 4 == 0 and K % 4 == 0:
                K += 1
            beta = float(rng.choice([0.0, 0.5]))
        A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        C0 = rng.uniform(-1, 1, (M, N)).astype(np.float32) if beta else np.zeros((M, N), np.float32)
        label = f"{'shape' if shapes else 'random'}{c}_{'' if op == 'NN' else op + '_'}{M}x{N}x{K}"
        # the variant sgemm_op would dispatch for these arguments (pointer alignment as torch gives it)
        lda, ldb = (M if op[0] == "T" else K), (K if op[1] == "T" else N)
        disp = sg.sgemm_variant_name(sg.sgemm_op_select_variant(op[0], op[1], M, N, K, 256, lda, 512, ldb, 768, N))
        recs = sweep(label, "random", A, B, C0, 1.0, beta, aligned, 4242 + c, op)
        good = [r for r in recs if r["parity"]]
        best = min(good, key=lambda r: r["ms_median"])
        mine = [r for r in good if r["variant"] == disp]
        regret = mine[0]["ms_median"] / best["ms_median"] if mine else float("nan")
        summary.append({"case": label, "dispatched": disp, "best": best["variant"], "regret": regret,
                        "best_tflops": best["tflops"]})
        log(f"-- {label}: dispatched {disp}, best {best['variant']} ({best['tflops']:.1f} TFLOP/s), "
            f"regret {regret:.3f}")
        records += recs
    rs = sorted(x["regret"] for x in summary if x["regret"] == x["regret"])
    if rs:
        log(f"regret over {len(rs)} shapes: median {rs[len(rs) // 2]:.3f}, p90 {rs[int(len(rs) * 0.9)]:.3f}, "
            f"max {rs[-1]:.3f}")
    os.makedirs(os.path.dirname(args.out), exist_ok=True)
    with open(args.out, "w") as f:
        json.dump({"time": time.strftime("%Y-%m-%d %H:%M:%S"), "results": records, "regret": summary}, f, indent=1)
    log(f"wrote {args.out}")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(tempfile.gettempdir(), "libsgemm_autotune.json"))
    ap.add_argument("--write-table", action="store_true")
    ap.add_argument("--classes",
                    default="large,huge,long_k,shallow,shallow_shortk,medium,tiny_k,small,small_full,small_multi,tiny,tiny_shortk,small_shortk,"
                            "small_longk,skinny,narrow")
    ap.add_argument("--min-time", type=float, default=0.15, help="seconds of timed launches per candidate")
    ap.add_argument("--points", type=int, default=2048, help="sampled outputs checked per candidate")
    ap.add_argument("--warm-time", type=float, default=0.03,
                    help="seconds of untimed launches before timing a candidate (the engine clock ramps "
                         "up under sustained load; short kernels alone would be timed at a lower clock)")
    ap.add_argument("--table-from", default=None,
                    help="write the table from saved results files, comma-separated: tuning sweeps and regret "
                         "runs, the later file wins for a (case, variant) both hold (no GPU)")
    ap.add_argument("--keep-margin", type=float, default=0.01,
                    help="keep the table's entry unless the winner's score beats it by more than this fraction")
    ap.add_argument("--regret", type=int, default=0,
                    help="instead of tuning: time every variant on this many random shapes and report how far "
                         "the dispatched variant is from the fastest")
    ap.add_argument("--regret-seed", type=int, default=2024)
    ap.add_argument("--shapes", default=None,
                    help="regret mode on these shapes instead of random ones: MxNxK,MxNxK,... (128-bit "
                         "loads where N and K are multiples of 4); with --only, a probe of chosen variants")
    ap.add_argument("--only", default=None,
                    help="comma-separated name substrings: sweep only the variants whose name contains one "
                         "(the table's current entries are always swept, so the winner is compared with them)")
    ap.add_argument("--vec-class", type=int, default=None, choices=[0, 1],
                    help="run only the cases of this vector-load class (0: unaligned, 1: aligned); with "
                         "--table-from, rewrite only its entries (--classes limits the classes likewise)")
    args = ap.parse_args()
    if args.table_from:
        classes = set(args.classes.split(","))
        results = [r for r in load_results(args.table_from.split(","))
                   if r["class"] in classes and (args.vec_class is None or r["vec_class"] == args.vec_class)]
        write_table(choose_winners(results, args.keep_margin))
        return 0

    import numpy as np
    import torch

    import fp32_gemm_05_amd as sg
    import oracle
    from fp32_gemm_05_amd.workloads import WORKLOADS, make_inputs, sample_points

    nvar = sg.sgemm_num_variants()
    infos = [sg.sgemm_variant_info(v) for v in range(nvar)]
    if args.only:
        keep = set(name for name, _ in read_table().values())
        subs = [x for x in args.only.split(",") if x]
        wanted = [info for info in infos if info["name"] in keep or any(x in info["name"] for x in subs)]
    else:
        wanted = infos
    stream = torch.cuda.current_stream()

    flush = {}

    def sweep(label, cls, A, B, C0, alpha, beta, vec_ok, points_seed, op="NN"):
        """Time every applicable variant of the operand form op ("NN": plain; "NT", "TN", "TT":
        op(A), op(B) with the transposed operands stored transposed, through sgemm_op) on one
        problem; parity-gate each on sampled outputs.  Returns the result records."""
        ta, tb = op[0] == "T", op[1] == "T"
        states = STATES if cls in COLD_CLASSES else ("warm",)
        if len(states) > 1 and not flush:
            flush["buf"] = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device="cuda")
            flush["out"] = torch.empty((), dtype=torch.float32, device="cuda")
        M, K = A.shape
        N = B.shape[1]
        out = []
        I, J = sample_points(M, N, args.points, seed=points_seed, tile=64)
        ref, bound = oracle.ref_points(A, B, C0, I, J, alpha, beta)
        dA = torch.from_numpy(np.ascontiguousarray(A.T) if ta else A).cuda()
        dB = torch.from_numpy(np.ascontiguousarray(B.T) if tb else B).cuda()
        lda, ldb = dA.shape[1], dB.shape[1]
        dC0 = torch.from_numpy(C0).cuda()
        dC = torch.empty_like(dC0)
        flops = 2.0 * M * N * K
        log(f"== {label} ({cls}, vec={vec_ok}): M={M} N={N} K={K} alpha={alpha} beta={beta}")
        for v, info in enumerate(infos):
            if info not in wanted:
                continue
            if info["vec"] and not vec_ok:
                continue
            if (bool(info["trans_a"]), bool(info["trans_b"])) != (ta, tb):
                continue  # each variant serves one operand form
            dC.copy_(dC0)

            def call():
                sg.sgemm_op_ex(op[0], op[1], M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb, beta,
                               dC.data_ptr(), N, stream=stream.cuda_stream, variant=v)

            call()
            torch.cuda.synchronize()
            got = dC.cpu().numpy()[I, J].astype(np.float64)
            ok = bool(np.isfinite(got).all() and (np.abs(got - ref) <= bound).all())
            ratio = float((np.abs(got - ref) / bound).max())
            # timing: beta != 0 keeps reading/writing C; the values drift but the work is identical
            for _ in range(2):
                call()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            est = max(e0.elapsed_time(e1) * 1e-3, 1e-6)
            for state in states:
                for _ in range(int(min(20000, args.warm_time / est))):
                    call()
                reps = int(max(5, min(500 if state == "warm" else 60, args.min_time / est)))
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(reps)]
                for i, (s, e) in enumerate(evs):
                    if state == "cold":
                        torch.sum(flush["buf"], dim=0, out=flush["out"])
                    elif state == "dirty":
                        flush["buf"].fill_(float(i))
                    s.record(stream)
                    call()
                    e.record(stream)
                torch.cuda.synchronize()
                ts = sorted(s.elapsed_time(e) for s, e in evs)
                med = ts[len(ts) // 2]
                case = label if len(states) == 1 else f"{label}@{state}"
                rec = {"case": case, "class": cls, "vec_class": int(vec_ok), "state": state, "op": op, "M": M, "N": N,
                       "K": K, "variant": info["name"], "variant_id": v, "parity": ok, "max_err_over_bound": ratio,
                       "ms_median": med, "ms_min": ts[0], "reps": reps, "tflops": flops / (med * 1e-3) / 1e12}
                out.append(rec)
                log(f"   {info['name']:36s} {'ok ' if ok else 'BAD'} err/bound={ratio:.3g} "
                    f"median {med:.4f} ms {state:5s}  {rec['tflops']:.2f} TFLOP/s")
        del dA, dB, dC, dC0
        torch.cuda.empty_cache()
        return out

    if args.regret or args.shapes:
        return regret_mode(args, sg, sweep)

    classes = set(args.classes.split(","))
    results = []
    for (label, cls, wname, M, N, K, dist, alpha, beta, vec_ok) in CASES:
        if cls not in classes:
            continue
        if args.vec_class is not None and int(vec_ok) != args.vec_class:
            continue
        w = WORKLOADS[wname]
        M = M or w.M
        N = N or w.N
        K = K or w.K
        alpha = w.alpha if alpha is None else alpha
        beta = w.beta if beta is None else beta
        A, B, C0 = make_inputs(w, M=M, N=N, K=K, dist=dist, beta=beta)
        results += sweep(label, cls, A, B, C0, alpha, beta, vec_ok, w.seed + 17)

    winners = choose_winners(results, args.keep_margin)
    os.makedirs(os.path.dirname(args.out), exist_ok=True)
    with open(args.out, "w") as f:
        json.dump({"time": time.strftime("%Y-%m-%d %H:%M:%S"), "results": results,
                   "winners": {f"{c}/{v}": w for (c, v), w in winners.items()}}, f, indent=1)
    log(f"wrote {args.out}")
    if args.write_table and winners:
        write_table(winners)
    return 0


if __name__ == "__main__":
    sys.exit(main())
