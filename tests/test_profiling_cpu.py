"""The profiling summaries from synthetic rocprofv3 output: `report` (the copy calibration, the HBM
bytes per launch, the MFMA count the problem needs for the variant's block size, the busy fractions,
the command list of a forced-variant run) and `lds-passes` (the LDS pass grouping from lane-pair
counters).  No GPU: the CSV files are written here.
"""
import csv
import json
import os
import sys

import pytest

from fp32_gemm_05_amd import profiling

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _counters(path, kernel, per_dispatch):
    """per_dispatch: [(duration_ns, {counter: value})]"""
    rows, t = [], 1000
    for i, (ns, cs) in enumerate(per_dispatch):
        for c, v in cs.items():
            rows.append([i + 1, kernel, c, v, t, t + ns])
        t += ns + 1000
    _write(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"], rows)


def _fake_run(d, tag, kernel, disp_ns, steps, gui_per_xcd, busy_frac, fetch_kib, write_kib, mfma):
    n = len(disp_ns)
    _write(os.path.join(d, f"trace_{tag}", "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
           [[kernel, n, sum(disp_ns) / n, min(disp_ns), max(disp_ns)], ["copyBuffer", 1, 5, 5, 5]])
    rows, t = [], 0
    for ns in disp_ns:
        rows.append([kernel, t, t + ns])
        t += ns + 100
    _write(os.path.join(d, f"trace_{tag}", "run_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           rows)
    gui = gui_per_xcd * profiling.N_XCD
    sq = {"GRBM_GUI_ACTIVE": gui, "SQ_VALU_MFMA_BUSY_CYCLES": busy_frac * profiling.N_SIMD * gui_per_xcd,
          "SQ_INSTS_MFMA": mfma, "SQ_LDS_BANK_CONFLICT": 0.0, "SQ_INSTS_LDS": 1.0, "SQ_INSTS_VALU": 1.0,
          "SQ_BUSY_CYCLES": 1.0, "SQ_WAVES": 1.0, "SQ_INSTS_VALU_MFMA_MOPS_F32": 1.0}
    _counters(os.path.join(d, f"sq_{tag}", "run_counter_collection.csv"), kernel, [(200_000, sq)] * 4)
    _counters(os.path.join(d, f"fetch_{tag}", "run_counter_collection.csv"), kernel,
              [(1000, {"FETCH_SIZE": fetch_kib})] * 4)
    _counters(os.path.join(d, f"write_{tag}", "run_counter_collection.csv"), kernel,
              [(1000, {"WRITE_SIZE": write_kib})] * 4)
    _counters(os.path.join(d, f"rdreq_{tag}", "run_counter_collection.csv"), kernel,
              [(1000, {"TCC_EA0_RDREQ_32B_sum": 0.0, "TCC_EA0_RDREQ_64B_sum": 0.0,
                       "TCC_EA0_RDREQ_128B_sum": 1000.0})] * 4)
    # a copy of 1 GiB that the counters see as 2 GiB read and 0.5 GiB written
    _counters(os.path.join(d, "copy_fetch", "run_counter_collection.csv"), "copyBuffer",
              [(1000, {"FETCH_SIZE": 2.0 * 1024 ** 2})])
    _counters(os.path.join(d, "copy_write", "run_counter_collection.csv"), "copyBuffer",
              [(1000, {"WRITE_SIZE": 0.5 * 1024 ** 2})])


@pytest.mark.parametrize("forced", [False, True])
def test_report_from_synthetic_runs(tmp_path, forced):
    W = "square1024_beta"
    variant = "mfma16l_64x64x32_w32x16_s3_cp_sp_vec" if forced else "mfma32l_64x64x32_w32x32_s3_cp_sp_vec"
    tag = f"{W}__{variant}" if forced else W
    d = str(tmp_path / "raw")
    steps = 10
    disp = [30_000] * 3 + [20_000] * steps + [21_000] * steps  # first calls, timed region, single launches
    M = N = K = 1024
    mfma = M * N * K / (1024 if forced else 2048)
    _fake_run(d, tag, "sgemm_kernel", disp, steps, gui_per_xcd=100_000, busy_frac=0.8, fetch_kib=4096.0,
              write_kib=8192.0, mfma=mfma)
    out = str(tmp_path / "profiles")
    args = profiling.argparse.Namespace(dir=d, workload=W, variant=variant, steps=steps, sq_warmup=1,
                                        trace_args="--warmup 100" + (f" --variant {variant}" if forced else ""),
                                        out_dir=out, note="", run_tag=tag)
    profiling.cmd_report(args)
    md = open(os.path.join(out, f"{variant}__{W}.md")).read()
    rec = json.load(open(os.path.join(out, f"traffic_{variant}_{W}.json")))
    assert rec["avg_ns_timed_region"] == 20_000  # the `steps` launches before the single ones
    # the copy reads count 2x and the writes 0.5x the bytes moved: scales 0.5 and 2
    assert rec["fetch_scale"] == pytest.approx(0.5) and rec["write_scale"] == pytest.approx(2.0)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(4096 * 1024 * 0.5 + 8192 * 1024 * 2.0)
    assert rec["mfma_busy"] == pytest.approx(0.8)
    assert rec["kernel_source_hash"] == profiling.kernel_source_hash(variant)
    need = "v_mfma_f32_16x16x4_f32" if forced else "v_mfma_f32_32x32x2_f32"
    assert f"the problem needs {mfma:.6g} {need}" in md
    if forced:
        assert f"--variant {variant}" in md and f"trace_{tag}" in md and f"--run-tag {tag}" in md
    else:
        assert "--variant" not in md.split("## Commands")[1].split("report")[0]


def test_kernel_sources_cover_every_family():
    """Every variant of the library maps to its kernel family's header (the hash of a counter
    summary covers the code the variant runs)."""
    from fp32_gemm_05_amd import _binding as sg
    for i in range(sg.sgemm_num_variants()):
        name = sg.sgemm_variant_name(i)
        assert len(profiling.kernel_sources(name)) == len(profiling.KERNEL_COMMON) + 1, name


def test_stamps_build_matches_the_library():
    """The phase-stamp build (libsgemm_stamps.so) has the product library's variants in the same
    order and exports sgemm_phase_stamps; the product library does not (its hooks compile away)."""
    import ctypes
    from fp32_gemm_05_amd import _binding as sg
    from fp32_gemm_05_amd import build as hb
    if not os.path.exists(hb.STAMPS_LIB):
        pytest.skip("libsgemm_stamps.so not built")
    st = sg.load_library(hb.STAMPS_LIB)
    prod = sg.load_library()
    assert st.sgemm_num_variants() == prod.sgemm_num_variants()
    for i in range(prod.sgemm_num_variants()):
        assert st.sgemm_variant_name(i) == prod.sgemm_variant_name(i)
    assert hasattr(st, "sgemm_phase_stamps")
    with pytest.raises(AttributeError):
        ctypes.CDLL(hb.LIB).sgemm_phase_stamps


def _lds_model_passes(width):
    """The pass grouping of the kernel model (tests/test_kernel_model.py)."""
    from test_kernel_model import lds_passes
    return lds_passes(width)


def test_lds_passes_report_round_trip(tmp_path):
    """`profiling lds-passes` recovers a pass grouping from the counters of the lane-pair probe:
    synthetic counters that conflict exactly when the two lanes share a pass of the kernel model."""
    plan = profiling.lds_probe_plan()
    rows = []
    for d, (width, i, j, _) in enumerate(plan):
        same = any(i in p and j in p for p in _lds_model_passes(width))
        rows.append([d + 1, "lds_probe_kernel", "SQ_LDS_BANK_CONFLICT", 64.0 if same else 0.0, 0, 1])
    path = str(tmp_path / "c.csv")
    _write(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"], rows)
    out = str(tmp_path / "lds.md")
    profiling.cmd_lds_passes(profiling.argparse.Namespace(csv=path, reps=64, out=out))
    md = open(out).read()
    assert "| 128-bit | 0 | 1-3, 12-15, 20-27 |" in md
    assert "| 64-bit | 32 | 33-63 |" in md and "| 32-bit | 8 | 0-7, 9-63 |" in md


def test_lds_model_matches_the_committed_measurement():
    """The kernel model's pass grouping is the one the committed probe summary measured."""
    import re
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles", "lds_passes.md")
    if not os.path.exists(path):
        pytest.skip("no committed LDS pass summary")
    table = {}
    for m in re.finditer(r"^\| (\d+)-bit \| (\d+) \| ([^|]*) \|$", open(path).read(), re.M):
        lanes = set()
        for part in m.group(3).split(","):
            part = part.strip()
            if part and part != "none":
                a, _, b = part.partition("-")
                lanes |= set(range(int(a), int(b or a) + 1))
        table[(int(m.group(1)) // 8, int(m.group(2)))] = lanes
    assert table, "no table rows in the summary"
    for (width, i), lanes in table.items():
        (mine,) = [set(p) - {i} for p in _lds_model_passes(width) if i in p]
        assert lanes == mine, (width, i)


def test_write_reference_rejects_bad_shapes_without_launching():
    """hbm_write_tiles checks its arguments before any HIP call: a null matrix, sizes that are not
    positive multiples of 64 and a row stride shorter than a row are refused with -1."""
    lib = profiling._hbm_read_lib()
    fake = 0x10000000
    assert lib.hbm_write_tiles(None, 64, 64, 64, 0, None) == -1
    assert lib.hbm_write_tiles(fake, 63, 64, 64, 0, None) == -1
    assert lib.hbm_write_tiles(fake, 64, 96, 128, 1, None) == -1
    assert lib.hbm_write_tiles(fake, 64, 128, 64, 0, None) == -1
    assert lib.hbm_write_tiles(fake, 0, 64, 64, 0, None) == -1
