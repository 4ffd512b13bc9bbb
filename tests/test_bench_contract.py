"""The bench's output contract: one JSON line with the fields the driver reads, the roofline
object of the dispatched kernel (against HBM for the tall-skinny workload), and the CPU baselines.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
        "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}
ROOF_KEYS = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


def _bench(*args, timeout=240):
    print(f"[bench] {' '.join(args)}", flush=True)
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                         capture_output=True, text=True, timeout=timeout)
    return res


def _line(res):
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout  # exactly one line on stdout
    return json.loads(lines[0])


def test_more_than_one_gpu_is_refused():
    res = _bench("--gpus", "2", timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_line_headline_fields():
    d = _line(_bench("--steps", "5", "--warmup", "2", "--workload", "square256"))
    assert KEYS <= set(d)
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["dtype"] == "f32"
    assert d["vs_baseline"] is None
    assert d["config"]["M"] == d["config"]["N"] == d["config"]["K"] == 256
    assert d["config"]["workload"].startswith("sgemm 256x256x256")
    r = d["roofline"]
    assert ROOF_KEYS <= set(r) and r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 157.3
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # 2*M*N*K over the time per step
    assert abs(d["value"] - 2 * 256 ** 3 / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"] + 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["unit"] == "TFLOP/s"
    assert d["parity"]["pass"] is True
    # the engine clock right before and right after the timed region, read on the GPU
    for when in ("before", "after"):
        assert 100.0 <= d["sclk_mhz"][when] <= 2600.0, d["sclk_mhz"]
    # the reported pre-roll, and the launch floor of the dispatched grid
    assert d["preroll"]["seconds"] >= 0 and d["preroll"]["steps"] >= 0
    lf = d["launch_floor"]
    from fp32_gemm_05_amd import _binding as sg
    info = next(sg.sgemm_variant_info(i) for i in range(sg.sgemm_num_variants())
                if sg.sgemm_variant_name(i) == d["config"]["variant"])
    tiles = -(-256 // info["BM"]) * -(-256 // info["BN"])
    assert lf["us"] > 0 and lf["workgroups"] == tiles and lf["threads"] == info["threads"]
    assert abs(lf["floor_over_launch"] - lf["us"] * 1e-3 / d["ms_per_step"]) <= 0.01 * lf["floor_over_launch"] + 1e-3


@pytest.mark.gpu
def test_bench_skinny_reports_against_hbm():
    d = _line(_bench("--steps", "20", "--warmup", "20", "--workload", "skinny65536x64x1024",
                     "--no-cpu-baseline"))
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    alg = 4.0 * (65536 * 1024 + 1024 * 64 + 65536 * 64)  # beta = 0: C written once
    assert abs(r["achieved"] - alg / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * r["achieved"]
    assert 0.0 < r["frac"] < 1.0
    rc = d["roofline_compute"]
    assert rc["bound"] == "mfma" and rc["unit"] == "TFLOP/s"
    assert d["cpu_baseline"] is None
