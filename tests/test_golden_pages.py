"""The pages' printed figures as fixed expected values (tests/golden/page_figures.json).

* The bench's FLOP count (2*M*N*K) and rate must turn the pages' measured times at 4096^3
  into the rates they print.
* The panel-read model the profiling summaries report must give the page's loads per output
  element and total traffic for its 64 x 64 tiling.
* The 128-bit load precondition of the library: the page's 15 x 15 example has row starts
  that are 16-byte aligned only on every fourth row, so a packed 15-column operand must be
  refused by the vector variants (the whole-kernel fallback the page takes), while the same
  rows padded to 16 columns must be accepted.
"""
import json
import math
import os

import pytest

import fp32_gemm_05_amd as sg
from fp32_gemm_05_amd.roofline import gemm_flops, panel_read_bytes, tflops

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


@pytest.mark.parametrize("fig", GOLDEN["flop_rates"], ids=lambda f: f"{f['ms']}ms")
def test_flop_rate_convention(fig):
    got = tflops(fig["M"], fig["N"], fig["K"], fig["ms"]) * 1e3
    # the printed time is rounded to 1 us and the printed rate to 0.1 GFLOP/s
    tol = got * 0.0005 / fig["ms"] + 0.05
    assert abs(got - fig["gflops"]) <= tol, (got, fig)
    # counting M*N*K (one per fused multiply-add) would miss by far more
    assert abs(got / 2 - fig["gflops"]) > 100 * tol


@pytest.mark.parametrize("fig", GOLDEN["speedups"], ids=lambda f: f"x{f['ratio']}")
def test_printed_speedups_are_time_ratios(fig):
    # rates at a fixed size are inverse to times, so the printed speedups are time ratios
    r = fig["ms_before"] / fig["ms_after"]
    digits = len(str(fig["ratio"]).split(".")[1])
    assert round(r, digits) == fig["ratio"]
    rate = lambda ms: tflops(4096, 4096, 4096, ms)  # noqa: E731
    assert math.isclose(rate(fig["ms_after"]) / rate(fig["ms_before"]), r, rel_tol=1e-12)


@pytest.mark.parametrize("fig", GOLDEN["panel_reads"], ids=lambda f: f"{f['BM']}x{f['BN']}")
def test_panel_read_model(fig):
    M, N, K, BM, BN = fig["M"], fig["N"], fig["K"], fig["BM"], fig["BN"]
    total = panel_read_bytes(M, N, K, BM, BN)
    assert total / (4.0 * M * N) == fig["loads_per_output"]
    assert round(total / 1e9, 2) == fig["total_GB"]
    # doubling both tile sides halves the panel traffic; the count is 2 FLOPs per loaded pair
    assert panel_read_bytes(M, N, K, 2 * BM, 2 * BN) == total / 2
    assert gemm_flops(M, N, K) == 2.0 * M * N * K


def _vec_variant():
    for i in range(sg.sgemm_num_variants()):
        info = sg.sgemm_variant_info(i)
        if info["vec"] and not info["trans_a"] and not info["trans_b"] and not info["wide"]:
            return i
    raise AssertionError("no 128-bit variant in the library")


@pytest.mark.parametrize("fig", GOLDEN["vector_alignment"], ids=lambda f: f"{f['rows']}x{f['cols']}")
def test_vector_alignment_example(fig):
    n, t = fig["cols"], fig["tile"]
    assert -(-fig["rows"] // t) == fig["tiles_per_dim"]
    r0, r1 = fig["tile_1_0_rows"]
    assert (r0, r1) == (1 * t, 2 * t) and tuple(fig["tile_1_0_cols"]) == (0, t)
    # element offsets of row starts in the packed matrix, and their 16-byte alignment
    for off in fig["float4_legal_offsets"]:
        assert off % n == 0 and (off * 4) % 16 == 0
    for off in fig["float4_illegal_offsets"]:
        assert off % n == 0 and (off * 4) % 16 != 0
    aligned_rows = [r for r in range(fig["rows"]) if (r * n * 4) % 16 == 0]
    assert aligned_rows == list(range(0, fig["rows"], 4))

    # The library takes the page's choice: with a 15-float row pitch some rows are misaligned,
    # so no 128-bit variant is selected or accepted; a 16-float pitch aligns every row.
    base = 1 << 20  # 16-byte aligned addresses; only their values are inspected
    A, B, C = base, base + (1 << 16), base + (1 << 17)
    m = k = fig["rows"]
    vid = sg.sgemm_select_variant(m, n, k, A, n, B, n, C, n)
    assert not sg.sgemm_variant_info(vid)["vec"]
    with pytest.raises(sg.SgemmArgumentError):
        sg.sgemm_ex(m, n, k, 1.0, A, n, B, n, 0.0, C, n, stream=0, variant=_vec_variant())
    # padded to 16 columns (a multiple of 4 floats) every row is aligned: n itself must also
    # be a multiple of 4 for the vector path, so use 16 columns of data
    vid16 = sg.sgemm_select_variant(16, 16, 16, A, 16, B, 16, C, 16)
    assert sg.sgemm_variant_info(vid16)["vec"]
