"""The autotuner's selection rule and the dispatch table it writes, checked on the CPU.

The rule: per (shape class, vector-load class), among the variants that ran and passed the
oracle check on every representative case, the one with the smallest geometric mean of
(time / per-case best); the table's current entry stays unless that winner beats it by more than
the keep margin.  The table must name only variants the library has, and a vector-load variant
never serves the scalar class.
"""
import json
import math
import re

import pytest

import autotune
import fp32_gemm_05_amd as sg


def _rec(case, variant, ms, parity=True, cls="large", vec=1):
    return {"case": case, "class": cls, "vec_class": vec, "variant": variant, "ms_median": ms,
            "parity": parity}


@pytest.fixture
def incumbent(monkeypatch):
    table = {}
    monkeypatch.setattr(autotune, "read_table", lambda: dict(table))
    return table


def test_geo_mean_winner(incumbent):
    res = [_rec("a", "x", 1.0), _rec("b", "x", 2.3),
           _rec("a", "y", 1.1), _rec("b", "y", 2.0)]
    # x: sqrt(1.0 * 1.15) = 1.072, y: sqrt(1.1 * 1.0) = 1.049
    win = autotune.choose_winners(res, 0.01)
    assert win[("large", 1)][0] == "y"
    assert math.isclose(win[("large", 1)][1], math.sqrt(1.1))


def test_incumbent_kept_within_margin(incumbent):
    incumbent[("large", 1)] = ("old", 1.0)
    res = [_rec("a", "old", 1.005), _rec("a", "new", 1.0)]
    assert autotune.choose_winners(res, 0.01)[("large", 1)][0] == "old"
    res = [_rec("a", "old", 1.02), _rec("a", "new", 1.0)]
    assert autotune.choose_winners(res, 0.01)[("large", 1)][0] == "new"
    # an incumbent that failed parity is never kept
    res = [_rec("a", "old", 1.0, parity=False), _rec("a", "new", 1.004)]
    assert autotune.choose_winners(res, 0.01)[("large", 1)][0] == "new"


def test_parity_failure_or_missing_case_disqualifies(incumbent):
    res = [_rec("a", "fast_wrong", 0.5, parity=False), _rec("b", "fast_wrong", 0.5),
           _rec("a", "partial", 0.6),  # never ran on case b
           _rec("a", "ok", 1.0), _rec("b", "ok", 1.0)]
    win = autotune.choose_winners(res, 0.01)
    assert win[("large", 1)][0] == "ok"
    # the per-case best counts every passing run: 0.6 on case a ("partial"), 0.5 on case b
    # ("fast_wrong" passed there)
    assert math.isclose(win[("large", 1)][1], math.sqrt(1.0 / 0.6 * 1.0 / 0.5))


def test_table_round_trip(tmp_path, monkeypatch):
    path = tmp_path / "table.inc"
    monkeypatch.setattr(autotune, "TABLE", str(path))
    winners = {("large", 1): ("mfma32_128x128x16_w64x64_d4_vec", 1.0),
               ("skinny", 0): ("mfma32_64x64x32_w32x32_d3_scalar", 1.0614)}
    autotune.write_table(winners)
    text = path.read_text()
    assert '{kLarge, 1, "mfma32_128x128x16_w64x64_d4_vec"}' in text
    assert "(warm, cold, dirty)" in text  # the skinny class is scored over three cache states
    back = autotune.read_table()
    assert back[("large", 1)][0] == "mfma32_128x128x16_w64x64_d4_vec"
    assert back[("skinny", 0)] == ("mfma32_64x64x32_w32x32_d3_scalar", 1.061)


def test_committed_table_names_real_variants():
    """Every entry of the committed table names a variant of the library, of its vector-load class
    (a scalar-load variant may serve the vector class, never the reverse) and with untransposed
    operands; every class has both entries."""
    text = open(autotune.TABLE).read()
    entries = re.findall(r'\{(k\w+), (\d), "([\w]+)"\}', text)
    names = {sg.sgemm_variant_name(v): v for v in range(sg.sgemm_num_variants())}
    seen = set()
    for cls, vec, name in entries:
        assert name in names, name
        info = sg.sgemm_variant_info(names[name])
        assert not (info["vec"] and vec == "0"), name
        assert info["trans_a"] == 0 and info["trans_b"] == 0, name
        seen.add((cls, vec))
    assert seen == {(c, v) for c in autotune.CLASS_IDS.values() for v in ("0", "1")}


def test_case_labels_match_the_library_classes():
    """Every representative case sits in the shape class it tunes: the library dispatches it to
    the table's entry for that (class, alignment)."""
    from fp32_gemm_05_amd.workloads import WORKLOADS
    table = autotune.read_table()
    names = {sg.sgemm_variant_name(i): i for i in range(sg.sgemm_num_variants())}
    A, B, C = 0x10000000, 0x20000000, 0x30000000  # aligned, never dereferenced
    for label, cls, wname, M, N, K, _dist, _a, _b, vec in autotune.CASES:
        w = WORKLOADS[wname]
        M, N, K = M or w.M, N or w.N, K or w.K
        if vec:
            assert N % 4 == 0 and K % 4 == 0, label
        want = names[table[(cls, int(vec))][0]]
        # a scalar case as the library sees unaligned data (A one float off 16-byte alignment)
        got = sg.sgemm_select_variant(M, N, K, A + (0 if vec else 4), K, B, N, C, N)
        assert got == want, (label, cls, sg.sgemm_variant_name(got), sg.sgemm_variant_name(want))


def test_shape_class_mirror_matches_the_library():
    """The tuner's restatement of the library's shape classes, on random shapes of the regret
    distribution and on each class boundary: the library dispatches every shape to the table's
    entry for the class the mirror gives it."""
    import numpy as np
    table = autotune.read_table()
    names = {sg.sgemm_variant_name(i): i for i in range(sg.sgemm_num_variants())}
    rng = np.random.default_rng(5)
    shapes = [(int(np.exp(rng.uniform(np.log(16), np.log(70000)))), int(np.exp(rng.uniform(np.log(4), np.log(9000)))),
               int(np.exp(rng.uniform(np.log(4), np.log(9000))))) for _ in range(400)]
    shapes += [(64 * 127, 64, 512), (64 * 128, 64, 512), (2048, 32 * 64, 511), (2048, 2048, 127), (2048, 2048, 128),
               (256 * 64, 64 * 128, 1024), (256 * 64, 64 * 128, 1025), (128 * 32, 128 * 64, 4096),
               (512, 1024, 700), (513, 1024, 700), (512, 1024, 300), (513, 1024, 300), (472, 1079, 2500),
               (1024, 1536, 700), (1025, 1536, 700), (1025, 1536, 2048)]
    for M, N, K in shapes:
        cls = autotune.shape_class(M, N, K)
        got = sg.sgemm_select_variant(M, N, K, 0x10000004, K, 0x20000000, N, 0x30000000, N)  # scalar class
        assert got == names[table[(cls, 0)][0]], (M, N, K, cls, sg.sgemm_variant_name(got))
        Na, Ka = N + (-N) % 4, K + (-K) % 4  # and the vector class (two classes can share a scalar entry)
        got = sg.sgemm_select_variant(M, Na, Ka, 0x10000000, Ka, 0x20000000, Na, 0x30000000, Na)
        cls = autotune.shape_class(M, Na, Ka)
        assert got == names[table[(cls, 1)][0]], (M, Na, Ka, cls, sg.sgemm_variant_name(got))


def test_parse_shapes():
    assert autotune.parse_shapes("472x1079x700,88X5431x2501") == [(472, 1079, 700, False, 0.0, "NN"),
                                                                   (88, 5431, 2501, False, 0.0, "NN")]
    assert autotune.parse_shapes("512x1024x560,nt:512x1024x560") == [(512, 1024, 560, True, 0.0, "NN"),
                                                                      (512, 1024, 560, True, 0.0, "NT")]
    # a transposed A is stored K x M: its rows are M long
    assert autotune.parse_shapes("TN:510x1024x560,TT:512x1024x560") == [(510, 1024, 560, False, 0.0, "TN"),
                                                                         (512, 1024, 560, True, 0.0, "TT")]
    for bad in ("0x4x4", "XN:4x4x4"):
        with pytest.raises(ValueError):
            autotune.parse_shapes(bad)


def test_transposed_records_stay_out_of_the_table(tmp_path):
    rec = {"case": "c", "class": "random", "vec_class": 1, "state": "warm", "M": 512, "N": 512, "K": 512,
           "variant": "v", "parity": True, "ms_median": 1.0}
    path = tmp_path / "r.json"
    path.write_text(json.dumps({"results": [dict(rec, op="TN"), dict(rec, variant="w"), dict(rec, variant="x", op="NN")]}))
    got = autotune.load_results([str(path)])
    assert sorted(r["variant"] for r in got) == ["w", "x"]
