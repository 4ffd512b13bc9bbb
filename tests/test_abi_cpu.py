"""CPU-side checks of the C ABI: the library loads, exports what include/sgemm.h declares,
validates arguments and chooses variants without touching a GPU.

No call here launches work: every call either fails validation, is a quick
return with M == 0 or N == 0, or is a pure host function.
"""
import ctypes
import os
import re

import pytest

import fp32_gemm_05_amd as sg
from fp32_gemm_05_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"SGEMM_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_abi():
    names = declared_symbols()
    for n in ["sgemm", "sgemm_ex", "sgemm_num_variants", "sgemm_variant_name", "sgemm_variant_info",
              "sgemm_select_variant", "sgemm_tile_order", "sgemm_last_variant", "sgemm_version"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sg.library_path())
    for n in declared_symbols():
        assert hasattr(lib, n), f"{n} declared in sgemm.h but not exported"


def test_version_and_variants():
    assert "libsgemm" in sg.sgemm_version()
    n = sg.sgemm_num_variants()
    assert n >= 4
    names = [sg.sgemm_variant_name(i) for i in range(n)]
    assert len(set(names)) == n
    assert sg.sgemm_variant_name(-1) is None and sg.sgemm_variant_name(n) is None
    kinds = set()
    for i in range(n):
        info = sg.sgemm_variant_info(i)
        kinds.add(info["kind"])
        if info["kind"] == "mfma":
            # the name's prefix gives the MFMA block edge
            assert info["name"].startswith(f"mfma{info['mfma_block']}")
            assert info["mfma_block"] in (32, 16)
        else:
            assert info["name"].startswith("valu_") and info["mfma_block"] == 0
        assert f"{info['BM']}x{info['BN']}x{info['BK']}" in info["name"]
        assert info["name"].endswith("_vec") == bool(info["vec"])
        assert info["threads"] % 64 == 0 and info["threads"] <= 1024
        assert info["lds_bytes"] <= 160 * 1024
    assert kinds == {"mfma", "valu"}
    with pytest.raises(ValueError):
        sg.sgemm_variant_info(n)


FAKE_A, FAKE_B, FAKE_C = 0x10000000, 0x20000000, 0x30000000  # never dereferenced


def _call(M, N, K, lda, ldb, ldc, A=FAKE_A, B=FAKE_B, C=FAKE_C, alpha=1.0, beta=0.0, variant=-1):
    lib = sg.load_library()
    return lib.sgemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None, variant)


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, 4, 4, 4), -1),
    ((4, -1, 4, 4, 1, 1), -2),
    ((4, 4, -1, 1, 4, 4), -3),
    ((4, 4, 4, 3, 4, 4), -6),
    ((4, 4, 4, 4, 3, 4), -8),
    ((4, 4, 4, 4, 4, 3), -11),
    ((4, 4, 0, 0, 4, 4), -6),   # lda >= max(1, K)
    ((4, 0, 4, 4, 0, 1), -8),   # ldb >= max(1, N)
])
def test_invalid_arguments(args, code):
    assert _call(*args) == code


def test_null_pointers():
    assert _call(4, 4, 4, 4, 4, 4, C=None) == -10
    assert _call(4, 4, 4, 4, 4, 4, A=None) == -5
    assert _call(4, 4, 4, 4, 4, 4, B=None) == -7


def test_overlapping_c_rejected():
    # C overlaps A's addressed range
    assert _call(4, 4, 4, 4, 4, 4, A=FAKE_C + 16) == -10
    # C overlaps B's addressed range
    assert _call(4, 4, 4, 4, 4, 4, B=FAKE_C - 16) == -10


def test_overlap_check_compares_address_spans():
    """Disjoint column ranges of the same rows (A = X[:, :4], C = X[:, 4:8] with ld 8) share no
    element, but their address spans interleave: the span check refuses them (-10), as
    include/sgemm.h states.  Disjoint row ranges of one allocation pass."""
    X = FAKE_A
    assert _call(4, 4, 4, 8, 4, 8, A=X, C=X + 16) == -10
    assert _call(4, 4, 4, 8, 4, 8, B=X, C=X + 16, A=FAKE_B) == -10
    # rows 0..3 for A (K = 8, ld 8), rows 4..7 for C: spans [X, X + 128) and [X + 128, X + 256);
    # validation passes and the out-of-range variant id is reported instead (nothing launches)
    assert _call(4, 8, 8, 8, 8, 8, A=X, C=X + 4 * 8 * 4, variant=sg.sgemm_num_variants()) == -13


def test_extents_beyond_the_limit_are_refused():
    """M, N or K above 2^31 - 1025 are refused before any launch (tile and slab coordinates would
    leave int), and the dispatcher reports no variant for them instead of a wrapped tile count."""
    big = 2 ** 31 - 1
    assert _call(big, 1, 1, 1, 1, 1) == -1
    assert _call(1, big, 1, 1, big, big) == -2
    assert _call(1, 1, big, big, 1, 1) == -3
    assert sg.sgemm_select_variant(big, 1, 1, FAKE_A, 1, FAKE_B, 1, FAKE_C, 1) == -1
    assert sg.sgemm_op_select_variant("N", "N", 1, big, 1, FAKE_A, 1, FAKE_B, big, FAKE_C, big) == -1
    lim = 2 ** 31 - 1025
    # at the limit the dispatcher still answers (a tall single column: the narrow class)
    v = sg.sgemm_select_variant(lim, 1, 1, FAKE_A, 1, FAKE_B, 1, FAKE_C, 1)
    assert v >= 0 and sg.sgemm_variant_info(v)["BN"] == 32


def test_last_variant_without_launches():
    """sgemm_last_variant is -1 after calls that enqueue no GEMM kernel (invalid arguments and
    quick returns); only a successful GEMM launch sets it (checked on the GPU)."""
    assert _call(-1, 4, 4, 4, 4, 4) == -1
    assert sg.sgemm_last_variant() == -1
    assert _call(0, 4, 4, 4, 4, 4, A=None, B=None, C=None) == 0
    assert sg.sgemm_last_variant() == -1


def test_quick_returns_need_no_gpu():
    assert _call(0, 4, 4, 4, 4, 4, A=None, B=None, C=None) == 0
    assert _call(4, 0, 4, 4, 1, 1, A=None, B=None, C=None) == 0


def test_bad_variant_id():
    assert _call(4, 4, 4, 4, 4, 4, variant=sg.sgemm_num_variants()) == -13


def test_vector_variant_refuses_misaligned():
    vec = [i for i in range(sg.sgemm_num_variants()) if sg.sgemm_variant_info(i)["vec"]]
    assert vec
    for v in vec:
        assert _call(8, 8, 8, 8, 8, 8, A=FAKE_A + 4, variant=v) == -13   # pointer not 16-byte aligned
        assert _call(8, 8, 8, 9, 8, 8, variant=v) == -13                 # lda % 4 != 0
        assert _call(8, 7, 8, 8, 7, 7, variant=v) == -13                 # N % 4 != 0
        assert _call(8, 8, 6, 8, 8, 8, variant=v) == -13                 # K % 4 != 0


def test_select_variant_classes():
    n = sg.sgemm_num_variants()
    big = sg.sgemm_select_variant(4096, 4096, 4096, FAKE_A, 4096, FAKE_B, 4096, FAKE_C, 4096)
    assert 0 <= big < n and sg.sgemm_variant_info(big)["vec"] == 1
    ragged = sg.sgemm_select_variant(3001, 5003, 777, FAKE_A, 777, FAKE_B, 5003, FAKE_C, 5003)
    assert 0 <= ragged < n and sg.sgemm_variant_info(ragged)["vec"] == 0
    skinny = sg.sgemm_select_variant(65536, 64, 1024, FAKE_A, 1024, FAKE_B, 64, FAKE_C, 64)
    assert 0 <= skinny < n and sg.sgemm_variant_info(skinny)["BN"] <= 64
    # N <= 32 streams: an aligned one gets 32-wide workgroups, not half-padded 64-wide ones
    narrow = sg.sgemm_select_variant(262144, 32, 512, FAKE_A, 512, FAKE_B, 32, FAKE_C, 32)
    assert 0 <= narrow < n and sg.sgemm_variant_info(narrow)["BN"] == 32
    mis = sg.sgemm_select_variant(4096, 4096, 4096, FAKE_A + 4, 4096, FAKE_B, 4096, FAKE_C, 4096)
    assert sg.sgemm_variant_info(mis)["vec"] == 0
    assert sg.sgemm_select_variant(0, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4) == -1


def _name(v):
    return sg.sgemm_variant_name(v)


@pytest.mark.parametrize("M,N,K,ld_odd,prefix", [
    (256, 256, 256, False, "mfma16l_32x64"),   # small_shortk: 32x64 tiles, two workgroups a CU
    (822, 124, 88, False, "mfma16l_32x64"),
    (512, 512, 512, False, "mfma16l_32x64"),   # tiny: under 128 64x64 tiles
    (333, 555, 777, True, "mfma16l_32x64"),
    (1554, 64, 5093, True, "mfma16l_32x64"),   # skinny with few tiles joins the small classes
    (1024, 1024, 1024, False, "mfma32l_64x64"),  # small, aligned: 64x64 workgroups fill the CUs
    (1001, 1003, 777, True, "mfma32r_32x32x96"),  # small, unaligned: the LDS-free kernel, 96-deep
    (1199, 587, 3229, True, "mfma32r_32x32x96"),  # small_longk, unaligned
    (1111, 1113, 1001, True, "mfma16l_32x64"),  # small_full, unaligned
    (1089, 728, 5752, False, "mfma32l_64x64"),  # small_longk, aligned: the direct-to-LDS ring
    (4096, 4096, 4096, False, "mfma32_128x128"),
    (65536, 64, 1024, False, "mfma32d_128x64"),  # skinny: the deep 128x64 kernel
])
def test_dispatch_families(M, N, K, ld_odd, prefix):
    """Which kernel family and workgroup tile the shape classes pick; the 128-bit forms exactly
    when the operands allow them."""
    lda, ldb = (K | 1, N | 1) if ld_odd else (K, N)
    v = sg.sgemm_select_variant(M, N, K, FAKE_A, lda, FAKE_B, ldb, FAKE_C, ldb)
    assert v >= 0
    assert _name(v).startswith(prefix), _name(v)
    assert bool(sg.sgemm_variant_info(v)["vec"]) == (not ld_odd)


@pytest.mark.parametrize("ta,tb,M,N,K,odd,direct", [
    ("T", "N", 333, 555, 777, True, True),     # tiny: every transposition
    ("N", "T", 333, 555, 777, True, True),
    ("T", "T", 512, 512, 512, False, True),
    ("T", "T", 88, 5428, 2500, False, True),      # tiny by the 32x64 tile count
    ("T", "N", 768, 512, 600, False, True),       # aligned T N: the 96-deep form unless K % 128 == 0
    ("T", "T", 640, 384, 700, False, True),       # aligned T T: the 128-deep form below K = 768
    ("T", "T", 332, 552, 776, False, True),       # ... and the 96-deep one from there on
    ("N", "T", 768, 512, 600, False, True),
    ("T", "N", 384, 640, 640, False, True),       # K a multiple of 128
    ("T", "N", 640, 384, 701, True, True),        # unaligned
    ("T", "N", 640, 896, 720, False, True),       # small, aligned: the LDS-free kernel too
    ("N", "T", 900, 1100, 1800, False, True),     # small_full with at most 1024 32x32 tiles
    ("T", "T", 901, 1101, 1801, True, True),
    ("T", "T", 1100, 1100, 1800, False, False),   # small_full with more: 64x64 transposed kernels
    ("T", "N", 1300, 1000, 1200, False, True),    # ... but for T N
    ("T", "N", 1001, 1003, 777, True, True),   # small: only with A transposed
    ("N", "T", 1001, 1003, 777, True, False),
    ("T", "T", 4096, 4096, 4096, False, False),
    ("N", "T", 262144, 32, 512, False, False),    # narrow stream, B transposed
    ("N", "T", 65536, 64, 1024, True, False),     # skinny stream, B transposed, unaligned
])
def test_op_dispatch_families(ta, tb, M, N, K, odd, direct):
    lda = M if ta == "T" else K
    ldb = K if tb == "T" else N
    ldc = N
    if odd:
        lda, ldb, ldc = lda | 1, ldb | 1, ldc | 1
    v = sg.sgemm_op_select_variant(ta, tb, M, N, K, FAKE_A, lda, FAKE_B, ldb, FAKE_C, ldc)
    info = sg.sgemm_variant_info(v)
    assert (info["trans_a"], info["trans_b"]) == (int(ta == "T"), int(tb == "T"))
    assert _name(v).startswith("mfma32r_") == direct, _name(v)
    if direct:  # its form: 128-deep 128-bit loads, or 96-deep 32-bit loads
        deep128 = not odd and (ta == "N" or K % 128 == 0 or (tb == "T" and K < 768))
        assert _name(v).startswith("mfma32r_32x32x128_" if deep128 else "mfma32r_32x32x96_"), _name(v)
    if ta == "N" and tb == "T" and N <= 64 and M >= 65536:
        assert "_nta_nt_" in _name(v) and info["BN"] == (32 if N <= 32 else 64), _name(v)


@pytest.mark.parametrize("tiles_m,tiles_n,group_m", [
    (1, 1, 8), (1, 7, 8), (7, 1, 8), (32, 32, 8), (24, 40, 8), (3, 5, 2), (512, 1, 8), (17, 9, 4),
    (64, 64, 8), (2, 2, 8), (9, 33, 16)])
def test_tile_order_is_a_bijection(tiles_m, tiles_n, group_m):
    tm, tn = _binding.tile_order(tiles_m, tiles_n, group_m)
    pairs = set(zip(tm, tn))
    assert len(pairs) == tiles_m * tiles_n
    assert all(0 <= a < tiles_m and 0 <= b < tiles_n for a, b in pairs)


def test_tile_order_gives_each_xcd_a_compact_block():
    """Workgroups w, w+8, w+16, ... share an XCD; their tiles should cluster (few distinct rows/cols)."""
    tiles_m = tiles_n = 32  # 4096^2 at 128x128 tiles
    tm, tn = _binding.tile_order(tiles_m, tiles_n, 8)
    for x in range(8):
        ws = list(range(x, tiles_m * tiles_n, 8))[:64]    # the first 64 workgroups on XCD x
        rows = {tm[w] for w in ws}
        cols = {tn[w] for w in ws}
        assert len(rows) * len(cols) <= 2 * len(ws), (x, len(rows), len(cols))


def test_huge_leading_dimension_uses_wide_offsets():
    """A workgroup panel spanning >= 4 GiB cannot use 32-bit offsets: sgemm picks a _wide variant,
    and a forced narrow variant is refused before any launch."""
    lda = 40_000_000  # (32 - 1) * lda * 4 bytes > 2^32: no narrow tile height fits
    vid = sg.sgemm_select_variant(200, 64, 64, FAKE_A, lda, FAKE_B, 64, FAKE_C, 64)
    info = sg.sgemm_variant_info(vid)
    assert info["wide"] == 1 and info["name"].endswith("_wide_vec")
    narrow = [i for i in range(sg.sgemm_num_variants()) if not sg.sgemm_variant_info(i)["wide"]
              and not sg.sgemm_variant_info(i)["trans_a"] and not sg.sgemm_variant_info(i)["trans_b"]]
    big_a = 0x100000000  # far from C, so no overlap
    for v in narrow:
        assert _call(200, 64, 64, lda, 64, 64, A=big_a, variant=v) == -13
    # 32-row tiles still fit where 64-row ones would not: (32 - 1) * 20e6 * 4 bytes < 2^32
    vid = sg.sgemm_select_variant(200, 64, 64, FAKE_A, 20_000_000, FAKE_B, 64, FAKE_C, 64)
    assert sg.sgemm_variant_info(vid)["wide"] == 0 and sg.sgemm_variant_info(vid)["BM"] == 32
    # an ordinary leading dimension keeps the narrow variant
    vid = sg.sgemm_select_variant(4096, 4096, 4096, FAKE_A, 4096, FAKE_B, 4096, FAKE_C, 4096)
    assert sg.sgemm_variant_info(vid)["wide"] == 0


# ---- transposed operands: sgemm_op / sgemm_op_ex -------------------------------------------

def _op(ta, tb, M, N, K, lda, ldb, ldc, A=FAKE_A, B=FAKE_B, C=FAKE_C, alpha=1.0, beta=0.0, variant=-1):
    lib = sg.load_library()
    return lib.sgemm_op_ex(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None, variant)


def _trans_variants(ta, tb):
    out = []
    for i in range(sg.sgemm_num_variants()):
        info = sg.sgemm_variant_info(i)
        if info["trans_a"] == ta and info["trans_b"] == tb:
            out.append(i)
    return out


def test_header_declares_the_op_entry_points():
    names = declared_symbols()
    for n in ["sgemm_op", "sgemm_op_ex", "sgemm_op_select_variant"]:
        assert n in names, n


def test_every_transposition_has_variants():
    for ta in (0, 1):
        for tb in (0, 1):
            vs = _trans_variants(ta, tb)
            assert vs, (ta, tb)
            # each has vector, scalar and 64-bit-offset forms
            infos = [sg.sgemm_variant_info(v) for v in vs]
            assert any(i["vec"] for i in infos) and any(not i["vec"] for i in infos)
            assert any(i["wide"] and i["vec"] for i in infos) and any(i["wide"] and not i["vec"] for i in infos)
    for v in _trans_variants(0, 1) + _trans_variants(1, 0) + _trans_variants(1, 1):
        name = sg.sgemm_variant_name(v)
        info = sg.sgemm_variant_info(v)
        tag = ("t" if info["trans_a"] else "n") + ("t" if info["trans_b"] else "n")
        assert f"_{tag}_" in name, name


@pytest.mark.parametrize("ta,tb,args,code", [
    (b"X", b"N", (4, 4, 4, 4, 4, 4), -1),
    (b"N", b"?", (4, 4, 4, 4, 4, 4), -2),
    (b"N", b"N", (-1, 4, 4, 4, 4, 4), -3),
    (b"T", b"N", (4, -1, 4, 4, 1, 1), -4),
    (b"N", b"T", (4, 4, -1, 1, 1, 4), -5),
    # op(A) = A^T: A is K x M, lda >= M
    (b"T", b"N", (8, 4, 4, 7, 4, 4), -8),
    (b"T", b"N", (8, 4, 16, 8, 4, 4), 0),    # lda = 8 < K = 16 is fine for A^T: validation passes
    (b"N", b"N", (8, 4, 16, 8, 4, 4), -8),  # ... but not for A
    # op(B) = B^T: B is N x K, ldb >= K
    (b"N", b"T", (4, 8, 16, 16, 15, 8), -10),
    (b"N", b"T", (4, 8, 16, 16, 8, 8), -10),
    (b"N", b"N", (4, 8, 16, 16, 8, 8), 0),
    (b"t", b"t", (4, 4, 4, 4, 4, 3), -13),
])
def test_op_invalid_arguments(ta, tb, args, code):
    if code == 0:
        # a valid call would launch: only check that it passes validation by forcing a bad variant id
        assert _op(ta, tb, *args, variant=sg.sgemm_num_variants()) == -15
    else:
        assert _op(ta, tb, *args) == code


def test_op_null_pointers_and_quick_returns():
    assert _op(b"T", b"T", 4, 4, 4, 4, 4, 4, C=None) == -12
    assert _op(b"T", b"T", 4, 4, 4, 4, 4, 4, A=None) == -7
    assert _op(b"T", b"T", 4, 4, 4, 4, 4, 4, B=None) == -9
    assert _op(b"T", b"N", 0, 4, 4, 1, 4, 4, A=None, B=None, C=None) == 0
    assert _op(b"N", b"T", 4, 0, 4, 4, 4, 1, A=None, B=None, C=None) == 0


def test_op_overlap_uses_stored_extents():
    # A^T stored K x M = 64 x 4 with lda 4 spans 256 floats; C placed 128 floats after A overlaps it
    assert _op(b"T", b"N", 4, 4, 64, 4, 4, 4, C=FAKE_A + 512) == -12
    # as an M x K = 4 x 64 A the same span is also 256 floats
    assert _op(b"N", b"N", 4, 4, 64, 64, 4, 4, C=FAKE_A + 512) == -12
    # B^T stored N x K = 8 x 4, ldb 4: 32 floats; C right after it does not overlap
    assert _op(b"N", b"T", 4, 8, 4, 4, 4, 8, C=FAKE_B + 128, variant=sg.sgemm_num_variants()) == -15
    assert _op(b"N", b"T", 4, 8, 4, 4, 4, 8, C=FAKE_B + 124) == -12


def test_variants_serve_only_their_transposition():
    n = sg.sgemm_num_variants()
    for v in range(n):
        info = sg.sgemm_variant_info(v)
        for ta in (0, 1):
            for tb in (0, 1):
                rc = _op(b"T" if ta else b"N", b"T" if tb else b"N", 8, 8, 8, 8, 8, 8, variant=v)
                if (ta, tb) != (info["trans_a"], info["trans_b"]):
                    assert rc == -15, (info["name"], ta, tb)
        if info["trans_a"] or info["trans_b"]:
            assert _call(8, 8, 8, 8, 8, 8, variant=v) == -13, info["name"]


def test_op_vector_variants_check_stored_row_lengths():
    for ta, tb in [(1, 0), (0, 1), (1, 1)]:
        for v in _trans_variants(ta, tb):
            if not sg.sgemm_variant_info(v)["vec"]:
                continue
            t = lambda x: b"T" if x else b"N"  # noqa: E731
            # stored A row length is M when ta (M = 6 not a multiple of 4), else K
            if ta:
                assert _op(t(ta), t(tb), 6, 8, 8, 8, 8, 8, variant=v) == -15
            else:
                assert _op(t(ta), t(tb), 8, 8, 6, 8, 8, 8, variant=v) == -15
            # stored B row length is K when tb, else N
            if tb:
                assert _op(t(ta), t(tb), 8, 8, 6, 8, 8, 8, variant=v) == -15
            assert _op(t(ta), t(tb), 8, 8, 8, 8, 8, 8, A=FAKE_A + 4, variant=v) == -15
            assert _op(t(ta), t(tb), 8, 8, 8, 8, 8, 9, variant=v) == -15


def test_op_select_variant():
    for ta, tb in [(b"N", b"N"), (b"N", b"T"), (b"T", b"N"), (b"T", b"T")]:
        v = sg.sgemm_op_select_variant(ta, tb, 4096, 4096, 4096, FAKE_A, 4096, FAKE_B, 4096, FAKE_C, 4096)
        info = sg.sgemm_variant_info(v)
        assert (info["trans_a"], info["trans_b"]) == (ta == b"T", tb == b"T")
        assert info["vec"] == 1 and info["wide"] == 0
        # misaligned -> scalar form
        v = sg.sgemm_op_select_variant(ta, tb, 4096, 4096, 4096, FAKE_A + 4, 4096, FAKE_B, 4096, FAKE_C, 4096)
        assert sg.sgemm_variant_info(v)["vec"] == 0
        # a panel span of 4 GiB or more (even a BK-row panel: 31 * 4e7 * 4 B) -> 64-bit offsets
        v = sg.sgemm_op_select_variant(ta, tb, 200, 200, 200, 0x100000000, 40_000_000, FAKE_B, 40_000_000,
                                       FAKE_C, 200)
        assert sg.sgemm_variant_info(v)["wide"] == 1
    nn = sg.sgemm_op_select_variant(b"N", b"N", 4096, 4096, 4096, FAKE_A, 4096, FAKE_B, 4096, FAKE_C, 4096)
    assert nn == sg.sgemm_select_variant(4096, 4096, 4096, FAKE_A, 4096, FAKE_B, 4096, FAKE_C, 4096)
    assert sg.sgemm_op_select_variant(b"Q", b"N", 4, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4) == -1


def test_binding_error_names_the_op_argument():
    with pytest.raises(sg.SgemmError, match=r"argument 8 \(lda\)"):
        sg.sgemm_op("T", "N", 8, 4, 4, 1.0, FAKE_A, 7, FAKE_B, 4, 0.0, FAKE_C, 4, stream=0)
    with pytest.raises(sg.SgemmError, match=r"argument 1 \(transa\)"):
        sg.sgemm_op("X", "N", 8, 4, 4, 1.0, FAKE_A, 8, FAKE_B, 4, 0.0, FAKE_C, 4, stream=0)


def test_binding_error_classes():
    """Negative codes raise SgemmArgumentError (also a ValueError), positive ones SgemmLaunchError;
    both are SgemmError."""
    with pytest.raises(ValueError) as e:
        sg.sgemm(-1, 4, 4, 1.0, FAKE_A, 4, FAKE_B, 4, 0.0, FAKE_C, 4, stream=0)
    assert isinstance(e.value, sg.SgemmArgumentError) and isinstance(e.value, sg.SgemmError)
    assert e.value.code == -1
    err = _binding._error(1, "sgemm")
    assert isinstance(err, sg.SgemmLaunchError) and not isinstance(err, ValueError)
    assert "hipError_t 1" in str(err)
