"""GPU parity of libsgemm against the float64 oracle, through the C ABI.

Bar (the operation C = alpha*A*B + beta*C of "SGEMM CUDA kernel (First Half)"):
  * random floats: |C_gpu - ref| <= 1e-5*(|alpha|*sum_k|a_ik*b_kj| + |beta*c_ij|) + 1e-6
    for every compared element, and every output finite;
  * integer-valued inputs (entries in -2..2, all partial sums exact in fp32):
    C_gpu equals the oracle exactly.
Small, reduced and full sizes are all compared element by element: the
full-size workloads run in the launch configuration the bench times (default
dispatch) and every output is checked against the oracle's full-matrix form.
The extreme extents (C beyond 4 GiB, a million-row column, K of a million) are
checked on every output too, in blocks of rows.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from fp32_gemm_05_amd.workloads import WORKLOADS, make_inputs
from tests.gemm_cases import SENTINEL, assert_border_untouched, check_exact, check_within_bound, device_matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import fp32_gemm_05_amd as sg  # noqa: E402


def _variants():
    """The variants sgemm / sgemm_ex serve (the transposed-operand ones are tested in test_gpu_trans)."""
    try:
        out = []
        for i in range(sg.sgemm_num_variants()):
            info = sg.sgemm_variant_info(i)
            if not info["trans_a"] and not info["trans_b"]:
                out.append((i, info["name"]))
        return out
    except OSError:
        return []


VARIANTS = _variants()
VARIANT_IDS = [v[1] for v in VARIANTS]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gemm(A, B, C, alpha, beta, variant=-1, pads=(0, 0, 0), offsets=(0, 0, 0), stream=None):
    """Run sgemm_ex on device copies of (A, B, C); returns (C_out as numpy, C buffer, C geometry)."""
    M, K = A.shape
    N = B.shape[1]
    bufA, vA, lda = device_matrix(A, pad_cols=pads[0], offset=offsets[0])
    bufB, vB, ldb = device_matrix(B, pad_cols=pads[1], offset=offsets[1])
    bufC, vC, ldc = device_matrix(C, pad_cols=pads[2], pad_rows=2, offset=offsets[2], fill=SENTINEL)
    sg.sgemm_ex(M, N, K, alpha, vA.data_ptr(), lda, vB.data_ptr(), ldb, beta, vC.data_ptr(), ldc,
                stream=stream, variant=variant)
    torch.cuda.synchronize()
    return vC.cpu().numpy(), bufC, (M, N, ldc, offsets[2])


def assert_c_border_untouched(bufC, geom):
    M, N, ldc, off = geom
    host = bufC.cpu().numpy()
    mask = np.ones(host.shape[0], dtype=bool)
    for r in range(M):
        mask[off + r * ldc: off + r * ldc + N] = False
    outside = host[mask]
    assert np.all(outside == SENTINEL), f"{np.count_nonzero(outside != SENTINEL)} writes outside C's M x N window"


def _applies(variant_id, vec_ok):
    info = sg.sgemm_variant_info(variant_id)
    return (not info["vec"]) or vec_ok


# ------------------------------------------------------------------------------------------
# every variant on small and reduced workloads, element by element
# ------------------------------------------------------------------------------------------

REDUCED = [
    # (label, workload, M, N, K)
    ("square256", "square256", 256, 256, 256),
    ("square1024_beta", "square1024_beta", 1024, 1024, 1024),
    ("ragged_reduced", "ragged3001x5003x777", 301, 503, 77),
    ("skinny_reduced", "skinny65536x64x1024", 4099, 64, 136),
    ("narrow_reduced", "skinny65536x64x1024", 4101, 28, 140),
    ("square_tail", "square4096", 389, 260, 300),
]


@pytest.mark.parametrize("vid", [v[0] for v in VARIANTS], ids=VARIANT_IDS)
@pytest.mark.parametrize("label,wname,M,N,K", REDUCED, ids=[r[0] for r in REDUCED])
def test_variant_reduced_float(vid, label, wname, M, N, K):
    w = WORKLOADS[wname]
    A, B, C = make_inputs(w, M=M, N=N, K=K)
    vec_ok = (K % 4 == 0) and (N % 4 == 0)
    _say(f"[parity] variant={sg.sgemm_variant_name(vid)} case={label} {M}x{N}x{K}")
    if not _applies(vid, vec_ok):
        with pytest.raises(sg.SgemmError) as e:
            run_gemm(A, B, C, w.alpha, w.beta, variant=vid)
        assert e.value.code == -13
        return
    got, bufC, geom = run_gemm(A, B, C, w.alpha, w.beta, variant=vid)
    ref, bound = oracle.ref_matmul(A, B, C, w.alpha, w.beta)
    check_within_bound(got, ref, bound, f"{label} {sg.sgemm_variant_name(vid)}")
    assert_c_border_untouched(bufC, geom)


@pytest.mark.parametrize("vid", [v[0] for v in VARIANTS], ids=VARIANT_IDS)
@pytest.mark.parametrize("label,wname,M,N,K", REDUCED, ids=[r[0] for r in REDUCED])
def test_variant_reduced_int_exact(vid, label, wname, M, N, K):
    w = WORKLOADS[wname].as_int()
    A, B, C = make_inputs(w, M=M, N=N, K=K)
    vec_ok = (K % 4 == 0) and (N % 4 == 0)
    if not _applies(vid, vec_ok):
        pytest.skip("vector variant does not apply to this shape")
    _say(f"[parity-int] variant={sg.sgemm_variant_name(vid)} case={label} {M}x{N}x{K}")
    got, bufC, geom = run_gemm(A, B, C, w.alpha, w.beta, variant=vid)
    ref, _ = oracle.ref_matmul(A, B, C, w.alpha, w.beta)
    check_exact(got, ref, f"{label}-int {sg.sgemm_variant_name(vid)}")
    assert_c_border_untouched(bufC, geom)


@pytest.mark.parametrize("vid", [v[0] for v in VARIANTS], ids=VARIANT_IDS)
def test_variant_padded_ld_nan_does_not_leak(vid):
    """Leading dimensions larger than the row length, padding filled with NaN."""
    w = WORKLOADS["square1024_beta"].as_int()
    M, N, K = 200, 136, 72
    A, B, C = make_inputs(w, M=M, N=N, K=K)
    _say(f"[padded] variant={sg.sgemm_variant_name(vid)}")
    got, bufC, geom = run_gemm(A, B, C, 1.0, -1.0, variant=vid, pads=(4, 8, 12))
    ref, _ = oracle.ref_matmul(A, B, C, 1.0, -1.0)
    check_exact(got, ref, f"padded {sg.sgemm_variant_name(vid)}")
    assert_c_border_untouched(bufC, geom)


@pytest.mark.parametrize("vid", [v[0] for v in VARIANTS], ids=VARIANT_IDS)
def test_variant_misaligned_pointers(vid):
    """Sub-matrix pointers one float off 16-byte alignment: vector variants refuse, scalar ones compute."""
    w = WORKLOADS["square1024_beta"]
    M, N, K = 130, 132, 68
    A, B, C = make_inputs(w, M=M, N=N, K=K)
    info = sg.sgemm_variant_info(vid)
    _say(f"[misaligned] variant={info['name']}")
    if info["vec"]:
        with pytest.raises(sg.SgemmError) as e:
            run_gemm(A, B, C, w.alpha, w.beta, variant=vid, offsets=(1, 1, 1))
        assert e.value.code == -13
        return
    got, bufC, geom = run_gemm(A, B, C, w.alpha, w.beta, variant=vid, offsets=(1, 3, 1))
    ref, bound = oracle.ref_matmul(A, B, C, w.alpha, w.beta)
    check_within_bound(got, ref, bound, f"misaligned {info['name']}")
    assert_c_border_untouched(bufC, geom)


# ------------------------------------------------------------------------------------------
# edge sweeps: integer data, bit-exact, default dispatch and every variant on a subset
# ------------------------------------------------------------------------------------------

EDGE_DIMS = [1, 2, 3, 4, 5, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257]


def _edge_shapes():
    rng = np.random.default_rng(7)
    shapes = [(1, 1, 1), (1, 257, 3), (257, 1, 5), (3, 5, 1), (65, 63, 129), (129, 255, 64),
              (256, 256, 8), (257, 129, 17), (64, 64, 4096)]
    for _ in range(24):
        shapes.append(tuple(int(rng.choice(EDGE_DIMS)) for _ in range(3)))
    return shapes


EDGE_SHAPES = _edge_shapes()


@pytest.mark.parametrize("M,N,K", EDGE_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in EDGE_SHAPES])
def test_edge_sweep_default_dispatch(M, N, K):
    w = WORKLOADS["ragged3001x5003x777"].as_int()
    A, B, C = make_inputs(w, M=M, N=N, K=K, seed=3000 + M + 7 * N + 13 * K)
    _say(f"[edge] {M}x{N}x{K}")
    got, bufC, geom = run_gemm(A, B, C, 0.5, -1.5)
    ref, _ = oracle.ref_rows(A, B, C, 0.5, -1.5)
    check_exact(got, ref, f"edge {M}x{N}x{K}")
    assert_c_border_untouched(bufC, geom)


EDGE_SUBSET = [(1, 1, 1), (33, 65, 7), (129, 127, 33), (257, 63, 129), (63, 257, 65), (200, 300, 4)]


@pytest.mark.parametrize("vid", [v[0] for v in VARIANTS], ids=VARIANT_IDS)
def test_edge_sweep_every_variant(vid):
    info = sg.sgemm_variant_info(vid)
    w = WORKLOADS["ragged3001x5003x777"].as_int()
    for (M, N, K) in EDGE_SUBSET:
        A, B, C = make_inputs(w, M=M, N=N, K=K, seed=4000 + M + N + K)
        if info["vec"] and (K % 4 or N % 4):
            continue
        _say(f"[edge-variant] {info['name']} {M}x{N}x{K}")
        got, bufC, geom = run_gemm(A, B, C, 1.0, 0.5, variant=vid)
        ref, _ = oracle.ref_rows(A, B, C, 1.0, 0.5)
        check_exact(got, ref, f"edge {info['name']} {M}x{N}x{K}")
        assert_c_border_untouched(bufC, geom)


# ------------------------------------------------------------------------------------------
# special cases of the definition
# ------------------------------------------------------------------------------------------

def test_beta_zero_does_not_read_c():
    w = WORKLOADS["square256"]
    A, B, _ = make_inputs(w, M=96, N=80, K=40)
    C = np.full((96, 80), np.nan, dtype=np.float32)
    got, _, _ = run_gemm(A, B, C, 1.0, 0.0)
    ref, bound = oracle.ref_rows(A, B, C, 1.0, 0.0)
    check_within_bound(got, ref, bound, "beta=0 with NaN C")


def test_alpha_zero_does_not_read_ab():
    rng = np.random.default_rng(5)
    A = np.full((70, 30), np.nan, dtype=np.float32)
    B = np.full((30, 50), np.inf, dtype=np.float32)
    C = rng.uniform(-1, 1, (70, 50)).astype(np.float32)
    got, bufC, geom = run_gemm(A, B, C, 0.0, -1.5)
    ref, _ = oracle.ref_rows(A, B, C, 0.0, -1.5)
    # one fp32 multiply per element: the result is the correctly rounded beta*c
    check_exact(got, ref.astype(np.float32).astype(np.float64), "alpha=0")
    assert_c_border_untouched(bufC, geom)
    got, _, _ = run_gemm(A, B, C, 0.0, 0.0)
    assert np.all(got == 0.0)
    got, _, _ = run_gemm(A, B, C, 0.0, 1.0)
    assert np.array_equal(got, C)


def test_k_zero_scales_c():
    rng = np.random.default_rng(6)
    C = rng.uniform(-1, 1, (33, 17)).astype(np.float32)
    A = np.zeros((33, 0), np.float32)
    B = np.zeros((0, 17), np.float32)
    got, _, _ = run_gemm(A, B, C, 2.0, 0.5)
    ref, _ = oracle.ref_rows(A, B, C, 2.0, 0.5)
    check_exact(got, ref, "K=0")


def test_empty_outputs_are_noops():
    dC = torch.full((4, 4), 7.0, device="cuda")
    sg.sgemm(0, 4, 4, 1.0, None, 4, None, 4, 0.0, dC.data_ptr(), 4)
    sg.sgemm(4, 0, 4, 1.0, None, 4, None, 1, 0.0, dC.data_ptr(), 1)
    torch.cuda.synchronize()
    assert torch.all(dC == 7.0)


def test_error_codes_no_launch():
    dC = torch.zeros((8, 8), device="cuda")
    for args, code in [((-1, 8, 8), -1), ((8, -1, 8), -2), ((8, 8, -1), -3)]:
        with pytest.raises(sg.SgemmError) as e:
            sg.sgemm(*args, 1.0, dC.data_ptr(), 8, dC.data_ptr(), 8, 0.0, dC.data_ptr(), 8)
        assert e.value.code == code
    dA = torch.zeros((8, 8), device="cuda")
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm(8, 8, 8, 1.0, dA.data_ptr(), 7, dA.data_ptr(), 8, 0.0, dC.data_ptr(), 8)
    assert e.value.code == -6
    with pytest.raises(sg.SgemmError) as e:  # C aliases A
        sg.sgemm(8, 8, 8, 1.0, dA.data_ptr(), 8, dA.data_ptr(), 8, 0.0, dA.data_ptr(), 8)
    assert e.value.code == -10
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_ex(8, 8, 8, 1.0, dA.data_ptr(), 8, dA.data_ptr(), 8, 0.0, dC.data_ptr(), 8,
                    variant=sg.sgemm_num_variants())
    assert e.value.code == -13


@pytest.mark.parametrize("M,lda,wide", [(40, 40_000_000, 1), (150, 20_000_000, 0)])
def test_huge_leading_dimension_wide_variant(M, lda, wide):
    """A strided A of 6.4 or 12 GB.  lda = 40,000,000: even a 32-row workgroup panel spans more
    than 4 GiB, so the dispatcher must use 64-bit offsets.  lda = 20,000,000: a 32-row panel spans
    2.5 GB and the dispatched narrow variant's 32-bit offsets still reach every row.  Either way
    the result must match the oracle exactly."""
    w = WORKLOADS["square1024_beta"].as_int()
    N, K = 64, 68
    A, B, C = make_inputs(w, M=M, N=N, K=K)
    bufA = torch.empty(M * lda, dtype=torch.float32, device="cuda")
    vA = bufA.as_strided((M, K), (lda, 1))
    vA.copy_(torch.from_numpy(A))
    dB = torch.from_numpy(B).cuda()
    dC = torch.from_numpy(C).cuda()
    vid = sg.sgemm_select_variant(M, N, K, vA, lda, dB, N, dC, N)
    _say(f"[huge-ld] M={M} lda={lda} variant={sg.sgemm_variant_name(vid)}")
    assert sg.sgemm_variant_info(vid)["wide"] == wide
    sg.sgemm(M, N, K, 1.0, vA, lda, dB, N, 0.5, dC, N)
    torch.cuda.synchronize()
    ref, _ = oracle.ref_rows(A, B, C, 1.0, 0.5)
    check_exact(dC.cpu().numpy(), ref, "huge lda")
    del bufA, vA
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------------------------
# self-consistency: scaling, determinism, streams, transpose identity
# ------------------------------------------------------------------------------------------

def test_alpha_two_is_exactly_double():
    w = WORKLOADS["square4096"]
    A, B, C = make_inputs(w, M=512, N=384, K=640)
    g1, _, _ = run_gemm(A, B, C, 1.0, 0.0)
    g2, _, _ = run_gemm(A, B, C, 2.0, 0.0)
    assert np.array_equal(g2, 2.0 * g1)


def test_repeated_runs_bitwise_identical():
    w = WORKLOADS["ragged3001x5003x777"]
    A, B, C = make_inputs(w, M=700, N=900, K=333)
    first, _, _ = run_gemm(A, B, C, w.alpha, w.beta)
    for _ in range(3):
        again, _, _ = run_gemm(A, B, C, w.alpha, w.beta)
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


def test_non_default_stream_ordering():
    """Two dependent calls on a non-default stream run in order, without host synchronisation."""
    w = WORKLOADS["square1024_beta"]
    A, B, C = make_inputs(w, M=640, N=512, K=256)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dA = torch.from_numpy(A).cuda()
        dB = torch.from_numpy(B).cuda()
        dC = torch.from_numpy(C).cuda()
        sg.gemm(dA, dB, dC, alpha=w.alpha, beta=w.beta)   # enqueued on s (the current stream)
        snap = dC.clone()                                  # ordered after the first call
        sg.gemm(dA, dB, dC, alpha=1.0, beta=1.0)           # reads the first call's output
    s.synchronize()
    first = snap.cpu().numpy()
    ref1, bound1 = oracle.ref_matmul(A, B, C, w.alpha, w.beta)
    check_within_bound(first, ref1, bound1, "first call on stream")
    ref2, bound2 = oracle.ref_matmul(A, B, first, 1.0, 1.0)
    check_within_bound(dC.cpu().numpy(), ref2, bound2, "second call on stream")


def test_transpose_identity_int():
    w = WORKLOADS["ragged3001x5003x777"].as_int()
    A, B, C = make_inputs(w, M=301, N=203, K=97)
    g1, _, _ = run_gemm(A, B, C, 1.0, 0.5)
    g2, _, _ = run_gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), np.ascontiguousarray(C.T), 1.0, 0.5)
    assert np.array_equal(g1, g2.T)


# ------------------------------------------------------------------------------------------
# the full-size workloads, default dispatch (what the bench times), every element
# ------------------------------------------------------------------------------------------

FULL = list(WORKLOADS)


@pytest.mark.parametrize("wname", FULL)
@pytest.mark.parametrize("kind", ["float", "int"])
def test_full_size_elementwise(wname, kind):
    """Every workload at its full size in the default dispatch -- the variant and grid the bench
    times, drain-ordered last rounds included -- compared with the oracle on EVERY element of C
    (its full-matrix form, float64 products), integer data exactly.  C sits in a buffer with
    sentinel columns and rows around it, which must come back untouched."""
    w = WORKLOADS[wname] if kind == "float" else WORKLOADS[wname].as_int()
    _say(f"[full] {w.describe()}")
    A, B, C = make_inputs(w)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    bufC, vC, ldc = device_matrix(C, pad_cols=4, pad_rows=2, fill=SENTINEL)
    vid = sg.sgemm_select_variant(w.M, w.N, w.K, dA, w.K, dB, w.N, vC, ldc)
    # ldc = N + 4 keeps the alignment class of ldc = N, so this is the bench's variant
    assert vid == sg.sgemm_select_variant(w.M, w.N, w.K, dA, w.K, dB, w.N, vC, w.N)
    _say(f"[full] variant={sg.sgemm_variant_name(vid)}")
    sg.sgemm(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, vC, ldc)
    assert sg.sgemm_last_variant() == vid
    torch.cuda.synchronize()
    host = bufC.cpu().numpy()
    del dA, dB, bufC, vC
    torch.cuda.empty_cache()
    assert_border_untouched(host, w.M, w.N, ldc, what=f"full {w.name}")
    got = host[: w.M * ldc].reshape(w.M, ldc)[:, : w.N]
    ref, bound = oracle.ref_matmul(A, B, C, w.alpha, w.beta)
    if kind == "int":
        check_exact(got, ref, f"full {w.name}")
    else:
        worst = check_within_bound(got, ref, bound, f"full {w.name}")
        _say(f"[full] {w.name}: max err/bound over all {w.M * w.N} outputs = {worst:.3g}")


# ------------------------------------------------------------------------------------------
# sub-matrices through pointer offsets, and subnormal behaviour
# ------------------------------------------------------------------------------------------

def test_submatrix_call_equals_block_of_full_product():
    """A call on a block -- A's rows i0.., B's columns j0.., through pointer offsets with the full
    leading dimensions -- equals that block of the full product (integer data: exact)."""
    w = WORKLOADS["ragged3001x5003x777"].as_int()
    M, N, K = 300, 260, 96
    A, B, C = make_inputs(w, M=M, N=N, K=K)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    full = torch.from_numpy(C).cuda()
    sg.sgemm(M, N, K, w.alpha, dA, K, dB, N, w.beta, full, N)
    for (i0, i1, j0, j1) in [(0, 128, 0, 128), (37, 261, 5, 203), (129, 300, 131, 260), (299, 300, 0, 1)]:
        blk = torch.from_numpy(C).cuda()  # same starting C, block updated in place
        ptrA = dA.data_ptr() + i0 * K * 4
        ptrB = dB.data_ptr() + j0 * 4
        ptrC = blk.data_ptr() + (i0 * N + j0) * 4
        _say(f"[submatrix] rows {i0}:{i1} cols {j0}:{j1}")
        sg.sgemm(i1 - i0, j1 - j0, K, w.alpha, ptrA, K, ptrB, N, w.beta, ptrC, N)
        torch.cuda.synchronize()
        got = blk.cpu().numpy()
        ref = full.cpu().numpy()
        assert np.array_equal(got[i0:i1, j0:j1], ref[i0:i1, j0:j1])
        outside = np.ones((M, N), bool)
        outside[i0:i1, j0:j1] = False
        assert np.array_equal(got[outside], C[outside]), "a store outside the block"


def _subnormal_case(vid, a_val, b_val, K=8):
    M, N = 64, 64
    A = np.full((M, K), a_val, np.float32)
    B = np.full((K, N), b_val, np.float32)
    C = np.zeros((M, N), np.float32)
    got, _, _ = run_gemm(A, B, C, 1.0, 0.0, variant=vid)
    return got


@pytest.mark.parametrize("vid", [v[0] for v in VARIANTS
                                 if "_o4" not in v[1] and "_wide" not in v[1] and "mfma32k" not in v[1]],
                         ids=[v[1] for v in VARIANTS
                              if "_o4" not in v[1] and "_wide" not in v[1] and "mfma32k" not in v[1]])
def test_subnormal_behaviour_recorded(vid):
    """Records whether a variant keeps fp32 subnormals (the method does not fix this; either way
    is accepted): products 2^-70 * 2^-70 = 2^-140 (subnormal results), and subnormal inputs
    2^-130 * 2^10 = 2^-120 (normal results).  Each output must be the exact value or zero."""
    name = sg.sgemm_variant_name(vid)
    sub_out = _subnormal_case(vid, 2.0 ** -70, 2.0 ** -70)          # exact: 8 * 2^-140 = 2^-137
    sub_in = _subnormal_case(vid, 2.0 ** -130, 2.0 ** 10)           # exact: 8 * 2^-120 = 2^-117
    outs = {}
    for label, got, exact in [("subnormal results", sub_out, 2.0 ** -137), ("subnormal inputs", sub_in, 2.0 ** -117)]:
        vals = set(np.unique(got.astype(np.float64)).tolist())
        assert vals <= {exact, 0.0}, (name, label, vals)
        outs[label] = "kept" if vals == {exact} else ("flushed" if vals == {0.0} else "mixed")
    _say(f"[subnormal] {name}: results {outs['subnormal results']}, inputs {outs['subnormal inputs']}")


# ------------------------------------------------------------------------------------------
# large extents: C beyond 4 GiB (64-bit element offsets in the epilogue), very tall and very
# long operands, K = 1
# ------------------------------------------------------------------------------------------

LARGE = [
    # (label, M, N, K, dist, alpha, beta)
    ("c_over_4gib", 33000, 33003, 8, "int", 1.0, 0.0),
    ("tall_n1", 1_000_003, 1, 64, "int", 0.5, 0.0),
    ("long_k", 96, 80, 1_000_001, "int", 1.0, 0.0),
    ("k1_wide", 4099, 20000, 1, "uniform", 2.0, 0.0),
    ("narrow_stream", 262144, 32, 512, "uniform", 1.0, 0.0),
    ("narrow_unaligned", 100003, 29, 777, "int", 1.0, 0.0),
]


@pytest.mark.parametrize("label,M,N,K,dist,alpha,beta", LARGE, ids=[x[0] for x in LARGE])
def test_large_extents_elementwise(label, M, N, K, dist, alpha, beta):
    """Default dispatch on extreme shapes, every output against the oracle's full-matrix form,
    taken in blocks of rows (C beyond 4 GiB has 1.1 G outputs); integer data exactly."""
    rng = np.random.default_rng(len(label) * 1000 + K)
    if dist == "int":
        A = rng.integers(-2, 3, (M, K)).astype(np.float32)
        B = rng.integers(-2, 3, (K, N)).astype(np.float32)
    else:
        A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    assert beta == 0.0  # C is neither read by the library nor needed by the oracle
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    vid = sg.sgemm_select_variant(M, N, K, dA, K, dB, N, dC, N)
    _say(f"[large] {label} {M}x{N}x{K} variant={sg.sgemm_variant_name(vid)}")
    sg.sgemm(M, N, K, alpha, dA, K, dB, N, beta, dC, N)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    del dA, dB, dC
    torch.cuda.empty_cache()
    rows = max(1, (1 << 25) // max(N, 1))  # about 32 M outputs per block
    worst = 0.0
    for r0 in range(0, M, rows):
        r1 = min(M, r0 + rows)
        ref, bound = oracle.ref_matmul(A[r0:r1], B, None, alpha, beta)
        if dist == "int":
            check_exact(out[r0:r1], ref, f"{label} rows {r0}:{r1}")
        else:
            worst = max(worst, check_within_bound(out[r0:r1], ref, bound, f"{label} rows {r0}:{r1}"))
    _say(f"[large] {label}: all {M * N} outputs checked (max err/bound {worst:.3g})")


# ------------------------------------------------------------------------------------------
# 32-bit offsets at their limits: leading dimensions just under a kernel's limit run it, just
# over are refused (a forced variant) or fall back to the 64-bit-offset variant (the dispatcher);
# every run exact on integer data
# ------------------------------------------------------------------------------------------

FREE_G8 = "mfma32r_32x32x128_w32x32_g8_cp_vec"  # LDS-free: a 32-row A panel, a 128-deep B panel
OFFSET_LIMITS = [
    # (label, lda, ldb, forced variant or None, expected family or None for "refused");
    # M, N, K = 40, 36, 600 (the tiny class)
    ("free_lda_under", 33_000_000, 36, FREE_G8, "mfma32r_"),    # (31*lda + 128)*4 < 2^32
    ("free_lda_over", 35_000_000, 36, FREE_G8, None),
    ("free_ldb_under", 600, 8_000_000, FREE_G8, "mfma32r_"),    # (127*ldb + 32)*4 < 2^32
    ("free_ldb_over", 600, 8_500_000, FREE_G8, None),
    ("tiny_lda_under", 34_000_000, 36, None, "mfma16l_32x64"),  # 32x64x32 tiles: (31*lda + 32)*4 < 2^32
    ("tiny_lda_over", 35_000_000, 36, None, "_wide"),
]


@pytest.mark.parametrize("label,lda,ldb,forced,family", OFFSET_LIMITS, ids=[x[0] for x in OFFSET_LIMITS])
def test_offset_limits(label, lda, ldb, forced, family):
    M, N, K = 40, 36, 600
    rng = np.random.default_rng(lda + ldb)
    A = rng.integers(-2, 3, (M, K)).astype(np.float32)
    B = rng.integers(-2, 3, (K, N)).astype(np.float32)
    C = np.zeros((M, N), np.float32)
    bufA, vA, lda_ = device_matrix(A, pad_cols=lda - K)
    bufB, vB, ldb_ = device_matrix(B, pad_cols=ldb - N)
    bufC, vC, ldc = device_matrix(C, fill=SENTINEL)
    assert (lda_, ldb_) == (lda, ldb)
    if forced is None:
        vid = sg.sgemm_select_variant(M, N, K, vA.data_ptr(), lda, vB.data_ptr(), ldb, vC.data_ptr(), ldc)
    else:
        vid = next(i for i in range(sg.sgemm_num_variants()) if sg.sgemm_variant_name(i) == forced)
    name = sg.sgemm_variant_name(vid)
    _say(f"[offset limits] {label}: lda={lda} ldb={ldb} variant={name}")
    if family is None:
        with pytest.raises(sg.SgemmError) as e:
            sg.sgemm_ex(M, N, K, 1.0, vA.data_ptr(), lda, vB.data_ptr(), ldb, 0.0, vC.data_ptr(), ldc, variant=vid)
        assert e.value.code == -13
    else:
        assert family in name
        sg.sgemm_ex(M, N, K, 1.0, vA.data_ptr(), lda, vB.data_ptr(), ldb, 0.0, vC.data_ptr(), ldc, variant=vid)
        torch.cuda.synchronize()
        assert sg.sgemm_last_variant() == vid
        ref, _ = oracle.ref_rows(A, B, C, 1.0, 0.0)
        check_exact(vC.cpu().numpy(), ref, label)
    del bufA, bufB, bufC, vA, vB, vC
    torch.cuda.empty_cache()
