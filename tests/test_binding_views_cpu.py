"""The tensor wrapper's marshalling of column-major views, checked on the CPU: which stored array,
leading dimension and transposition flag reach the C ABI for each combination (the ABI calls are
recorded instead of run; the GPU test of the same combinations checks the results)."""
import itertools

import pytest

torch = pytest.importorskip("torch")

from fp32_gemm_05_amd import _binding as b  # noqa: E402


def test_column_major_detection():
    x = torch.zeros(3, 5)
    assert not b._column_major(x)
    assert b._column_major(x.t())
    assert not b._column_major(torch.zeros(1, 5).t())  # a single row or column is both
    assert not b._column_major(torch.zeros(4, 6)[:, ::2])  # strided columns: neither layout


@pytest.fixture
def calls(monkeypatch):
    rec = []
    monkeypatch.setattr(b, "_check_matrix",
                        lambda t, name: t.stride(0) if t.shape[0] > 1 else max(1, t.shape[1]))
    monkeypatch.setattr(b, "sgemm_ex", lambda *a: rec.append(("NN",) + a))
    monkeypatch.setattr(b, "sgemm_op_ex", lambda *a: rec.append(a))
    return rec


M, N, K = 6, 5, 4


@pytest.mark.parametrize("a_view,b_view,c_view,ta,tb", list(itertools.product([False, True], repeat=5)))
def test_views_reach_the_abi_as_row_major_storage(calls, a_view, b_view, c_view, ta, tb):
    # the logical operands: op(A) is M x K and op(B) is K x N
    As = torch.zeros((K, M) if ta else (M, K))
    Bs = torch.zeros((N, K) if tb else (K, N))
    A = As.t().contiguous().t() if a_view else As  # same shape, column-major storage
    B = Bs.t().contiguous().t() if b_view else Bs
    C = torch.zeros(N, M).t() if c_view else torch.zeros(M, N)
    b.gemm(A, B, C, alpha=2.0, beta=0.5, trans_a=ta, trans_b=tb)
    assert len(calls) == 1
    call = calls[0]
    if call[0] == "NN":
        _, m, n, k, alpha, pa, lda, pb, ldb, beta, pc, ldc, stream, variant = call
        tra = trb = False
    else:
        tra, trb, m, n, k, alpha, pa, lda, pb, ldb, beta, pc, ldc, stream, variant = call
    for t in (pa, pb, pc):
        assert t.stride(1) == 1  # every array reaches the ABI row-major
    if c_view:
        # C^T (N x M) = op(B)^T op(A)^T on C's storage
        assert (m, n, k) == (N, M, K) and pc.data_ptr() == C.data_ptr()
    else:
        assert (m, n, k) == (M, N, K) and pc is C
    assert (alpha, beta, variant) == (2.0, 0.5, -1)
    # the stored first operand's shape matches its flag: rows x cols = (k x m) if transposed else (m x k)
    assert tuple(pa.shape) == ((k, m) if tra else (m, k))
    assert tuple(pb.shape) == ((n, k) if trb else (k, n))
    assert lda == pa.shape[1] and ldb == pb.shape[1] and ldc == pc.shape[1]


def test_forced_variant_needs_row_major_c(calls):
    with pytest.raises(ValueError):
        b.gemm(torch.zeros(M, K), torch.zeros(K, N), torch.zeros(N, M).t(), variant=3)


@pytest.fixture
def recorder(monkeypatch):
    """The real layout checks with the device check and the ABI calls replaced by a recorder."""
    rec = []
    monkeypatch.setattr(b, "_require_device", lambda t, name: None)
    monkeypatch.setattr(b, "sgemm_ex", lambda *a: rec.append(("NN",) + a))
    monkeypatch.setattr(b, "sgemm_op_ex", lambda *a: rec.append(a))
    return rec


def _broadcast_rows(rows, cols):
    return torch.ones(1, cols).expand(rows, cols)        # row stride 0


def _broadcast_cols(rows, cols):
    return torch.ones(rows, 1).expand(rows, cols)        # column stride 0


def _unfolded(rows, cols):
    return torch.arange(rows + cols, dtype=torch.float32).unfold(0, cols, 1)[:rows]  # row stride 1


BAD_VIEWS = {"broadcast_rows": _broadcast_rows, "broadcast_cols": _broadcast_cols, "unfolded": _unfolded}


@pytest.mark.parametrize("which", ["A", "B", "C"])
@pytest.mark.parametrize("kind", list(BAD_VIEWS))
def test_shared_storage_views_are_refused(recorder, which, kind):
    """Views whose rows share storage (stride-0 broadcasts, overlapping unfolds) have no leading
    dimension: the wrapper refuses them and calls nothing, instead of raising ld to the row length
    (which made the library address past their storage)."""
    shapes = {"A": (M, K), "B": (K, N), "C": (M, N)}
    args = {k: torch.zeros(*v) for k, v in shapes.items()}
    args[which] = BAD_VIEWS[kind](*shapes[which])
    with pytest.raises(ValueError):
        b.gemm(args["A"], args["B"], args["C"])
    assert recorder == []


def test_real_leading_dimensions_reach_the_abi(recorder):
    """A padded view passes its real row stride, not the row length."""
    A = torch.zeros(M, K + 3)[:, :K]
    B = torch.zeros(K, N + 5)[:, :N]
    C = torch.zeros(M, N + 7)[:, :N]
    b.gemm(A, B, C)
    (_, m, n, k, _, _, lda, _, ldb, _, _, ldc, _, _), = recorder
    assert (m, n, k, lda, ldb, ldc) == (M, N, K, K + 3, N + 5, N + 7)


def test_single_row_and_empty_operands_keep_a_valid_ld(recorder):
    b.gemm(torch.zeros(1, K), torch.zeros(K, N), torch.zeros(1, N))
    b.gemm(torch.zeros(M, 0), torch.zeros(0, N), torch.zeros(M, N))
    (_, _, _, _, _, _, lda1, _, ldb1, _, _, ldc1, _, _), (_, _, _, k2, _, _, lda2, _, _, _, _, _, _, _) = recorder
    assert (lda1, ldb1, ldc1) == (K, N, N)
    assert k2 == 0 and lda2 == 1
