"""The tensor wrapper ``gemm`` on column-major views: operands given as transposed views (unit
row stride, e.g. ``x.t()``) and a column-major C are handled without copies (storage passed with
the transposition flipped; a column-major C computed as C^T = op(B)^T op(A)^T on its storage).
Integer-valued data: every output equals the oracle's exactly, and C's storage holds nothing else.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import fp32_gemm_05_amd as sg  # noqa: E402

# an unaligned shape (scalar variants only) and an aligned one (the swapped column-major C then
# dispatches 128-bit variants too)
SHAPES = [(131, 70, 53), (256, 128, 64)]
CASES = list(itertools.product([False, True], repeat=5))  # A view, B view, C view, trans_a, trans_b


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _logical_to_tensor(x: np.ndarray, stored_transposed: bool, view: bool):
    """A device tensor whose value as passed is `x` (stored_transposed: the caller passes x^T and
    asks for op = T); with `view`, that tensor is a column-major view of contiguous storage."""
    arr = x.T if stored_transposed else x
    if view:
        return torch.from_numpy(np.ascontiguousarray(arr.T)).cuda().t()  # same values, column-major
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


@pytest.mark.parametrize("M,N,K", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
@pytest.mark.parametrize("a_view,b_view,c_view,ta,tb", CASES,
                         ids=[f"A{'v' if a else 'r'}{'T' if ta else 'N'}_B{'v' if b else 'r'}{'T' if tb else 'N'}"
                              f"_C{'v' if c else 'r'}" for a, b, c, ta, tb in CASES])
def test_gemm_views(a_view, b_view, c_view, ta, tb, M, N, K):
    rng = np.random.default_rng(17 + 2 * a_view + 4 * b_view + 8 * c_view + 16 * ta + 32 * tb + M)
    A = rng.integers(-2, 3, (M, K)).astype(np.float32)
    B = rng.integers(-2, 3, (K, N)).astype(np.float32)
    C0 = rng.integers(-2, 3, (M, N)).astype(np.float32)
    dA = _logical_to_tensor(A, ta, a_view)
    dB = _logical_to_tensor(B, tb, b_view)
    dC = _logical_to_tensor(C0, False, c_view)
    assert (dA.stride(0) == 1) == a_view and (dC.stride(0) == 1) == c_view
    sg.gemm(dA, dB, dC, alpha=0.5, beta=-1.5, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    ref, _ = oracle.ref_rows(A, B, C0, 0.5, -1.5)
    got = dC.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref), f"max |diff| {np.abs(got - ref).max()}"


# A column-major C whose swap turns a wide, short C into a tall C^T: 20000 x 24 (the narrow class,
# N <= 32) or 20000 x 64 (the skinny class).  The swapped call is op(B)^T op(A)^T, so with B passed
# transposed it reads the stored B as plain A' and runs the nontemporal stream kernels (N N or N T);
# without, the transposed 64x64 variants (T T, T N).
STREAM_SWAPS = [(24, 20000, 64), (64, 20000, 96)]


@pytest.mark.parametrize("M,N,K", STREAM_SWAPS, ids=[f"C{m}x{n}_K{k}" for m, n, k in STREAM_SWAPS])
@pytest.mark.parametrize("ta,tb", list(itertools.product([False, True], repeat=2)))
def test_column_major_c_swaps_into_stream_classes(M, N, K, ta, tb):
    rng = np.random.default_rng(M + N + K + 2 * ta + tb)
    A = rng.integers(-2, 3, (M, K)).astype(np.float32)
    B = rng.integers(-2, 3, (K, N)).astype(np.float32)
    C0 = rng.integers(-2, 3, (M, N)).astype(np.float32)
    dA = _logical_to_tensor(A, ta, False)
    dB = _logical_to_tensor(B, tb, False)
    dC = _logical_to_tensor(C0, False, True)
    sg.gemm(dA, dB, dC, alpha=0.5, beta=-1.5, trans_a=ta, trans_b=tb)
    vid = sg.sgemm_last_variant()
    name = sg.sgemm_variant_name(vid)
    print(f"[views] column-major C {M}x{N}, K={K}, op {ta:d}{tb:d}: swapped call ran {name}", flush=True)
    # the swapped call: A' = the stored B with op flipped, B' = the stored A with op flipped
    want = sg.sgemm_op_select_variant(not tb, not ta, N, M, K, dB, dB.shape[1], dA, dA.shape[1],
                                      dC, M)
    assert vid == want
    if tb:  # A' = B read as stored: a streamed workgroup shape over C^T's long side
        info = sg.sgemm_variant_info(vid)
        assert info["BN"] <= 64 and info["BM"] >= 128 and not info["trans_a"], name
    torch.cuda.synchronize()
    ref, _ = oracle.ref_rows(A, B, C0, 0.5, -1.5)
    got = dC.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref), f"max |diff| {np.abs(got - ref).max()}"
