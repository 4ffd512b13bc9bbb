"""Pins for the float64 oracle, checked against facts that do not come from the oracle.

Each pin is a function ``pin(ref_fn) -> None`` that raises AssertionError when
``ref_fn(A, B, C, alpha, beta) -> (ref, bound)`` is wrong.  The pins are run
against the real oracle (both forms: the C triple loop and the numpy-matmul
form), and against planted-mistake oracles written here in Python (a dropped
term, a wrong sign, a transposed operand, ...): every planted mistake must be
caught by at least one pin, which shows the pins can tell.

What pins the result (the definition of GEMM in "SGEMM CUDA kernel (First
Half)", introduction and "Part 1: CPU version"):
  * exact rational arithmetic (fractions.Fraction) on tiny random-float inputs;
  * an integer matrix product in int64 on integer-valued inputs;
  * closed forms: identity, permutation and rank-1 operands;
  * the transpose identity (B^T A^T) = (A B)^T;
  * the special cases beta == 0 (C not read), alpha == 0 / K == 0 (A, B not
    read) and padded leading dimensions (padding never read).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

pytestmark = []


# --------------------------------------------------------------------------------------
# oracle forms under test
# --------------------------------------------------------------------------------------

def _loop(A, B, C, alpha, beta):
    return oracle.ref_rows(A, B, C, alpha, beta)


def _matmul(A, B, C, alpha, beta):
    return oracle.ref_matmul(A, B, C, alpha, beta)


def _points_all(A, B, C, alpha, beta):
    M, N = C.shape
    I, J = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref, bound = oracle.ref_points(A, B, C, I.ravel(), J.ravel(), alpha, beta)
    return ref.reshape(M, N), bound.reshape(M, N)


ORACLE_FORMS = {"loop": _loop, "matmul": _matmul, "points": _points_all}


# --------------------------------------------------------------------------------------
# input helpers (local to the pins; the workloads module is checked separately)
# --------------------------------------------------------------------------------------

def _rand(rng, shape):
    return rng.uniform(-1.0, 1.0, shape).astype(np.float32)


def _ints(rng, shape, lo=-2, hi=3):
    return rng.integers(lo, hi, shape).astype(np.float32)


def _frac_ref(A, B, C, alpha, beta):
    """Exact rational value of alpha*A@B + beta*C and of sum |a*b| (Fraction)."""
    M, K = A.shape
    N = B.shape[1]
    fa, fb = Fraction(float(alpha)), Fraction(float(beta))
    out, sabs, cabs = [], [], []
    for i in range(M):
        row, rs, rc = [], [], []
        for j in range(N):
            s = Fraction(0)
            sa = Fraction(0)
            for k in range(K):
                p = Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
                s += p
                sa += abs(p)
            c = fb * Fraction(float(C[i, j])) if beta != 0 else Fraction(0)
            row.append(fa * s + c)
            rs.append(sa)
            rc.append(abs(c))
        out.append(row)
        sabs.append(rs)
        cabs.append(rc)
    return out, sabs, cabs


# --------------------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------------------

def pin_fraction(ref_fn):
    """Random floats, tiny shapes: ref within double rounding of the exact rational value,
    and bound equal to 1e-5*(|alpha|*sum|ab| + |beta*c|) + 1e-6 computed exactly."""
    rng = np.random.default_rng(11)
    cases = [(1, 1, 1, 1.0, 0.0), (2, 3, 4, 1.0, 0.5), (3, 2, 5, -0.75, 1.25),
             (4, 4, 6, 2.0, -1.5), (5, 3, 2, 0.5, 0.0), (1, 6, 3, 1.0, 1.0)]
    for (M, N, K, alpha, beta) in cases:
        A, B, C = _rand(rng, (M, K)), _rand(rng, (K, N)), _rand(rng, (M, N))
        ref, bound = ref_fn(A, B, C, alpha, beta)
        exact, sabs, cabs = _frac_ref(A, B, C, alpha, beta)
        for i in range(M):
            for j in range(N):
                scale = abs(alpha) * float(sabs[i][j]) + float(cabs[i][j])
                err = abs(Fraction(float(ref[i, j])) - exact[i][j])
                assert float(err) <= (K + 3) * 2.0 ** -52 * scale + 1e-300, (M, N, K, i, j)
                want_bound = 1e-5 * (abs(alpha) * float(sabs[i][j]) + float(cabs[i][j])) + 1e-6
                assert abs(bound[i, j] - want_bound) <= 1e-12 * want_bound, (M, N, K, i, j)


def pin_int64(ref_fn):
    """Integer-valued inputs: ref equals the int64 matrix product exactly (alpha, beta dyadic)."""
    rng = np.random.default_rng(12)
    for (M, N, K, alpha, beta) in [(7, 9, 11, 1.0, 0.0), (16, 5, 13, 0.5, -1.5), (3, 17, 20, -2.0, 1.0),
                                   (8, 8, 8, 1.0, 0.0)]:
        A, B, C = _ints(rng, (M, K)), _ints(rng, (K, N)), _ints(rng, (M, N))
        ref, _ = ref_fn(A, B, C, alpha, beta)
        prod = A.astype(np.int64) @ B.astype(np.int64)
        want = alpha * prod.astype(np.float64) + (beta * C.astype(np.float64) if beta != 0 else 0.0)
        assert np.array_equal(ref, want), (M, N, K)


def pin_identity(ref_fn):
    """A = I gives alpha*B + beta*C; B = I gives alpha*A + beta*C (exact)."""
    rng = np.random.default_rng(13)
    n, N = 9, 7
    B, C = _rand(rng, (n, N)), _rand(rng, (n, N))
    ref, _ = ref_fn(np.eye(n, dtype=np.float32), B, C, 0.5, 2.0)
    assert np.array_equal(ref, 0.5 * B.astype(np.float64) + 2.0 * C.astype(np.float64))
    M = 6
    A, C2 = _rand(rng, (M, n)), _rand(rng, (M, n))
    ref, _ = ref_fn(A, np.eye(n, dtype=np.float32), C2, 1.0, -1.0)
    assert np.array_equal(ref, A.astype(np.float64) - C2.astype(np.float64))


def pin_permutation(ref_fn):
    """A = a permutation matrix P gives the rows of B permuted (exact)."""
    rng = np.random.default_rng(14)
    n, N = 8, 5
    perm = rng.permutation(n)
    P = np.zeros((n, n), dtype=np.float32)
    P[np.arange(n), perm] = 1.0
    B = _rand(rng, (n, N))
    ref, _ = ref_fn(P, B, np.zeros((n, N), np.float32), 1.0, 0.0)
    assert np.array_equal(ref, B[perm].astype(np.float64))


def pin_rank1(ref_fn):
    """A[i][k] = u_i, B[k][j] = v_j gives K*u_i*v_j (exact for integers and for K a power of two)."""
    rng = np.random.default_rng(15)
    for (M, N, K, ints) in [(5, 4, 7, True), (3, 6, 16, False)]:
        u = _ints(rng, (M,), -9, 10) if ints else _rand(rng, (M,))
        v = _ints(rng, (N,), -9, 10) if ints else _rand(rng, (N,))
        A = np.repeat(u[:, None], K, axis=1)
        B = np.repeat(v[None, :], K, axis=0)
        ref, _ = ref_fn(A, B, np.zeros((M, N), np.float32), 1.0, 0.0)
        want = K * np.outer(u.astype(np.float64), v.astype(np.float64))
        assert np.array_equal(ref, want), (M, N, K, ints)


def pin_transpose(ref_fn):
    """(B^T A^T) = (A B)^T: the oracle applied to the transposed problem is the transpose."""
    rng = np.random.default_rng(16)
    M, N, K = 6, 5, 9
    A, B, C = _ints(rng, (M, K)), _ints(rng, (K, N)), _ints(rng, (M, N))
    r1, _ = ref_fn(A, B, C, 1.0, 0.5)
    r2, _ = ref_fn(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), np.ascontiguousarray(C.T), 1.0, 0.5)
    assert np.array_equal(r1, r2.T)
    # a non-symmetric-in-roles float case: products must pair A's row with B's column
    A, B = _rand(rng, (M, K)), _rand(rng, (K, N))
    r1, _ = ref_fn(A, B, np.zeros((M, N), np.float32), 1.0, 0.0)
    r2, _ = ref_fn(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), np.zeros((N, M), np.float32), 1.0, 0.0)
    np.testing.assert_allclose(r1, r2.T, rtol=1e-14, atol=1e-15)


def pin_beta_zero(ref_fn):
    """beta == 0: C is not read, NaN/Inf in C do not reach the result."""
    rng = np.random.default_rng(17)
    A, B = _ints(rng, (4, 6)), _ints(rng, (6, 3))
    Cnan = np.full((4, 3), np.nan, dtype=np.float32)
    Cnan[0, 0] = np.inf
    ref, bound = ref_fn(A, B, Cnan, 1.0, 0.0)
    assert np.all(np.isfinite(ref)) and np.all(np.isfinite(bound))
    assert np.array_equal(ref, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64))


def pin_alpha_zero(ref_fn):
    """alpha == 0: A and B are not read; the result is beta*C exactly."""
    rng = np.random.default_rng(18)
    A = np.full((4, 5), np.nan, dtype=np.float32)
    B = np.full((5, 3), np.inf, dtype=np.float32)
    C = _rand(rng, (4, 3))
    ref, bound = ref_fn(A, B, C, 0.0, -1.5)
    assert np.array_equal(ref, -1.5 * C.astype(np.float64))
    assert np.allclose(bound, 1e-5 * np.abs(1.5 * C.astype(np.float64)) + 1e-6, rtol=1e-12)


def pin_k_zero(ref_fn):
    """K == 0: the sum is empty; the result is beta*C."""
    rng = np.random.default_rng(19)
    C = _rand(rng, (3, 4))
    ref, _ = ref_fn(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32), C, 2.0, 0.5)
    assert np.array_equal(ref, 0.5 * C.astype(np.float64))


def pin_padding(ref_fn):
    """Padded leading dimensions: NaN in the padding never leaks into the result."""
    from fp32_gemm_05_amd.workloads import padded
    rng = np.random.default_rng(20)
    M, N, K = 5, 7, 6
    A, B, C = _ints(rng, (M, K)), _ints(rng, (K, N)), _ints(rng, (M, N))
    r_packed, _ = ref_fn(A, B, C, 1.0, -1.0)
    r_pad, _ = ref_fn(padded(A, 3), padded(B, 5), padded(C, 1), 1.0, -1.0)
    assert np.all(np.isfinite(r_pad))
    assert np.array_equal(r_packed, r_pad)


PINS = [pin_fraction, pin_int64, pin_identity, pin_permutation, pin_rank1, pin_transpose,
        pin_beta_zero, pin_alpha_zero, pin_k_zero, pin_padding]


@pytest.mark.parametrize("form", sorted(ORACLE_FORMS))
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pinned(form, pin):
    pin(ORACLE_FORMS[form])


# --------------------------------------------------------------------------------------
# planted mistakes: every one must be caught by some pin
# --------------------------------------------------------------------------------------

def _py_oracle(mistake):
    """A slow Python oracle with one planted mistake (None = no mistake)."""
    def ref_fn(A, B, C, alpha, beta):
        A = np.asarray(A)
        B = np.asarray(B)
        C = np.asarray(C)
        M, K = A.shape
        N = B.shape[1]
        ref = np.zeros((M, N))
        bound = np.zeros((M, N))
        for i in range(M):
            for j in range(N):
                s = np.float32(0) if mistake == "f32_accumulate" else 0.0
                sa = 0.0
                kk = K - 1 if mistake == "drop_last_term" else K
                if alpha != 0 or mistake == "reads_ab_when_alpha0":
                    for k in range(kk):
                        if mistake == "transposed_b" and M == K == N:
                            b = B[j, k]
                        else:
                            b = B[k, j]
                        a = A[(i + 1) % M, k] if mistake == "row_off_by_one" else A[i, k]
                        if mistake == "f32_accumulate":
                            s = np.float32(s + np.float32(a) * np.float32(b))
                        else:
                            s += float(a) * float(b)
                        sa += abs(float(a) * float(b))
                if mistake == "reads_c_when_beta0" or beta != 0:
                    c = (-beta if mistake == "beta_sign" else beta) * float(C[i, j])
                else:
                    c = 0.0
                if mistake == "alpha_scales_c":
                    ref[i, j] = alpha * (float(s) + c)
                else:
                    ref[i, j] = alpha * float(s) + c
                cterm = 0.0 if mistake == "bound_drops_c" else abs(c)
                bound[i, j] = 1e-5 * (abs(alpha) * sa + cterm) + 1e-6
        return ref, bound
    return ref_fn


MISTAKES = ["drop_last_term", "transposed_b", "row_off_by_one", "f32_accumulate", "beta_sign",
            "alpha_scales_c", "reads_c_when_beta0", "reads_ab_when_alpha0", "bound_drops_c"]


def _caught(ref_fn):
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ref_fn)
        except AssertionError:
            return pin.__name__
    return None


def test_python_oracle_without_mistake_passes_all_pins():
    assert _caught(_py_oracle(None)) is None


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_mistake_is_caught(mistake):
    assert _caught(_py_oracle(mistake)) is not None, f"no pin catches {mistake}"


# --------------------------------------------------------------------------------------
# consistency of the oracle's entry points at moderate size
# --------------------------------------------------------------------------------------

def test_rows_points_matmul_agree():
    from fp32_gemm_05_amd.workloads import WORKLOADS, make_inputs, sample_points
    w = WORKLOADS["ragged3001x5003x777"]
    A, B, C = make_inputs(w, M=131, N=97, K=77)
    ref_l, b_l = oracle.ref_rows(A, B, C, w.alpha, w.beta)
    ref_m, b_m = oracle.ref_matmul(A, B, C, w.alpha, w.beta)
    np.testing.assert_allclose(ref_l, ref_m, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b_l, b_m, rtol=1e-12)
    part, _ = oracle.ref_rows(A, B, C, w.alpha, w.beta, rows=(40, 77))
    assert np.array_equal(part, ref_l[40:77])
    I, J = sample_points(131, 97, 50, seed=3, tile=32)
    ref_p, b_p = oracle.ref_points(A, B, C, I, J, w.alpha, w.beta)
    assert np.array_equal(ref_p, ref_l[I, J]) and np.array_equal(b_p, b_l[I, J])


def test_thread_count_does_not_change_result():
    from fp32_gemm_05_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS["square1024_beta"]
    A, B, C = make_inputs(w, M=64, N=48, K=200)
    r1, _ = oracle.ref_rows(A, B, C, w.alpha, w.beta, nthreads=1)
    r4, _ = oracle.ref_rows(A, B, C, w.alpha, w.beta, nthreads=4)
    assert np.array_equal(r1, r4)


def test_integer_workload_exact_at_256():
    """Integer-valued 256^3 inputs: the loop oracle equals the int64 product exactly."""
    from fp32_gemm_05_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS["square256"].as_int()
    A, B, C = make_inputs(w)
    ref, _ = oracle.ref_rows(A, B, C, w.alpha, w.beta)
    assert np.array_equal(ref, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64))


def test_bad_arguments_rejected():
    A = np.zeros((3, 4), np.float32)
    B = np.zeros((4, 5), np.float32)
    C = np.zeros((3, 5), np.float32)
    with pytest.raises(ValueError):
        oracle.ref_rows(A, B, C, 1.0, 0.0, rows=(2, 5))
    with pytest.raises(ValueError):
        oracle.ref_points(A, B, C, [3], [0], 1.0, 0.0)
    with pytest.raises(ValueError):
        oracle.ref_rows(A, np.zeros((5, 5), np.float32), C, 1.0, 0.0)


@pytest.mark.slow
@pytest.mark.parametrize("wname", ["square1024_beta", "ragged3001x5003x777", "skinny65536x64x1024"])
def test_integer_workloads_exact_full(wname):
    """Integer-valued inputs at the workloads' own sizes: the loop oracle equals an independent exact
    path (float64 BLAS product of integer matrices: every partial sum is an integer far below 2^53,
    so it is exact, as are alpha*s and beta*c for the dyadic alpha, beta)."""
    from fp32_gemm_05_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS[wname].as_int()
    A, B, C = make_inputs(w)
    ref, _ = oracle.ref_rows(A, B, C, w.alpha, w.beta)
    exact = w.alpha * (A.astype(np.float64) @ B.astype(np.float64))
    if w.beta != 0:
        exact += w.beta * C.astype(np.float64)
    assert np.array_equal(ref, exact)


@pytest.mark.slow
@pytest.mark.parametrize("wname", ["square4096", "square8192"])
def test_integer_workloads_exact_sampled(wname):
    """The large integer workloads, on sampled outputs: the loop oracle's points equal int64 dot
    products of the sampled rows and columns."""
    from fp32_gemm_05_amd.workloads import WORKLOADS, make_inputs, sample_points
    w = WORKLOADS[wname].as_int()
    A, B, C = make_inputs(w)
    I, J = sample_points(w.M, w.N, n_random=512, seed=w.seed, tile=128)
    ref, _ = oracle.ref_points(A, B, C, I, J, w.alpha, w.beta)
    Ai = A.astype(np.int64)
    Bi = B.astype(np.int64)
    exact = np.array([w.alpha * float(Ai[i] @ Bi[:, j]) for i, j in zip(I, J)])
    if w.beta != 0:
        exact += w.beta * C[I, J].astype(np.float64)
    assert np.array_equal(ref, exact)
