"""Pins of the CPU oracle to facts fixed by the mathematics and the pages.

None of these re-types the oracle's formulas: each compares it with an exact
construction, a closed form, a brute-force determinant, a library routine or
an error bound.  Together they catch a dropped term, a wrong sign or index,
a missing conjugate and a transposed operand in any of potrf, potrs, logdet.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle

EPS64 = np.finfo(np.float64).eps
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ helpers ----

def int_lower(n, rng, cplx=False, diag_max=4, off=3):
    """Lower-triangular matrix of small integers (Gaussian integers if cplx)
    with a positive integer diagonal."""
    L = np.tril(rng.integers(-off, off + 1, size=(n, n)), -1).astype(np.int64)
    if cplx:
        L = L + 1j * np.tril(rng.integers(-off, off + 1, size=(n, n)), -1)
    d = rng.integers(1, diag_max + 1, size=n)
    L = L + np.diag(d)
    return L


def exact_gram(L):
    """L L^H in exact integer arithmetic (Python ints), returned as a numpy array."""
    n = L.shape[0]
    if np.iscomplexobj(L):
        re = [[int(v.real) for v in row] for row in L]
        im = [[int(v.imag) for v in row] for row in L]
        A = np.zeros((n, n), dtype=np.complex128)
        for i in range(n):
            for j in range(n):
                sr = sum(re[i][k] * re[j][k] + im[i][k] * im[j][k] for k in range(n))
                si = sum(im[i][k] * re[j][k] - re[i][k] * im[j][k] for k in range(n))
                assert abs(sr) < 2**53 and abs(si) < 2**53
                A[i, j] = complex(sr, si)
        return A
    Li = [[int(v) for v in row] for row in L]
    A = np.zeros((n, n), dtype=np.float64)
    for i in range(n):
        for j in range(n):
            s = sum(Li[i][k] * Li[j][k] for k in range(n))
            assert abs(s) < 2**53
            A[i, j] = float(s)
    return A


def laplace_det(M):
    """Determinant by cofactor expansion along the first row, exact (Fraction)."""
    n = len(M)
    if n == 0:
        return Fraction(1)
    if n == 1:
        return M[0][0]
    total = Fraction(0)
    for c in range(n):
        if M[0][c] == 0:
            continue
        minor = [row[:c] + row[c + 1:] for row in M[1:]]
        term = M[0][c] * laplace_det(minor)
        total += term if c % 2 == 0 else -term
    return total


def _cmul(a, b):
    return (a[0] * b[0] - a[1] * b[1], a[0] * b[1] + a[1] * b[0])


def laplace_det_complex(M):
    """Cofactor expansion over exact Gaussian rationals: entries are (re, im)
    pairs of Fractions."""
    n = len(M)
    if n == 1:
        return M[0][0]
    tr, ti = Fraction(0), Fraction(0)
    for c in range(n):
        if M[0][c] == (0, 0):
            continue
        minor = [row[:c] + row[c + 1:] for row in M[1:]]
        pr, pi = _cmul(M[0][c], laplace_det_complex(minor))
        if c % 2:
            pr, pi = -pr, -pi
        tr, ti = tr + pr, ti + pi
    return tr, ti


def rigal_gaches(A, x, b):
    """Normwise backward error per column: ||b - A x||_inf / (||A||_inf ||x||_inf + ||b||_inf)."""
    A = np.asarray(A, dtype=np.result_type(A, np.float64))
    r = b - A @ x
    nA = np.abs(A).sum(axis=1).max()
    return np.abs(r).max(axis=0) / (nA * np.abs(x).max(axis=0) + np.abs(b).max(axis=0))


def random_spd(n, seed, cplx=False, delta=0.5):
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((n, n))
    if cplx:
        G = (G + 1j * rng.standard_normal((n, n))) / math.sqrt(2)
    A = G @ G.conj().T / n + delta * np.eye(n)
    A = np.tril(A, -1) + np.tril(A, -1).conj().T + np.diag(np.diag(A).real)
    return A


# --------------------------------------------------------------- potrf ---

@pytest.mark.parametrize("n,seed", [(1, 0), (2, 1), (8, 2), (17, 3), (40, 4)])
@pytest.mark.parametrize("cplx", [False, True])
def test_potrf_recovers_integer_factor_exactly(n, seed, cplx):
    """A = L L^H built exactly from an integer L: every sqrt is of a perfect
    square and every division is exact, so the oracle must return L bit for bit."""
    rng = np.random.default_rng(seed)
    L = int_lower(n, rng, cplx)
    A = exact_gram(L)
    Lo, info = oracle.potrf(A)
    assert info == 0
    np.testing.assert_array_equal(Lo, L.astype(Lo.dtype))


@pytest.mark.parametrize("cplx", [False, True])
def test_potrf_reads_lower_triangle_only(cplx):
    rng = np.random.default_rng(7)
    L = int_lower(12, rng, cplx)
    A = exact_gram(L)
    poisoned = A.copy()
    poisoned[np.triu_indices(12, 1)] = np.nan
    if cplx:  # only the real part of the diagonal may be read
        poisoned[np.diag_indices(12)] += 123j
    Lo, info = oracle.potrf(poisoned)
    assert info == 0
    np.testing.assert_array_equal(Lo, L.astype(Lo.dtype))


@pytest.mark.parametrize("n", [5, 20, 28])
def test_potrf_pascal(n):
    """Pascal matrix P_ij = C(i+j, i) has Cholesky factor L_ij = C(i, j)
    exactly (all partial sums stay integers below 2^53 for n <= 28)."""
    P = np.array([[math.comb(i + j, i) for j in range(n)] for i in range(n)], dtype=np.float64)
    Lx = np.array([[math.comb(i, j) for j in range(n)] for i in range(n)], dtype=np.float64)
    Lo, info = oracle.potrf(P)
    assert info == 0
    np.testing.assert_array_equal(Lo, Lx)
    assert oracle.logdet(Lo) == 0.0


def test_potrf_tridiagonal_closed_form():
    """tridiag(-1, 2, -1): L_kk = sqrt((k+1)/k), L_{k+1,k} = -sqrt(k/(k+1))
    (1-based k), det = n + 1."""
    n = 1000
    A = 2.0 * np.eye(n) - np.eye(n, k=1) - np.eye(n, k=-1)
    Lo, info = oracle.potrf(A)
    assert info == 0
    k = np.arange(1, n + 1, dtype=np.float64)
    np.testing.assert_allclose(np.diag(Lo), np.sqrt((k + 1) / k), rtol=64 * EPS64, atol=0)
    np.testing.assert_allclose(np.diag(Lo, -1), -np.sqrt(k[:-1] / (k[:-1] + 1)), rtol=64 * EPS64, atol=0)
    assert np.count_nonzero(np.tril(Lo, -2)) == 0
    assert abs(oracle.logdet(Lo) - math.log(n + 1)) < 1e-12


def test_n1_and_n2_closed_forms():
    L1, info = oracle.potrf(np.array([[9.0]]))
    assert info == 0 and L1[0, 0] == 3.0
    assert oracle.potrs(L1, np.array([[18.0]]))[0, 0] == 2.0
    assert abs(oracle.logdet(L1) - math.log(9.0)) < 1e-15

    a, b, c = 2.0, 0.7, 3.1
    A = np.array([[a, b], [b, c]])
    L, info = oracle.potrf(A)
    assert info == 0
    l11 = math.sqrt(a)
    l21 = b / l11
    l22 = math.sqrt(c - l21 * l21)
    np.testing.assert_allclose(L, [[l11, 0.0], [l21, l22]], rtol=2 * EPS64, atol=0)
    rhs = np.array([[1.0, -2.0], [0.5, 4.0]])
    det = a * c - b * b
    x = np.array([[c * rhs[0, k] - b * rhs[1, k], -b * rhs[0, k] + a * rhs[1, k]] for k in range(2)]).T / det
    np.testing.assert_allclose(oracle.potrs(L, rhs), x, rtol=1e-14, atol=1e-15)
    assert abs(oracle.logdet(L) - math.log(det)) < 1e-14


def test_empty():
    L, info = oracle.potrf(np.zeros((0, 0)))
    assert info == 0 and L.shape == (0, 0)
    assert oracle.logdet(L) == 0.0
    assert oracle.potrs(L, np.zeros((0, 3))).shape == (0, 3)


# --------------------------------------------------------------- potrs ---

@pytest.mark.parametrize("cplx", [False, True])
def test_potrs_exact_integer_solution(cplx):
    """A = L L^H, b = A x* with integer L and x*: both substitutions stay in
    exact integers, so x* must come back bit for bit."""
    rng = np.random.default_rng(11)
    n, nrhs = 24, 5
    L = int_lower(n, rng, cplx, diag_max=1)  # unit diagonal keeps every quotient integral
    A = exact_gram(L)
    xs = rng.integers(-5, 6, size=(n, nrhs)).astype(np.float64)
    if cplx:
        xs = xs + 1j * rng.integers(-5, 6, size=(n, nrhs))
    Li = L.astype(np.complex128 if cplx else np.float64)
    b = Li @ (Li.conj().T @ xs)  # exact: small integers
    Lo, info = oracle.potrf(A)
    assert info == 0
    x = oracle.potrs(Lo, b)
    np.testing.assert_array_equal(x, xs)


def test_potrs_uses_both_triangular_solves_in_order():
    """Non-symmetric check of the two sweeps: with a non-trivial L the solve of
    L L^T x = b differs from the solve of L^T L x = b; only the former is right."""
    rng = np.random.default_rng(5)
    L = int_lower(10, rng, diag_max=1).astype(np.float64)
    b = rng.standard_normal((10, 2))
    x = oracle.potrs(L, b)
    np.testing.assert_allclose(L @ (L.T @ x), b, rtol=0, atol=1e-9 * np.abs(b).max())
    assert not np.allclose(L.T @ (L @ x), b)


# -------------------------------------------------------------- logdet ---

@pytest.mark.parametrize("n,seed", [(1, 0), (2, 1), (3, 2), (4, 3), (5, 4), (6, 5)])
@pytest.mark.parametrize("cplx", [False, True])
def test_logdet_vs_cofactor_expansion(n, seed, cplx):
    rng = np.random.default_rng(100 + seed)
    M = rng.integers(-3, 4, size=(n, n))
    if cplx:
        # Hermitian positive-definite Gaussian-integer matrix C C^H + I with
        # C = M + i Mi; its determinant is real and positive.
        Mi = rng.integers(-3, 4, size=(n, n))
        Ar = M @ M.T + Mi @ Mi.T + np.eye(n, dtype=np.int64)
        Ai = Mi @ M.T - M @ Mi.T
        A = Ar + 1j * Ai
        det_r, det_i = laplace_det_complex(
            [[(Fraction(int(Ar[i, j])), Fraction(int(Ai[i, j]))) for j in range(n)] for i in range(n)])
        assert det_i == 0 and det_r > 0
        ref = math.log(det_r)
    else:
        A = (M @ M.T + np.eye(n, dtype=np.int64)).astype(np.float64)
        det = laplace_det([[Fraction(int(v)) for v in row] for row in A])
        ref = math.log(det)
    L, info = oracle.potrf(A.astype(np.complex128 if cplx else np.float64))
    assert info == 0
    got = oracle.logdet(L)
    assert abs(got - ref) <= 1e-14 * max(1.0, abs(ref)), (got, ref)


def test_diag_benchmark_golden():
    """The pages' own potrs benchmark input, A = diag(1..N), b = ones."""
    with open(os.path.join(GOLDEN, "diag_benchmark.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        n = case["n"]
        A = np.diag(np.arange(1, n + 1, dtype=np.float64))
        L, info = oracle.potrf(A)
        assert info == 0
        x = oracle.potrs(L, np.ones(n))
        xe = np.array([float(Fraction(s)) for s in case["x"]])
        np.testing.assert_allclose(x, xe, rtol=4 * EPS64, atol=0)
        ref = math.log(int(case["det"]))
        assert abs(oracle.logdet(L) - ref) <= 4 * EPS64 * max(1.0, ref)


@pytest.mark.parametrize("n", [256, 2048])
def test_diag_benchmark_large(n):
    A = np.diag(np.arange(1, n + 1, dtype=np.float64))
    L, info = oracle.potrf(A)
    assert info == 0
    x = oracle.potrs(L, np.ones((n, 1)))
    np.testing.assert_allclose(x[:, 0], 1.0 / np.arange(1, n + 1), rtol=4 * EPS64, atol=0)
    ref = math.lgamma(n + 1)
    assert abs(oracle.logdet(L) - ref) <= 1e-14 * ref
    if n == 256:
        assert abs(ref - 1167.2572785628802) < 1e-9


# ---------------------------------------------------- library / bounds ---

@pytest.mark.parametrize("n,cplx,seed", [(64, False, 0), (257, False, 1), (1024, False, 2),
                                         (200, True, 3), (513, True, 4)])
def test_vs_lapack(n, cplx, seed):
    """Same results as LAPACK's Cholesky and Cholesky solve (via SciPy)."""
    A = random_spd(n, seed, cplx, delta=0.1)
    rng = np.random.default_rng(seed + 50)
    b = rng.standard_normal((n, 3))
    if cplx:
        b = b + 1j * rng.standard_normal((n, 3))
    L, info = oracle.potrf(A)
    assert info == 0
    Lref = scipy.linalg.cholesky(A, lower=True)
    assert np.abs(L - Lref).max() <= 1e-12 * np.abs(Lref).max()
    x = oracle.potrs(L, b)
    xref = scipy.linalg.cho_solve((Lref, True), b)
    assert np.linalg.norm(x - xref) <= 1e-12 * np.linalg.norm(xref)
    sign, ld = np.linalg.slogdet(A)
    assert abs(oracle.logdet(L) - ld) <= 1e-12 * max(1.0, abs(ld))


@pytest.mark.parametrize("n,cplx", [(256, False), (1000, False), (300, True)])
def test_backward_error_bound(n, cplx):
    """Higham, Accuracy and Stability of Numerical Algorithms, Thm 10.3/10.4:
    Cholesky + substitution is backward stable; the normwise backward error of
    x and the factorization residual must lie well inside 64 n eps."""
    A = random_spd(n, 9, cplx, delta=0.05)
    rng = np.random.default_rng(10)
    b = rng.standard_normal((n, 4)) + (1j * rng.standard_normal((n, 4)) if cplx else 0)
    L, info = oracle.potrf(A)
    assert info == 0
    x = oracle.potrs(L, b)
    eta = rigal_gaches(A, x, b)
    assert eta.max() <= 64 * n * EPS64
    fac = np.linalg.norm(A - L @ L.conj().T) / np.linalg.norm(A)
    assert fac <= 64 * n * EPS64


# ---------------------------------------------------------------- info ---

def test_info_negative_diagonal():
    A = random_spd(50, 1)
    for j in (0, 7, 49):
        B = A.copy()
        B[j, j] = -1.0
        _, info = oracle.potrf(B)
        # the leading j x j block is untouched and positive definite; at j the
        # pivot -1 - sum |L_jk|^2 is negative
        assert info == j + 1


def test_info_nan_and_zero():
    A = random_spd(10, 2)
    A[0, 0] = np.nan
    assert oracle.potrf(A)[1] == 1
    assert oracle.potrf(np.zeros((5, 5)))[1] == 1
    x, ld, info = oracle.solve(np.zeros((3, 3)), np.ones((3, 1)), want_logdet=True)
    assert info == 1 and np.isnan(x).all() and math.isnan(ld)


@pytest.mark.parametrize("j0", [0, 1, 3, 5])
def test_info_matches_leading_minors(j0):
    """info = first k whose leading k x k minor is not positive.  A = U D U^T
    with integer unit-lower U, D = (1, 4, 9, ...) except D[j0] <= 0: every
    pivot is exact and the brute-force minors are products of D."""
    n = 6
    rng = np.random.default_rng(j0)
    U = np.tril(rng.integers(-2, 3, size=(n, n)), -1) + np.eye(n, dtype=np.int64)
    D = np.array([(i + 1) ** 2 for i in range(n)], dtype=np.int64)
    D[j0] = -(j0 % 2)  # 0 or -1
    A = U @ np.diag(D) @ U.T
    minors = [laplace_det([[Fraction(int(v)) for v in row[:k]] for row in A[:k]]) for k in range(1, n + 1)]
    first_bad = next(k for k, m in enumerate(minors, start=1) if m <= 0)
    _, info = oracle.potrf(A.astype(np.float64))
    assert info == first_bad == j0 + 1


# ------------------------------------------- forward solve, GP likelihood ---
# JAXMg paper, "Research Impact Statement", "Cholesky solve (potrs)": the
# Gaussian-process marginal log-likelihood -1/2 r^T A^-1 r - 1/2 log det A -
# (N/2) log 2 pi, r = y - m.

@pytest.mark.parametrize("n,seed", [(1, 0), (7, 1), (50, 2), (200, 3)])
def test_gp_loglik_matches_scipy_multivariate_normal(n, seed):
    """scipy's multivariate normal log-density (computed through an eigen-
    decomposition of the covariance) is the same quantity."""
    import scipy.stats
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((n, n))
    A = G @ G.T / n + 0.3 * np.eye(n)
    m = rng.standard_normal(n)
    ys = rng.standard_normal((n, 3))
    v, info = oracle.gp_loglik(A, ys - m[:, None])
    assert info == 0
    ref = scipy.stats.multivariate_normal(mean=m, cov=A).logpdf(ys.T)
    np.testing.assert_allclose(v, np.atleast_1d(ref), rtol=1e-11, atol=1e-11)


def test_gp_loglik_diagonal_closed_form():
    rng = np.random.default_rng(4)
    n = 300
    d = 0.1 + rng.random(n)
    r = rng.standard_normal((n, 2))
    v, info = oracle.gp_loglik(np.diag(d), r)
    ref = -0.5 * (r ** 2 / d[:, None]).sum(0) - 0.5 * np.log(d).sum() - 0.5 * n * np.log(2 * np.pi)
    np.testing.assert_allclose(v, ref, rtol=1e-13)


def test_gp_loglik_one_point():
    """N = 1: -r^2 / (2 a) - log(a) / 2 - log(2 pi) / 2 exactly."""
    v, info = oracle.gp_loglik(np.array([[4.0]]), np.array([2.0]))
    assert info == 0 and abs(v - (-0.5 - 0.5 * np.log(4.0) - 0.5 * np.log(2 * np.pi))) < 1e-15


def test_gp_loglik_not_positive_definite():
    A = np.array([[1.0, 2.0], [2.0, 1.0]])
    v, info = oracle.gp_loglik(A, np.ones((2, 2)))
    assert info == 2 and np.isnan(v).all()


@pytest.mark.parametrize("cplx", [False, True])
def test_forward_solve_exact_integers(cplx):
    """Unit lower-triangular integer L and integer y: b = L y is exact, so the
    substitution must return y bit for bit."""
    rng = np.random.default_rng(12)
    n = 30
    L = int_lower(n, rng, cplx, diag_max=1).astype(np.complex128 if cplx else np.float64)
    y = rng.integers(-4, 5, size=(n, 2)).astype(np.float64)
    if cplx:
        y = y + 1j * rng.integers(-4, 5, size=(n, 2))
    b = L @ y
    np.testing.assert_array_equal(oracle.forward_solve(L, b), y)


def test_forward_solve_matches_scipy_and_keeps_input():
    import scipy.linalg
    rng = np.random.default_rng(13)
    n = 80
    A = random_spd(n, 3, False, delta=0.2)
    L, info = oracle.potrf(A)
    for b in (rng.standard_normal((n, 1)), rng.standard_normal(n), rng.standard_normal((n, 4))):
        b0 = b.copy()
        y = oracle.forward_solve(L, b)
        assert np.array_equal(b, b0)  # the caller's array is never written
        ref = scipy.linalg.solve_triangular(L, b, lower=True)
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
        x = oracle.potrs(L, b)
        assert np.array_equal(b, b0)


# ----------------------------------------------- generalized eigenproblem ---
# Page "Differentiable Generalized Eigenvalue Decomposition", section "API
# Reference": type 1 is A v = w B v, type 2 A B v = w v, type 3 B A v = w v.

def _herm(n, seed, cplx):
    """Hermitian (not definite) test matrix with a real diagonal."""
    rng = np.random.default_rng(seed)
    M = rng.standard_normal((n, n))
    if cplx:
        M = M + 1j * rng.standard_normal((n, n))
    M = M + M.conj().T
    return np.tril(M, -1) + np.tril(M, -1).conj().T + np.diag(np.diag(M).real)


@pytest.mark.parametrize("itype", [1, 2, 3])
@pytest.mark.parametrize("n,cplx", [(1, False), (5, False), (60, False), (7, True), (50, True)])
def test_sygst_eigenvalues_match_scipy_generalized_eigh(itype, n, cplx):
    """The standard form has the generalized problem's eigenvalues; scipy's
    generalized eigh (LAPACK's own reduction and solver) gives them."""
    A = _herm(n, 20 + n, cplx)
    B = random_spd(n, 40 + n, cplx, delta=0.5)
    L, info = oracle.potrf(B)
    assert info == 0
    C = oracle.sygst(itype, A, L)
    np.testing.assert_allclose(C, C.conj().T, rtol=0, atol=1e-12 * np.abs(C).max())
    w = np.linalg.eigvalsh(C)
    ref = scipy.linalg.eigh(A, B, type=itype, eigvals_only=True)
    np.testing.assert_allclose(w, ref, rtol=0, atol=1e-10 * max(1.0, np.abs(ref).max()))


@pytest.mark.parametrize("itype", [1, 2, 3])
@pytest.mark.parametrize("cplx", [False, True])
def test_sygst_eigenvectors_solve_the_generalized_problem(itype, cplx):
    """Back-transformed eigenvectors of C solve the original problem:
    v = L^-H u for types 1 and 2, v = L u for type 3."""
    n = 40
    A = _herm(n, 5, cplx)
    B = random_spd(n, 6, cplx, delta=0.3)
    L, _ = oracle.potrf(B)
    w, U = np.linalg.eigh(oracle.sygst(itype, A, L))
    if itype == 3:
        V = L @ U
    else:
        V = scipy.linalg.solve_triangular(L.conj().T, U, lower=False)
    lhs = {1: A @ V, 2: A @ B @ V, 3: B @ A @ V}[itype]
    rhs = (B @ V) * w if itype == 1 else V * w
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-9 * np.abs(lhs).max())


@pytest.mark.parametrize("itype", [1, 2, 3])
@pytest.mark.parametrize("cplx", [False, True])
def test_sygst_identity_factor_returns_A(itype, cplx):
    """B = I gives C = A exactly, and only A's lower triangle is read."""
    n = 9
    A = _herm(n, 8, cplx)
    Araw = np.tril(A) + np.triu(np.full((n, n), 7.5), 1)  # upper triangle is junk
    C = oracle.sygst(itype, Araw, np.eye(n))
    np.testing.assert_array_equal(C, A)


@pytest.mark.parametrize("itype", [1, 2, 3])
def test_sygst_diagonal_factor_closed_form(itype):
    """Diagonal L = diag(s) with powers of two: C_ij = A_ij / (s_i s_j) for
    type 1 and A_ij s_i s_j for types 2 and 3, exactly."""
    n = 12
    A = _herm(n, 9, False)
    s = 2.0 ** np.arange(-3, n - 3)
    C = oracle.sygst(itype, A, np.diag(s))
    ref = A / np.outer(s, s) if itype == 1 else A * np.outer(s, s)
    np.testing.assert_array_equal(C, ref)


def _exact_mat(a):
    return [[Fraction(int(v)) for v in row] for row in a]


def _exact_mul(x, y):
    n, m, p = len(x), len(y), len(y[0])
    return [[sum(x[i][k] * y[k][j] for k in range(m)) for j in range(p)] for i in range(n)]


@pytest.mark.parametrize("itype", [1, 2])
def test_sygst_exact_integer_brute_force(itype):
    """Unit lower-triangular integer L: L^-1 is an integer matrix, so with an
    integer A every result is a small integer; compared with exact rational
    arithmetic (a transposed or unconjugated operand changes the values)."""
    rng = np.random.default_rng(31)
    n = 8
    L = int_lower(n, rng, diag_max=1, off=2).astype(np.float64)
    Ai = rng.integers(-5, 6, size=(n, n))
    A = np.tril(Ai, -1) + np.tril(Ai, -1).T + np.diag(np.diag(Ai))
    Lx, Ax = _exact_mat(L), _exact_mat(A)
    if itype == 1:
        # inverse of the unit lower-triangular L by exact forward substitution
        inv = [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]
        for i in range(n):
            for j in range(n):
                inv[i][j] -= sum(Lx[i][k] * inv[k][j] for k in range(i))
        invH = [list(r) for r in zip(*inv)]
        ref = _exact_mul(_exact_mul(inv, Ax), invH)
    else:
        LH = [list(r) for r in zip(*Lx)]
        ref = _exact_mul(_exact_mul(LH, Ax), Lx)
    assert all(v.denominator == 1 and abs(v) < 2**50 for row in ref for v in row)
    C = oracle.sygst(itype, A.astype(np.float64), L)
    np.testing.assert_array_equal(C, np.array([[float(v) for v in row] for row in ref]))


# ------------------------------------------- factorization by column ranges ---

@pytest.mark.parametrize("cplx", [False, True])
def test_factorization_by_ranges_recovers_integer_factor(cplx):
    """Taken a range of columns at a time, the factorization still recovers
    a hand-built integer factor bit for bit, and equals potrf's bits on a
    random input for any split."""
    rng = np.random.default_rng(11)
    L = int_lower(30, rng, cplx)
    f = oracle.Factorization(exact_gram(L))
    for j1 in (1, 7, 8, 29, 30):
        assert f.advance(j1) == 0
    assert f.done
    np.testing.assert_array_equal(f.l, L.astype(f.l.dtype))
    A = random_spd(257, 12, cplx)
    Lo, _ = oracle.potrf(A)
    for parts in (1, 3, 8):
        g = oracle.Factorization(A)
        for j1 in oracle.Factorization.equal_work_bounds(257, parts):
            g.advance(j1)
        assert g.done and g.info == 0
        np.testing.assert_array_equal(g.l, Lo)


def test_factorization_by_ranges_stops_at_the_failing_pivot():
    """A non-positive leading minor inside the second range stops the
    factorization there with the 1-based column, as potrf does."""
    rng = np.random.default_rng(13)
    L = int_lower(20, rng)
    A = exact_gram(L)
    A[12, 12] = -1.0
    f = oracle.Factorization(A)
    assert f.advance(10) == 0 and not f.done
    assert f.advance(20) == 13 and f.done
    assert oracle.potrf(A)[1] == 13


def test_equal_work_bounds():
    """Boundaries are increasing, end at n, and split the n^3/6 multiply-adds
    into parts within one column's work of each other."""
    n, parts = 4096, 8
    b = oracle.Factorization.equal_work_bounds(n, parts)
    assert len(b) == parts and b[-1] == n and all(x < y for x, y in zip(b, b[1:]))
    work = lambda j: n * j * j / 2.0 - j**3 / 3.0  # noqa: E731
    edges = [0] + b
    shares = [work(y) - work(x) for x, y in zip(edges, edges[1:])]
    assert max(shares) - min(shares) <= 2 * n * n / 4


# ------------------------------------------------------ single precision ---

EPS32 = float(np.finfo(np.float32).eps)


@pytest.mark.parametrize("n,seed", [(1, 0), (8, 2), (17, 3)])
def test_single_recovers_integer_factor_exactly(n, seed):
    """Single precision: every partial sum of the integer Gram matrix stays
    below 2^24 and every sqrt is of a perfect square, so L comes back bit for
    bit."""
    L = int_lower(n, np.random.default_rng(seed))
    A = exact_gram(L)
    assert np.abs(A).max() < 2**24
    Lo, info = oracle.potrf_single(A)
    assert info == 0 and Lo.dtype == np.float32
    np.testing.assert_array_equal(Lo, L.astype(np.float32))


def test_single_pascal_and_closed_forms():
    n = 12  # the largest Pascal entry C(22, 11) < 2^24
    P = np.array([[math.comb(i + j, i) for j in range(n)] for i in range(n)], dtype=np.float32)
    Lx = np.array([[math.comb(i, j) for j in range(n)] for i in range(n)], dtype=np.float32)
    Lo, info = oracle.potrf_single(P)
    assert info == 0
    np.testing.assert_array_equal(Lo, Lx)
    assert oracle.logdet_single(Lo) == 0.0
    L1, info = oracle.potrf_single(np.array([[16.0]], dtype=np.float32))
    assert info == 0 and L1[0, 0] == 4.0
    assert oracle.potrs_single(L1, np.array([[8.0]], dtype=np.float32))[0, 0] == 0.5
    A = np.eye(5, dtype=np.float32)
    A[3, 3] = -2.0
    assert oracle.potrf_single(A)[1] == 4


@pytest.mark.parametrize("n,seed", [(64, 0), (500, 1)])
def test_single_vs_lapack_spotrf(n, seed):
    """Single-precision LAPACK (SciPy's cholesky / cho_solve on float32
    input: spotrf / spotrs) agrees within single-precision rounding, and the
    normwise backward error of x stays inside 64 n eps(float32)."""
    A = random_spd(n, seed, False, delta=0.5).astype(np.float32)
    b = np.random.default_rng(seed + 3).standard_normal((n, 3)).astype(np.float32)
    L, info = oracle.potrf_single(A)
    assert info == 0 and L.dtype == np.float32
    Lref = scipy.linalg.cholesky(A, lower=True)
    assert Lref.dtype == np.float32
    assert np.abs(L - Lref).max() <= 64 * n * EPS32 * np.abs(Lref).max()
    x = oracle.potrs_single(L, b)
    xref = scipy.linalg.cho_solve((Lref, True), b)
    assert np.linalg.norm(x - xref) <= 1e-3 * np.linalg.norm(xref)
    eta = rigal_gaches(A.astype(np.float64), x.astype(np.float64), b.astype(np.float64))
    assert eta.max() <= 64 * n * EPS32
    _, ld = np.linalg.slogdet(A.astype(np.float64))
    assert abs(oracle.logdet_single(L) - ld) <= 1e-3 * max(1.0, abs(ld))
