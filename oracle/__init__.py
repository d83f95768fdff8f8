"""Test infrastructure only: ctypes wrapper of the plain CPU oracle (oracle.c).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg use this package.  It shares no code with the GPU library: it has its own
C source, built by the host compiler with OpenMP into ``liboracle.so`` next to
this file.

Every function takes *logical* NumPy matrices (any memory order) and returns
NumPy arrays.  Real inputs are computed in float64 and complex inputs in
complex128, whatever their storage precision (a float32 input is widened
exactly first).

JAXMg paper, "Software design": potrs solves A x = b for symmetric
(Hermitian) positive-definite A through a Cholesky factorization, and the
same factorization optionally gives log det(A).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc and OpenMP into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            i64, vp = ctypes.c_int64, ctypes.c_void_p
            lib.oracle_num_threads.restype = ctypes.c_int
            for suf in ("d", "z"):
                f = getattr(lib, "oracle_potrf_cols_" + suf)
                f.argtypes, f.restype = [i64, vp, vp, i64, i64], ctypes.c_int
            for suf in ("d", "z", "s"):
                f = getattr(lib, "oracle_potrf_" + suf)
                f.argtypes, f.restype = [i64, vp, vp], ctypes.c_int
                f = getattr(lib, "oracle_potrs_" + suf)
                f.argtypes, f.restype = [i64, i64, vp, vp], None
                f = getattr(lib, "oracle_logdet_" + suf)
                f.argtypes, f.restype = [i64, vp], ctypes.c_double
                if suf != "s":
                    f = getattr(lib, "oracle_fwd_" + suf)
                    f.argtypes, f.restype = [i64, i64, vp, vp], None
            _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().oracle_num_threads())


def _wide(x) -> np.ndarray:
    x = np.asarray(x)
    dt = np.complex128 if np.iscomplexobj(x) else np.float64
    return np.ascontiguousarray(x, dtype=dt)


def _p(x: np.ndarray):
    return x.ctypes.data_as(ctypes.c_void_p)


def potrf(a):
    """Cholesky factor of the lower triangle of ``a``: returns (L, info).

    L is lower triangular with a positive real diagonal and zeros above it.
    info = 0 on success, else j + 1 for the first column j whose pivot is not
    positive (then L holds the columns finished before j and zeros after)."""
    a = _wide(a)
    n = a.shape[0]
    if a.shape != (n, n):
        raise ValueError("a must be square")
    l = np.zeros_like(a)
    if n == 0:
        return l, 0
    f = _load().oracle_potrf_z if np.iscomplexobj(a) else _load().oracle_potrf_d
    info = f(n, _p(a), _p(l))
    return l, int(info)


class Factorization:
    """The factorization of :func:`potrf` taken a range of columns at a time
    (the same arithmetic, so the same bits): ``advance(j1)`` computes columns
    up to ``j1``, and ``done`` is true once all ``n`` are there or a pivot
    failed.  For large orders, where one call runs for minutes, this lets a
    caller report progress between ranges.  ``a`` is read as potrf reads it
    (lower triangle; real part of the diagonal)."""

    def __init__(self, a):
        self.a = _wide(a)
        self.n = self.a.shape[0]
        if self.a.shape != (self.n, self.n):
            raise ValueError("a must be square")
        self.l = np.zeros_like(self.a)
        self.next = 0
        self.info = 0

    @property
    def done(self) -> bool:
        return self.info != 0 or self.next >= self.n

    def advance(self, j1: int) -> int:
        j1 = min(int(j1), self.n)
        if self.done or j1 <= self.next:
            return self.info
        f = _load().oracle_potrf_cols_z if np.iscomplexobj(self.a) else _load().oracle_potrf_cols_d
        self.info = int(f(self.n, _p(self.a), _p(self.l), self.next, j1))
        self.next = j1
        return self.info

    @staticmethod
    def equal_work_bounds(n: int, parts: int):
        """Column boundaries splitting the factorization of order n into
        ``parts`` ranges of about equal work (column j costs about (n - j) j
        multiply-adds)."""
        total = n**3 / 6.0
        bounds, j = [], 0
        for p in range(1, parts):
            goal = total * p / parts
            while j < n and (n * j * j / 2.0 - j**3 / 3.0) < goal:
                j += 1
            bounds.append(j)
        bounds.append(n)
        return bounds


def potrs(l, b):
    """Solve (L L^H) X = B given the factor L: L Y = B, then L^H X = Y."""
    l = _wide(l)
    n = l.shape[0]
    b = np.asarray(b)
    vec = b.ndim == 1
    b2 = b.reshape(n, 1) if vec else b
    cplx = np.iscomplexobj(l) or np.iscomplexobj(b2)
    dt = np.complex128 if cplx else np.float64
    l = np.ascontiguousarray(l, dtype=dt)
    # right-hand-side columns one after another: the transpose, row-major
    bt = np.array(b2.T, dtype=dt, order="C", copy=True)  # never the caller's memory
    nrhs = bt.shape[0]
    if n > 0 and nrhs > 0:
        f = _load().oracle_potrs_z if cplx else _load().oracle_potrs_d
        f(n, nrhs, _p(l), _p(bt))
    x = bt.T.copy()
    return x.reshape(b.shape) if vec else x


def forward_solve(l, b):
    """Y with L Y = B (forward substitution only) given the factor L."""
    l = _wide(l)
    n = l.shape[0]
    b = np.asarray(b)
    vec = b.ndim == 1
    b2 = b.reshape(n, 1) if vec else b
    cplx = np.iscomplexobj(l) or np.iscomplexobj(b2)
    dt = np.complex128 if cplx else np.float64
    l = np.ascontiguousarray(l, dtype=dt)
    bt = np.array(b2.T, dtype=dt, order="C", copy=True)  # never the caller's memory
    if n > 0 and bt.shape[0] > 0:
        f = _load().oracle_fwd_z if cplx else _load().oracle_fwd_d
        f(n, bt.shape[0], _p(l), _p(bt))
    y = bt.T.copy()
    return y.reshape(b.shape) if vec else y


def gp_loglik(a, r):
    """Gaussian-process marginal log-likelihood per column r_j of R (JAXMg
    paper, "Research Impact Statement", "Cholesky solve (potrs)"): with
    r = y - m the residual and A = K + Sigma,

        log L = -1/2 r^T A^{-1} r - 1/2 log det A - (N/2) log(2 pi),

    written out directly: x = A^{-1} r by the oracle's solve, the quadratic
    term as the dot product r . x, log det A from the factor.  Real A only.
    Returns (values, info); values are NaN when info != 0."""
    a = np.asarray(a)
    if np.iscomplexobj(a):
        raise ValueError("the likelihood is defined for real A")
    r = np.asarray(r, dtype=np.float64)
    vec = r.ndim == 1
    r2 = r.reshape(-1, 1) if vec else r
    n = r2.shape[0]
    x, ld, info = solve(a, r2, want_logdet=True)
    if info != 0:
        out = np.full(r2.shape[1], np.nan)
    else:
        quad = np.einsum("ij,ij->j", r2, x)
        out = -0.5 * quad - 0.5 * ld - 0.5 * n * np.log(2.0 * np.pi)
    return (out[0] if vec else out), info


def sygst(itype: int, a, l):
    """Standard form of the Hermitian-definite generalized eigenproblem for
    (A, B = L L^H), the reduction behind the page "Differentiable Generalized
    Eigenvalue Decomposition", section "API Reference" (types 1: A v = w B v,
    2: A B v = w v, 3: B A v = w v), written as its definition:

        itype 1:    C = L^-1 A L^-H     (L^-1 by forward substitution on I)
        itype 2, 3: C = L^H A L

    Only the lower triangle of ``a`` is read (A Hermitian, the diagonal's
    imaginary part taken as zero); ``l`` is the lower-triangular factor.
    Returns the full n x n matrix C."""
    if itype not in (1, 2, 3):
        raise ValueError("itype must be 1, 2 or 3")
    a = _wide(a)
    n = a.shape[0]
    cplx = np.iscomplexobj(a) or np.iscomplexobj(l)
    dt = np.complex128 if cplx else np.float64
    low = np.tril(a, -1).astype(dt)
    full = low + low.conj().T + np.diag(np.real(np.diagonal(a))).astype(dt)
    lt = np.tril(np.asarray(l, dtype=dt))
    if n == 0:
        return np.zeros((0, 0), dtype=dt)
    if itype == 1:
        linv = forward_solve(lt, np.eye(n, dtype=dt))
        return linv @ full @ linv.conj().T
    return lt.conj().T @ full @ lt


def logdet(l) -> float:
    """log det(A) = 2 * sum_i log L_ii from the Cholesky factor L of A."""
    l = _wide(l)
    n = l.shape[0]
    if n == 0:
        return 0.0
    f = _load().oracle_logdet_z if np.iscomplexobj(l) else _load().oracle_logdet_d
    return float(f(n, _p(l)))


def solve(a, b, want_logdet: bool = False):
    """potrf, then potrs (and log det).  Returns (X, info) or (X, logdet, info);
    X and logdet are NaN when info != 0."""
    l, info = potrf(a)
    b = np.asarray(b)
    if info != 0:
        x = np.full(b.shape, np.nan, dtype=np.result_type(b.dtype, np.asarray(a).dtype, np.float64))
        return (x, float("nan"), info) if want_logdet else (x, info)
    x = potrs(l, b)
    if want_logdet:
        return x, logdet(l), info
    return x, info


# ------------------------------------------------------ single precision ---
# The same routines with every operation in IEEE single precision, for the CPU
# baseline of float32 workloads in their own working precision.  Parity is
# always checked against the double-precision routines above.

def _single(x) -> np.ndarray:
    x = np.asarray(x)
    if np.iscomplexobj(x):
        raise ValueError("the single-precision oracle is real only")
    return np.ascontiguousarray(x, dtype=np.float32)


def potrf_single(a):
    """:func:`potrf` in single precision: returns (L float32, info)."""
    a = _single(a)
    n = a.shape[0]
    if a.shape != (n, n):
        raise ValueError("a must be square")
    l = np.zeros_like(a)
    if n == 0:
        return l, 0
    return l, int(_load().oracle_potrf_s(n, _p(a), _p(l)))


def potrs_single(l, b):
    """:func:`potrs` in single precision."""
    l = _single(l)
    n = l.shape[0]
    b = np.asarray(b)
    vec = b.ndim == 1
    b2 = b.reshape(n, 1) if vec else b
    bt = np.array(b2.T, dtype=np.float32, order="C", copy=True)
    if n > 0 and bt.shape[0] > 0:
        _load().oracle_potrs_s(n, bt.shape[0], _p(l), _p(bt))
    x = bt.T.copy()
    return x.reshape(b.shape) if vec else x


def logdet_single(l) -> float:
    """2 * sum_i log L_ii of a single-precision factor, summed in double."""
    l = _single(l)
    n = l.shape[0]
    return 0.0 if n == 0 else float(_load().oracle_logdet_s(n, _p(l)))
