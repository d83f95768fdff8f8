"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Small and medium sizes, with ragged tiles in all four dtypes, and the two
small benchmark workloads are compared element by element with the oracle run
on the very same input bytes; so are the invariants (bitwise determinism,
power-of-two scaling, untouched upper triangle and padding, info on failed
pivots).  The three large workloads are in test_gpu_workloads.py, every kernel
variant they use at oracle-sized orders in test_gpu_variants.py.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import spdgen
from helpers import EPS, L_TOL, LOGDET_TOL, X_TOL, backward_error, logdet_rel, rel_err_cols, wide

pytestmark = pytest.mark.gpu


def cm_copy(t: torch.Tensor, ld: int | None = None, pad_value=0.0) -> torch.Tensor:
    """Column-major copy of a logical matrix (on the same device)."""
    return spdgen.to_colmajor(t, ld, pad_value)


def bits(t: torch.Tensor) -> torch.Tensor:
    t = torch.view_as_real(t) if t.is_complex() else t
    return t.contiguous().view(torch.int64 if t.dtype == torch.float64 else torch.int32)


def gpu_solve(spd, A, B, T_A, want_logdet=True):
    """potrf -> logdet -> potrs in place on A and B; returns (info, logdet)."""
    n = A.shape[0]
    nrhs = B.shape[1]
    work = spd.workspace(A.dtype, n, nrhs, T_A)
    info = spd.potrf(A, T_A, work=work)
    ld = spd.logdet(A, info) if want_logdet else None
    spd.potrs(A, B, T_A, info=info, work=work)
    torch.cuda.synchronize()
    return int(info.item()), (float(ld.item()) if ld is not None else None)


def check_against_oracle(spd, dt, n, nrhs, T_A, seed=0, delta=0.5, A=None, B=None):
    if A is None:
        A = spdgen.make_A(n, dt, delta, seed, device="cuda")
    if B is None:
        B = spdgen.make_B(n, nrhs, dt, seed, device="cuda")
    A_np = wide(A)  # the exact input bytes, widened for the oracle
    B_np = wide(B)
    L = cm_copy(A)
    X = cm_copy(B)
    info, ld = gpu_solve(spd, L, X, T_A)
    assert info == 0
    Lo, info_o = oracle.potrf(A_np)
    assert info_o == 0
    Xo = oracle.potrs(Lo, B_np)
    ldo = oracle.logdet(Lo)

    Lg = np.tril(wide(L))
    err_L = np.abs(Lg - Lo).max() / np.abs(Lo).max()
    err_x = rel_err_cols(X, Xo)
    eta = backward_error(A, X, B)
    err_ld = logdet_rel(ld, ldo)
    tol_ld = LOGDET_TOL if dt in ("f64", "c128") else 1e-4
    msg = f"{dt} n={n} nrhs={nrhs} T_A={T_A}: L {err_L:.2e} x {err_x:.2e} eta {eta:.2e} logdet {err_ld:.2e}"
    print(msg)
    assert err_L <= L_TOL[dt], msg
    assert err_x <= X_TOL[dt], msg
    assert eta <= 64 * n * EPS[dt], msg
    assert err_ld <= tol_ld, msg
    return L, X, ld


SMALL_CASES = [
    ("f64", 1, 1, 64), ("f64", 2, 3, 1), ("f64", 63, 2, 16), ("f64", 64, 1, 64), ("f64", 65, 5, 64),
    ("f64", 127, 4, 32), ("f64", 130, 7, 100), ("f64", 300, 16, 128), ("f64", 777, 3, 1000),
    ("f64", 1000, 33, 256), ("f64", 1500, 8, 512), ("f64", 2100, 130, 192),
    ("f32", 65, 2, 64), ("f32", 300, 16, 128), ("f32", 1000, 33, 256), ("f32", 1500, 64, 512),
    ("c128", 1, 1, 8), ("c128", 65, 3, 64), ("c128", 300, 16, 100), ("c128", 1000, 32, 256),
    ("c64", 130, 4, 64), ("c64", 700, 8, 256),
]


@pytest.mark.parametrize("dt,n,nrhs,T_A", SMALL_CASES)
def test_parity_sweep(gpu, dt, n, nrhs, T_A):
    check_against_oracle(gpu, dt, n, nrhs, T_A, seed=n % 7)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_config1_full(gpu, seed):
    """fp64 N=256, N_RHS=1, T_A=64, A = G G^T/N + I: element-by-element."""
    A, B, c = spdgen.make_config(1, seed, device="cuda")
    check_against_oracle(gpu, c["dtype"], c["n"], c["nrhs"], c["T_A"], A=A, B=B)


def test_config2_full(gpu):
    """fp64 N=4096, N_RHS=16, T_A=256, delta=0.1: element-by-element."""
    A, B, c = spdgen.make_config(2, 0, device="cuda")
    check_against_oracle(gpu, c["dtype"], c["n"], c["nrhs"], c["T_A"], A=A, B=B)


# ------------------------------------------------------- invariants -------

def test_pages_benchmark_input(gpu):
    """A = diag(1..N), b = ones (the JAXMg paper's potrs benchmark input):
    x_i = 1/i, log det = ln N!."""
    for n, T in ((256, 64), (2048, 512), (1000, 96)):
        A, B = spdgen.diag_benchmark(n, 2, "f64", device="cuda")
        info, ld = gpu_solve(gpu, A, B, T)
        assert info == 0
        xe = 1.0 / np.arange(1, n + 1)
        np.testing.assert_allclose(wide(B)[:, 0], xe, rtol=4 * EPS["f64"], atol=0)
        np.testing.assert_allclose(wide(B)[:, 1], xe, rtol=4 * EPS["f64"], atol=0)
        assert logdet_rel(ld, math.lgamma(n + 1)) <= 1e-13


@pytest.mark.parametrize("dt", ["f64", "c128", "f32"])
def test_deterministic(gpu, dt):
    n, nrhs, T = 700, 9, 128
    A = spdgen.make_A(n, dt, 0.3, 5, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, 5, device="cuda")
    outs = []
    for _ in range(2):
        L, X = cm_copy(A), cm_copy(B)
        info, ld = gpu_solve(gpu, L, X, T)
        assert info == 0
        outs.append((torch.tril(L).clone(), X.clone(), ld))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
    assert outs[0][2] == outs[1][2]


def test_power_of_two_scaling(gpu):
    """A -> 4A must give exactly L -> 2L and X -> X/4 (every operation scales
    by a power of two)."""
    n, nrhs, T = 600, 5, 128
    A = spdgen.make_A(n, "f64", 0.2, 8, device="cuda")
    B = spdgen.make_B(n, nrhs, "f64", 8, device="cuda")
    L1, X1 = cm_copy(A), cm_copy(B)
    gpu_solve(gpu, L1, X1, T)
    L4, X4 = cm_copy(A * 4.0), cm_copy(B)
    gpu_solve(gpu, L4, X4, T)
    assert torch.equal(torch.tril(L4), 2.0 * torch.tril(L1))
    assert torch.equal(X4, X1 / 4.0)


@pytest.mark.parametrize("dt", ["f64", "c128"])
def test_upper_triangle_and_padding_untouched(gpu, dt):
    """NaN in the strict upper triangle and in the lda/ldb padding must be
    ignored and left exactly as it was."""
    n, nrhs, T = 333, 6, 64
    A = spdgen.make_A(n, dt, 0.5, 3, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, 3, device="cuda")
    lda, ldb = n + 5, n + 3
    Lp = cm_copy(A, lda, pad_value=float("nan"))
    iu = torch.triu_indices(n, n, 1, device="cuda")
    Lp[iu[0], iu[1]] = float("nan")
    Xp = cm_copy(B, ldb, pad_value=float("nan"))
    base_A = Lp.as_strided((lda * n,), (1,)).clone()
    base_B = Xp.as_strided((ldb * nrhs,), (1,)).clone()
    info, ld = gpu_solve(gpu, Lp, Xp, T)
    assert info == 0
    Lc, Xc = cm_copy(A), cm_copy(B)
    info2, ld2 = gpu_solve(gpu, Lc, Xc, T)
    assert torch.equal(torch.tril(Lp), torch.tril(Lc))
    assert torch.equal(Xp, Xc)
    assert ld == ld2
    after_A = Lp.as_strided((lda * n,), (1,))
    after_B = Xp.as_strided((ldb * nrhs,), (1,))
    # the upper triangle and padding keep their exact bits (NaN)
    colA = torch.arange(n, device="cuda").repeat_interleave(lda)
    rowA = torch.arange(lda, device="cuda").repeat(n)
    untouched = (rowA < colA) | (rowA >= n)
    assert torch.equal(bits(after_A[untouched]), bits(base_A[untouched]))
    rowB = torch.arange(ldb, device="cuda").repeat(nrhs)
    assert torch.equal(bits(after_B[rowB >= n]), bits(base_B[rowB >= n]))


@pytest.mark.parametrize("j", [0, 5, 64, 100, 299])
def test_info_negative_pivot(gpu, j):
    n, T = 300, 64
    A = spdgen.make_A(n, "f64", 0.5, 4, device="cuda")
    A[j, j] = -1.0
    _, info_o = oracle.potrf(wide(A))
    L, X = cm_copy(A), cm_copy(spdgen.make_B(n, 2, "f64", 4, device="cuda"))
    info, ld = gpu_solve(gpu, L, X, T)
    assert info == info_o == j + 1
    assert math.isnan(ld)
    assert torch.isnan(X).all()


@pytest.mark.parametrize("dt,j", [("c128", 0), ("c128", 21), ("c128", 64), ("c128", 150), ("c128", 299),
                                  ("c64", 37), ("c64", 200)])
def test_info_negative_pivot_complex(gpu, dt, j):
    """A negative pivot anywhere in a complex leaf (inside a 16 x 16 diagonal
    block, on a block boundary, in a later tile) stops the factorization at
    the oracle's column."""
    n, T = 300, 64
    A = spdgen.make_A(n, dt, 0.5, 5, device="cuda")
    A[j, j] = -1.0
    _, info_o = oracle.potrf(wide(A))
    L, X = cm_copy(A), cm_copy(spdgen.make_B(n, 2, dt, 5, device="cuda"))
    info, ld = gpu_solve(gpu, L, X, T)
    assert info == info_o == j + 1
    assert math.isnan(ld)
    assert torch.isnan(torch.view_as_real(X)).all()


def test_info_nan_and_zero(gpu):
    n = 100
    A = spdgen.make_A(n, "c128", 0.5, 4, device="cuda")
    A[0, 0] = float("nan")
    L, X = cm_copy(A), cm_copy(spdgen.make_B(n, 1, "c128", 4, device="cuda"))
    info, ld = gpu_solve(gpu, L, X, 32)
    assert info == 1 and math.isnan(ld)
    Z = spdgen.to_colmajor(torch.zeros(n, n, dtype=torch.float64, device="cuda"))
    X = spdgen.to_colmajor(torch.ones(n, 1, dtype=torch.float64, device="cuda"))
    info, ld = gpu_solve(gpu, Z, X, 32)
    assert info == 1 and math.isnan(ld) and torch.isnan(X).all()
    with pytest.raises(gpu.LinAlgError):
        gpu.solve(spdgen.to_colmajor(torch.zeros(4, 4, dtype=torch.float64, device="cuda")),
                  spdgen.to_colmajor(torch.ones(4, 1, dtype=torch.float64, device="cuda")), 2)


def test_empty(gpu):
    A = torch.empty((0, 0), dtype=torch.float64, device="cuda")
    info = gpu.potrf(A, 16)
    ld = gpu.logdet(A, info)
    torch.cuda.synchronize()
    assert int(info.item()) == 0 and float(ld.item()) == 0.0


def test_rhs_chunks_bitwise(gpu):
    """Each column of X depends only on its own column of B."""
    n, nrhs, T = 520, 40, 128
    A = spdgen.make_A(n, "f64", 0.5, 9, device="cuda")
    B = spdgen.make_B(n, nrhs, "f64", 9, device="cuda")
    L = cm_copy(A)
    work = gpu.workspace(L.dtype, n, nrhs, T)
    info = gpu.potrf(L, T, work=work)
    Xall = cm_copy(B)
    gpu.potrs(L, Xall, T, info=info, work=work)
    parts = []
    for c0 in range(0, nrhs, 7):
        Xc = cm_copy(B[:, c0:c0 + 7])
        gpu.potrs(L, Xc, T, info=info, work=work)
        parts.append(Xc)
    torch.cuda.synchronize()
    assert torch.equal(Xall, torch.cat(parts, dim=1))


def test_binding_rejects_bad_arguments(gpu):
    A = spdgen.make_A(8, "f64", 0.5, 0, device="cuda")
    with pytest.raises(ValueError):
        gpu.potrf(A[:, :7], 4)  # not square
    with pytest.raises(ValueError, match="argument 5"):
        gpu.potrf(A, 0)  # T_A < 1
    with pytest.raises(ValueError):
        gpu.potrf(torch.empty(8, 8, device="cuda", dtype=torch.float64), 4)  # row-major storage


@pytest.mark.parametrize("dt,n,nrhs,T_A", [("f64", 1000, 5, 128), ("f64", 1300, 3, 128), ("f32", 1024, 4, 128),
                                           ("c128", 700, 3, 64), ("f64", 2048, 16, 256)])
def test_two_step_schedule_parity(gpu, dt, n, nrhs, T_A):
    """The two-step factorization schedule (pairs of steps share one trailing
    update of depth 2 T_A) pairs only while 32 T_A rows remain beyond a pair;
    SPD_OPT_PAIR_ROWS = 0 makes it pair every step at these sizes, with odd and
    even tile counts and a ragged last tile."""
    with gpu.options({gpu.OPT_PAIR_ROWS: 0}):
        _two_step_case(gpu, dt, n, nrhs, T_A)


def _two_step_case(gpu, dt, n, nrhs, T_A):
    A = spdgen.make_A(n, dt, 0.5, 21, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, 21, device="cuda")
    A_np, B_np = wide(A), wide(B)
    L = spdgen.to_colmajor(A)
    info = gpu.potrf(L, T_A)
    X = spdgen.to_colmajor(B)
    gpu.potrs(L, X, T_A, info=info)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    Lo, info_o = oracle.potrf(A_np)
    assert info_o == 0
    assert np.abs(np.tril(wide(L)) - Lo).max() <= L_TOL[dt] * np.abs(Lo).max()
    assert rel_err_cols(X, oracle.potrs(Lo, B_np)) <= X_TOL[dt]



def posv_check(gpu, dt, n, nrhs, T_A, seed=31, lda_pad=0):
    A = spdgen.make_A(n, dt, 0.5, seed, lda=n + lda_pad, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, seed, device="cuda")
    A_np, B_np = wide(A), wide(B)
    ld = torch.zeros(1, dtype=torch.float64, device="cuda")
    info = gpu.posv(A, B, T_A, logdet_out=ld)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    Lo, info_o = oracle.potrf(A_np)
    assert info_o == 0
    assert np.abs(np.tril(wide(A)) - Lo).max() <= L_TOL[dt] * np.abs(Lo).max()
    err = rel_err_cols(B, oracle.potrs(Lo, B_np))
    assert err <= X_TOL[dt], err
    if dt in ("f64", "c128"):
        assert logdet_rel(float(ld.item()), oracle.logdet(Lo)) <= LOGDET_TOL
    return err


@pytest.mark.parametrize("dt,n,nrhs,T_A,pad", [("f64", 1000, 5, 128, 0), ("f64", 1300, 33, 128, 3),
                                               ("f64", 2048, 16, 256, 0), ("f32", 1024, 4, 128, 0),
                                               ("c128", 700, 3, 64, 0), ("c128", 1300, 17, 256, 5),
                                               ("c64", 1000, 5, 128, 3), ("f64", 300, 2, 100, 0),
                                               ("f64", 600, 130, 128, 0)])
def test_posv_parity(gpu, dt, n, nrhs, T_A, pad):
    """spd_posv against the oracle: the fused path (T_A a multiple of the
    trailing-update tile, three or more tiles; block-update substitutions for
    real types, the general product for complex ones) and the fallback to the
    three calls."""
    posv_check(gpu, dt, n, nrhs, T_A, lda_pad=pad)


@pytest.mark.parametrize("dt,n,nrhs,T_A", [("f64", 1300, 9, 128), ("f64", 1024, 3, 128)])
def test_posv_paired_steps(gpu, dt, n, nrhs, T_A):
    """With every step paired, the forward substitution follows the tiles as
    the pairs finish them."""
    with gpu.options({gpu.OPT_PAIR_ROWS: 0}):
        posv_check(gpu, dt, n, nrhs, T_A)


def test_posv_failed_factorization(gpu):
    n, T_A = 1000, 128
    A = spdgen.make_A(n, "f64", 0.5, 5, device="cuda")
    A[700, 700] = -1.0
    B = spdgen.make_B(n, 3, "f64", 5, device="cuda")
    ld = torch.zeros(1, dtype=torch.float64, device="cuda")
    info = gpu.posv(A, B, T_A, logdet_out=ld)
    torch.cuda.synchronize()
    assert int(info.item()) == 701
    assert torch.isnan(B).all() and math.isnan(float(ld.item()))


def test_huge_leading_dimension(gpu):
    """A leading dimension of 7e7 elements: 64 columns of A span more than
    2^32 elements, so the trailing update must address A with 64-bit offsets
    (45 GB of device storage, 160 x 160 of it used)."""
    posv_check(gpu, "f32", 160, 3, 64, lda_pad=70_000_000 - 160)
