"""GPU parity of the Cholesky-based reduction of a Hermitian-definite
generalized eigenproblem to standard form (page "Differentiable Generalized
Eigenvalue Decomposition", section "API Reference": types 1-3), through the
C ABI, against the CPU oracle.

C = L^-1 A L^-H (itype 1) or L^H A L (itypes 2, 3) with B = L L^H.  The GPU's
L comes from spd_potrf, the oracle's from its own potrf of the same B.
Tolerance: the lower triangle of C, Frobenius norm of the difference over
that of the oracle's C, within the substitution tolerance of the working
precision (1e-9 double, 1e-3 single; B has condition number below 10, so the
reduction amplifies rounding by less than 100).  At the full size the checks
are the identity L C L^H = A (itype 1) on the whole matrix and the definition
C_ij = l_i^T A l_j on sampled entries (itype 2), both within 64 n eps of the
scale of the matrix, in double.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import spdgen
from helpers import EPS, X_TOL, wide

pytestmark = pytest.mark.gpu


def lower_rel_err(c, cref) -> float:
    d = np.tril(wide(c) - cref)
    return float(np.linalg.norm(d) / np.linalg.norm(np.tril(cref)))


def run(gpu, itype, dt, n, T_A, pad=0, seed=3):
    B = spdgen.make_A(n, dt, 0.5, seed, device="cuda")
    A = spdgen.make_herm(n, dt, seed + 1, lda=n + pad, device="cuda", pad_value=-7.25)
    A_np, B_np = wide(A), wide(B)
    L = spdgen.to_colmajor(B)
    info = gpu.potrf(L, T_A)
    before = A.as_strided((n + pad, n), (1, n + pad)).clone()
    gpu.sygst(itype, A, L, T_A, info=info)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    after = A.as_strided((n + pad, n), (1, n + pad))
    # the strict upper triangle and the padding rows are never written
    keep = torch.ones((n + pad, n), dtype=torch.bool, device="cuda")
    keep[:n, :] = torch.triu(keep[:n, :], 1)
    assert torch.equal(after[keep], before[keep])
    Lo, info_o = oracle.potrf(B_np)
    assert info_o == 0
    Co = oracle.sygst(itype, A_np, Lo)
    err = lower_rel_err(A, Co)
    print(f"sygst itype={itype} {dt} n={n} T_A={T_A} pad={pad}: rel err {err:.2e}", flush=True)
    assert err <= X_TOL[dt]
    if dt in ("c128", "c64"):
        assert torch.all(torch.diagonal(A).imag == 0)  # C is Hermitian: real diagonal


# (1000, 128) and (1000, 256) also cover the ordering of the packed L panels
# against the one-block lookahead of the final substitution (type 1)
SHAPES = [("f64", 1, 8, 0), ("f64", 33, 32, 0), ("f64", 300, 64, 3), ("f64", 1000, 256, 0), ("f64", 1000, 128, 0),
          ("f64", 777, 100, 5), ("f32", 518, 128, 0), ("f32", 200, 64, 2), ("c128", 300, 100, 1), ("c64", 130, 64, 0)]


@pytest.mark.parametrize("itype", [1, 2, 3])
@pytest.mark.parametrize("dt,n,T_A,pad", SHAPES)
def test_sygst_parity(gpu, itype, dt, n, T_A, pad):
    run(gpu, itype, dt, n, T_A, pad)


@pytest.mark.parametrize("itype", [1, 2])
def test_sygst_failed_factor_gives_nan(gpu, itype):
    n, T_A = 200, 64
    B = spdgen.make_A(n, "f64", 0.5, 5, device="cuda")
    B[150, 150] = -1.0  # not positive definite from column 150 on
    A = spdgen.make_herm(n, "f64", 6, device="cuda")
    L = spdgen.to_colmajor(B)
    info = gpu.potrf(L, T_A)
    before = A.clone()
    gpu.sygst(itype, A, L, T_A, info=info)
    torch.cuda.synchronize()
    assert int(info.item()) > 0
    low = torch.tril(torch.ones(n, n, dtype=torch.bool, device="cuda"))
    assert torch.all(torch.isnan(A[low]))
    assert torch.equal(A[~low], before[~low])


def test_sygst_repeatable(gpu):
    """Two calls on the same input give identical bits (fixed reduction order)."""
    n, T_A = 700, 128
    B = spdgen.make_A(n, "f64", 0.5, 8, device="cuda")
    L = spdgen.to_colmajor(B)
    info = gpu.potrf(L, T_A)
    outs = []
    for _ in range(2):
        A = spdgen.make_herm(n, "f64", 9, device="cuda")
        gpu.sygst(1, A, L, T_A, info=info)
        outs.append(A)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("itype", [1, 2])
def test_sygst_full_size(gpu, itype):
    """n = 16384, T_A = 512 in fp64 (the reduction's benchmark shape)."""
    n, T_A = 16384, 512
    B = spdgen.make_A(n, "f64", 0.5, 11, device="cuda")
    A = spdgen.make_herm(n, "f64", 12, device="cuda")
    A0 = A.clone()
    L = spdgen.to_colmajor(B)
    del B
    info = gpu.potrf(L, T_A)
    gpu.sygst(itype, A, L, T_A, info=info)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    Lt = torch.tril(L)
    C = torch.tril(A, -1)
    C = C + C.mT + torch.diag_embed(torch.diagonal(A))
    assert not torch.isnan(C).any()
    if itype == 1:
        # L C L^H must give back A
        R = Lt @ C @ Lt.mT
        A0s = torch.tril(A0, -1)
        A0s = A0s + A0s.mT + torch.diag_embed(torch.diagonal(A0))
        err = float(((R - A0s).abs().max() / A0s.abs().max()).item())
        print(f"sygst itype=1 n={n}: max |L C L^T - A| / max |A| = {err:.2e}", flush=True)
        assert err <= 64 * n * EPS["f64"]
    else:
        # sampled entries of C = L^T A L from the definition, C_ij = l_i . (A l_j)
        # with l_i the i-th column of L, in double on the host
        Ln = Lt.cpu().numpy()
        An = wide(A0)
        An = np.tril(An, -1) + np.tril(An, -1).T + np.diag(np.diag(An))
        Cn = C.cpu().numpy()
        rng = np.random.default_rng(0)
        idx = [(0, 0), (n - 1, n - 1), (n - 1, 0), (5000, 123)]
        idx += [tuple(sorted(rng.integers(0, n, 2).tolist(), reverse=True)) for _ in range(8)]
        scale = np.abs(Cn).max()
        for i, j in idx:
            v = Ln[:, i] @ (An @ Ln[:, j])
            assert abs(Cn[i, j] - v) <= 64 * n * EPS["f64"] * scale, (i, j, Cn[i, j], v)
