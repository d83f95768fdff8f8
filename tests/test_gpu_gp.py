"""GPU parity of the forward substitution alone and of the Gaussian-process
marginal log-likelihood (JAXMg paper, "Research Impact Statement", "Cholesky
solve (potrs)"), through the C ABI, against the CPU oracle.

The oracle's likelihood is the definition written out (a full solve, the
quadratic term as r . A^-1 r, log det from the factor); the library computes
-1/2 |L^-1 r|^2 - sum log L_ii - (n/2) log 2 pi.  Tolerance: the absolute
difference must be within TOL x (|quadratic term|/2 + |log det|/2 +
(n/2) log 2 pi), TOL = 1e-10 in fp64 and 1e-3 in fp32 (the scale of the terms,
so that cancellation between them cannot hide or inflate an error).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import spdgen
from helpers import X_TOL, rel_err_cols, wide

pytestmark = pytest.mark.gpu

GP_TOL = {"f64": 1e-10, "f32": 1e-3}


def factor(spd, A, T_A):
    L = spdgen.to_colmajor(A)
    info = spd.potrf(L, T_A)
    return L, info


@pytest.mark.parametrize("dt,n,nrhs,T_A", [("f64", 256, 1, 64), ("f64", 333, 6, 64), ("f64", 1000, 16, 256),
                                           ("f64", 777, 3, 100), ("f32", 518, 64, 512), ("f32", 300, 9, 128),
                                           ("c128", 300, 4, 100), ("c64", 130, 4, 64)])
def test_forward_solve_parity(gpu, dt, n, nrhs, T_A):
    A = spdgen.make_A(n, dt, 0.5, 7, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, 7, device="cuda")
    A_np, B_np = wide(A), wide(B)
    L, info = factor(gpu, A, T_A)
    Y = spdgen.to_colmajor(B)
    gpu.forward_solve(L, Y, T_A, info=info)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    Lo, info_o = oracle.potrf(A_np)
    assert info_o == 0
    Yo = oracle.forward_solve(Lo, B_np)
    err = rel_err_cols(Y, Yo)
    print(f"{dt} n={n} nrhs={nrhs} T_A={T_A}: forward solve rel err {err:.2e}")
    assert err <= X_TOL[dt]
    # and the other half of potrs on top of it gives the full solve
    Xo = oracle.potrs(Lo, B_np)
    X = spdgen.to_colmajor(B)
    gpu.potrs(L, X, T_A, info=info)
    torch.cuda.synchronize()
    assert rel_err_cols(X, Xo) <= X_TOL[dt]


def gp_check(gpu, dt, n, nrhs, T_A, delta, seed):
    A = spdgen.make_A(n, dt, delta, seed, device="cuda")
    Rm = spdgen.make_B(n, nrhs, dt, seed + 1, device="cuda")
    A_np, R_np = wide(A), wide(Rm)
    L, info = factor(gpu, A, T_A)
    Rc = spdgen.to_colmajor(Rm)
    out = gpu.gp_loglik(L, Rc, T_A, info=info)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    v = out.cpu().numpy()
    vo, info_o = oracle.gp_loglik(A_np, R_np)
    assert info_o == 0
    Lo, _ = oracle.potrf(A_np)
    quad = np.einsum("ij,ij->j", R_np, oracle.potrs(Lo, R_np))
    scale = 0.5 * np.abs(quad) + 0.5 * abs(oracle.logdet(Lo)) + 0.5 * n * math.log(2 * math.pi)
    err = np.max(np.abs(v - vo) / scale)
    print(f"{dt} n={n} nrhs={nrhs} T_A={T_A} delta={delta}: loglik scaled err {err:.2e}")
    assert err <= GP_TOL[dt]
    # R now holds L^-1 R
    assert rel_err_cols(Rc, oracle.forward_solve(Lo, R_np)) <= X_TOL[dt]


@pytest.mark.parametrize("dt,n,nrhs,T_A,delta", [("f64", 256, 1, 64, 1.0), ("f64", 4096, 16, 256, 0.1),
                                                 ("f64", 1000, 33, 100, 0.5), ("f64", 2049, 5, 512, 0.05),
                                                 ("f32", 1024, 8, 128, 1.0), ("f32", 777, 3, 64, 0.5)])
def test_gp_loglik_parity(gpu, dt, n, nrhs, T_A, delta):
    gp_check(gpu, dt, n, nrhs, T_A, delta, seed=3)


def test_gp_loglik_diagonal_full_size(gpu):
    """At the full benchmark size (N = 32768, 128 columns, T_A = 512) on a
    diagonal A the likelihood has a closed form: -1/2 sum r_i^2 / d_i -
    1/2 sum log d_i - (N/2) log 2 pi."""
    n, nrhs, T = 32768, 128, 512
    g = torch.Generator(device="cpu").manual_seed(5)
    d = 0.5 + torch.rand(n, generator=g, dtype=torch.float64)
    Rm = torch.randn(n, nrhs, generator=g, dtype=torch.float64)
    A = torch.diag(d.cuda())
    L, info = factor(gpu, A, T)
    del A
    Rc = spdgen.to_colmajor(Rm.cuda())
    out = gpu.gp_loglik(L, Rc, T, info=info).cpu().numpy()
    assert int(info.item()) == 0
    dn, rn = d.numpy(), Rm.numpy()
    quad = (rn ** 2 / dn[:, None]).sum(axis=0)
    ref = -0.5 * quad - 0.5 * np.log(dn).sum() - 0.5 * n * math.log(2 * math.pi)
    scale = 0.5 * quad + 0.5 * abs(np.log(dn).sum()) + 0.5 * n * math.log(2 * math.pi)
    assert np.max(np.abs(out - ref) / scale) <= 1e-12


def test_gp_loglik_deterministic_and_nan_on_failure(gpu):
    n, nrhs, T = 700, 4, 128
    A = spdgen.make_A(n, "f64", 0.2, 9, device="cuda")
    Rm = spdgen.make_B(n, nrhs, "f64", 10, device="cuda")
    L, info = factor(gpu, A, T)
    o1 = gpu.gp_loglik(L, spdgen.to_colmajor(Rm), T, info=info).clone()
    o2 = gpu.gp_loglik(L, spdgen.to_colmajor(Rm), T, info=info).clone()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int64), o2.view(torch.int64))
    # a matrix that is not positive definite: every value is NaN, as in the oracle
    A2 = A.clone()
    A2[100, 100] = -1.0
    L2, info2 = factor(gpu, A2, T)
    R2 = spdgen.to_colmajor(Rm)
    o3 = gpu.gp_loglik(L2, R2, T, info=info2).cpu()
    assert int(info2.item()) == 101
    assert torch.isnan(o3).all() and torch.isnan(R2).all()
    vo, info_o = oracle.gp_loglik(wide(A2), wide(Rm))
    assert info_o == 101 and np.isnan(vo).all()


def test_gp_loglik_rejects_complex(gpu):
    A = spdgen.make_A(64, "c128", 1.0, 1, device="cuda")
    L, info = factor(gpu, A, 64)
    with pytest.raises(Exception):
        gpu.gp_loglik(L, spdgen.to_colmajor(spdgen.make_B(64, 1, "c128", 1, device="cuda")), 64, info=info)
