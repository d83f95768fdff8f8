"""GPU parity of the one-launch diagonal tile (tile_kernel).

Each diagonal tile of the factorization is factored and inverted by one
launch whose workgroups own 64 x 64 blocks and wait for each other's blocks
through flags.  These tests compare it with the oracle on tiles of one to
sixteen blocks, with short last blocks and short last tiles, through the
one-call solve (which applies the tile inverses it builds) and the three
calls, launched both with and without CU-holding workgroups
(SPD_OPT_TILE_HOLD_ROWS); they check the previous launch sequence
(SPD_OPT_TILE_LAUNCH = 0) the same way, a failing pivot in every block position of a tile, and the bounded
wait: with a zero time limit the launch gives up at once, reports info = -1
and clears its flags, so the next call on the same workspace is exact again.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import spdgen
from helpers import L_TOL, LOGDET_TOL, X_TOL, logdet_rel, rel_err_cols, wide

pytestmark = pytest.mark.gpu

# (dtype, n, nrhs, T): one-block tiles, short last blocks (T = 100, 1000),
# short last tiles, and up to 16 blocks per tile
CASES = [("f64", 300, 3, 64), ("f64", 333, 4, 100), ("f64", 900, 5, 192), ("f64", 1100, 6, 320),
         ("f64", 1500, 7, 512), ("f64", 2100, 3, 1000), ("f32", 777, 5, 100), ("f32", 1300, 6, 512),
         ("f32", 1030, 2, 1024), ("c128", 333, 2, 100), ("c128", 1100, 3, 256), ("c128", 700, 2, 512),
         ("c64", 900, 4, 256), ("c64", 530, 3, 192)]


def solve_one_call(spd, A, B, T, work=None):
    L, X = spdgen.to_colmajor(A), spdgen.to_colmajor(B)
    ld = torch.zeros(1, dtype=torch.float64, device="cuda")
    info = spd.posv(L, X, T, logdet_out=ld, work=work)
    torch.cuda.synchronize()
    return int(info.item()), L, X, float(ld.item())


def solve_three_calls(spd, A, B, T):
    L, X = spdgen.to_colmajor(A), spdgen.to_colmajor(B)
    n, nrhs = B.shape
    work = spd.workspace(L.dtype, n, nrhs, T)
    info = spd.potrf(L, T, work=work)
    ld = spd.logdet(L, info)
    spd.potrs(L, X, T, info=info, work=work)
    torch.cuda.synchronize()
    return int(info.item()), L, X, float(ld.item())


def check(dt, n, A, B, res):
    info, L, X, ld = res
    assert info == 0, (dt, n)
    Lo, info_o = oracle.potrf(wide(A))
    assert info_o == 0
    assert np.abs(np.tril(wide(L)) - Lo).max() <= L_TOL[dt] * np.abs(Lo).max(), (dt, n)
    assert rel_err_cols(X, oracle.potrs(Lo, wide(B))) <= X_TOL[dt], (dt, n)
    if dt in ("f64", "c128"):
        assert logdet_rel(ld, oracle.logdet(Lo)) <= LOGDET_TOL, (dt, n)


@pytest.mark.parametrize("launch,hold", [(1, 8192), (1, 0), (0, 8192)])
@pytest.mark.parametrize("dt,n,nrhs,T", CASES)
def test_tile_parity(gpu, launch, hold, dt, n, nrhs, T):
    """hold 8192 (the default): every tile of these sizes is launched with
    CU-holding workgroups (real types); hold 0: never."""
    A = spdgen.make_A(n, dt, 0.5, 11, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, 11, device="cuda")
    with gpu.options({gpu.OPT_TILE_LAUNCH: launch, gpu.OPT_TILE_HOLD_ROWS: hold}):
        check(dt, n, A, B, solve_one_call(gpu, A, B, T))
        check(dt, n, A, B, solve_three_calls(gpu, A, B, T))


@pytest.mark.parametrize("dt", ["f64", "f32", "c128"])
@pytest.mark.parametrize("j", [0, 17, 64, 130, 255, 300, 511, 512, 700])
def test_tile_info(gpu, dt, j):
    """A pivot that is not positive in any block of a 8-block tile (first,
    inner, last column of a block; first column of the second tile) stops the
    factorization at the oracle's column; the solve then gives NaN."""
    n, T = 1100, 512
    A = spdgen.make_A(n, dt, 0.5, 12, device="cuda")
    A[j, j] = -1.0
    _, info_o = oracle.potrf(wide(A))
    B = spdgen.make_B(n, 2, dt, 12, device="cuda")
    info, _, X, ld = solve_one_call(gpu, A, B, T)
    assert info == info_o == j + 1
    assert math.isnan(ld) and torch.isnan(torch.view_as_real(X) if X.is_complex() else X).all()
    info3, _, _, _ = solve_three_calls(gpu, A, B, T)
    assert info3 == j + 1


def test_tile_wait_limit(gpu):
    """With a zero wait limit the launch gives up at its first wait: info is
    -1, the solution NaN; every workgroup still counts itself out, so the
    flags are clear and the next call on the same workspace is exact."""
    dt, n, nrhs, T = "f64", 1500, 3, 512
    A = spdgen.make_A(n, dt, 0.5, 13, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, 13, device="cuda")
    work = gpu.workspace(torch.float64, n, nrhs, T)
    with gpu.options({gpu.OPT_TILE_WAIT_US: 0}):
        info, _, X, ld = solve_one_call(gpu, A, B, T, work=work)
    assert info == -1
    assert math.isnan(ld) and torch.isnan(X).all()
    check(dt, n, A, B, solve_one_call(gpu, A, B, T, work=work))
