"""GPU parity of the one-launch back substitution (subst_kernel).

L^H X = Y is solved by tile rows from the last one up; each tile row is cut
into 32-row pieces and 32- or 64-column pieces whose workgroups hand their
results to each other through flags (SPD_OPT_SUBST_LAUNCH sets the largest
n * n_rhs that takes it).  These tests force it on, and off (the block-step
path), for every dtype, ragged orders and tile sizes that are not multiples
of the 32-row pieces, one to 200 right-hand sides (one and several column
pieces, short last ones), through the one-call solve and the three calls, and
compare each with the oracle.  A zero wait limit makes a wait run out: spd_potrs
then leaves d_info alone and returns NaN, and the flags are clear for the
next call on the same workspace.
"""
from __future__ import annotations

import math

import pytest
import torch

import spdgen
from test_gpu_tile import check, solve_one_call, solve_three_calls

pytestmark = pytest.mark.gpu

ALWAYS = 1 << 50

# (dtype, n, nrhs, T)
CASES = [("f64", 300, 1, 64), ("f64", 1000, 33, 100), ("f64", 2100, 65, 512), ("f64", 1500, 128, 250),
         ("f64", 777, 200, 1000), ("f32", 1300, 7, 512), ("f32", 777, 64, 100), ("f32", 1030, 97, 256),
         ("c128", 700, 32, 256), ("c128", 513, 40, 64), ("c128", 999, 3, 300), ("c64", 900, 5, 192),
         ("c64", 650, 70, 128)]


@pytest.mark.parametrize("launch", [ALWAYS, 0])
@pytest.mark.parametrize("dt,n,nrhs,T", CASES)
def test_subst_parity(gpu, launch, dt, n, nrhs, T):
    A = spdgen.make_A(n, dt, 0.5, 21, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, 21, device="cuda")
    with gpu.options({gpu.OPT_SUBST_LAUNCH: launch}):
        check(dt, n, A, B, solve_one_call(gpu, A, B, T))
        check(dt, n, A, B, solve_three_calls(gpu, A, B, T))


def test_subst_wait_limit(gpu):
    """With a zero wait limit a wait of the launch runs out: X is NaN and
    spd_potrs's (read-only) info stays 0; the last workgroup out clears the
    flags, so the next call on the same workspace is exact."""
    dt, n, nrhs, T = "f64", 1500, 3, 100
    A = spdgen.make_A(n, dt, 0.5, 22, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, 22, device="cuda")
    L = spdgen.to_colmajor(A)
    work = gpu.workspace(torch.float64, n, nrhs, T)
    info = gpu.potrf(L, T, work=work)
    ld = gpu.logdet(L, info)
    with gpu.options({gpu.OPT_SUBST_LAUNCH: ALWAYS}):
        X = spdgen.to_colmajor(B)
        with gpu.options({gpu.OPT_TILE_WAIT_US: 0}):
            gpu.potrs(L, X, T, info=info, work=work)
        torch.cuda.synchronize()
        assert int(info.item()) == 0
        assert torch.isnan(X).all()
        X = spdgen.to_colmajor(B)
        gpu.potrs(L, X, T, info=info, work=work)
        torch.cuda.synchronize()
    check(dt, n, A, B, (int(info.item()), L, X, float(ld.item())))
    assert not math.isnan(float(ld.item()))
