"""GPU parity of the alternative factorization schedules.

SPD_OPT_LOOKAHEAD = 0 selects the sequential schedule (every kernel on the
caller's stream) and SPD_OPT_TWO_STEP = 0 the one-step lookahead instead of
the paired-step schedule; SPD_OPT_COLUMN_FIRST_ROWS moves the point from which
the caller's update waits for the next tile column (never, or in every single
step; with SPD_OPT_PAIR_ROWS past N every step is single), and
SPD_OPT_TILE_UPDATE_ROWS the steps whose diagonal tile takes its own last
update (none, or every single step; with SPD_OPT_TILE_LAUNCH = 0 the tile is
the launch sequence, which never does); SPD_OPT_TRIPLE_ROWS the steps taken
in threes on orders of 40 tiles and more (test_step_groups).  Under each, potrf, log det and potrs run through
the one-call entry point (which falls back to the three calls when its fused
path is off) on small real and complex inputs, checked against the oracle on
the same bytes; and the auxiliary streams can be released and made again.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import spdgen
from helpers import L_TOL, LOGDET_TOL, X_TOL, logdet_rel, rel_err_cols, wide

pytestmark = pytest.mark.gpu

CASES = [("f64", 1000, 5, 128), ("f64", 1300, 7, 256), ("f64", 2100, 3, 128), ("f32", 1024, 4, 128),
         ("c128", 700, 3, 64)]


_ORACLE = {}


def oracle_solution(dt, n, nrhs, A_np, B_np):
    """The oracle's factor, solution and log det of one seeded input (the same
    bytes for every schedule of a case, so computed once)."""
    key = (dt, n, nrhs)
    if key not in _ORACLE:
        Lo, info_o = oracle.potrf(A_np)
        assert info_o == 0
        _ORACLE[key] = (Lo, oracle.potrs(Lo, B_np), oracle.logdet(Lo))
    return _ORACLE[key]


def run_case(spd, dt, n, nrhs, T):
    A = spdgen.make_A(n, dt, 0.5, 7, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, 7, device="cuda")
    A_np, B_np = wide(A), wide(B)
    L, X = spdgen.to_colmajor(A), spdgen.to_colmajor(B)
    ld = torch.zeros(1, dtype=torch.float64, device="cuda")
    info = spd.posv(L, X, T, logdet_out=ld)
    torch.cuda.synchronize()
    assert int(info.item()) == 0, dt
    Lo, Xo, ldo = oracle_solution(dt, n, nrhs, A_np, B_np)
    assert np.abs(np.tril(wide(L)) - Lo).max() <= L_TOL[dt] * np.abs(Lo).max(), (dt, n)
    assert rel_err_cols(X, Xo) <= X_TOL[dt], (dt, n)
    if dt in ("f64", "c128"):
        assert logdet_rel(float(ld.item()), ldo) <= LOGDET_TOL, (dt, n)


SCHEDULES = {
    "sequential": lambda g: {g.OPT_LOOKAHEAD: 0},
    "one-step": lambda g: {g.OPT_TWO_STEP: 0},
    "one-step, column first everywhere": lambda g: {g.OPT_TWO_STEP: 0, g.OPT_COLUMN_FIRST_ROWS: 1 << 40},
    "column first never": lambda g: {g.OPT_COLUMN_FIRST_ROWS: 0},
    "column first everywhere": lambda g: {g.OPT_COLUMN_FIRST_ROWS: 1 << 40, g.OPT_PAIR_ROWS: 1 << 40},
    "tile's own update never": lambda g: {g.OPT_TILE_UPDATE_ROWS: 0},
    "tile's own update everywhere": lambda g: {g.OPT_TILE_UPDATE_ROWS: 1 << 40, g.OPT_PAIR_ROWS: 1 << 40},
    "tile's own update, launch sequence": lambda g: {g.OPT_TILE_LAUNCH: 0},
}


@pytest.mark.parametrize("opt", list(SCHEDULES))
@pytest.mark.parametrize("dt,n,nrhs,T", CASES)
def test_schedule_parity(gpu, opt, dt, n, nrhs, T):
    values = SCHEDULES[opt](gpu)
    with gpu.options(values):
        run_case(gpu, dt, n, nrhs, T)


def test_release_and_recreate_streams(gpu):
    """spd_release waits for and destroys the auxiliary streams; the next call
    makes them again and still matches the oracle."""
    run_case(gpu, "f64", 1300, 7, 256)
    gpu.release()
    gpu.release()  # nothing left: a no-op
    run_case(gpu, "f64", 1300, 7, 256)
    gpu.release()


# (triple rows, pair rows): the default mix, threes until the last tiles then
# pairs from the start, threes then single steps, pairs only
GROUPS = [(-1, -1), (1, 0), (1, 1 << 40), (0, 0)]


@pytest.mark.parametrize("triple_rows,pair_rows", GROUPS)
@pytest.mark.parametrize("dt,n,nrhs,T", [("f64", 6001, 3, 128), ("f32", 5120, 2, 128), ("c128", 5200, 2, 128)])
def test_step_groups(gpu, dt, n, nrhs, T, triple_rows, pair_rows):
    """Orders of 40 tiles and more (47, 40, 41 here; a ragged last tile for
    fp64) keep six trailing-update panels and take steps in threes while the
    trailing matrix is large: every mix of threes, pairs and single steps
    matches the oracle."""
    with gpu.options({gpu.OPT_TRIPLE_ROWS: triple_rows, gpu.OPT_PAIR_ROWS: pair_rows}):
        run_case(gpu, dt, n, nrhs, T)
