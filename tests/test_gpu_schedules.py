"""GPU parity of the alternative factorization schedules.

The library reads SPD_LOOKAHEAD (0: the sequential schedule, every kernel on
the caller's stream) and SPD_TWO_STEP (0: one-step lookahead instead of the
paired-step schedule) once per process, so each setting runs in a child
process: potrf, log det and potrs through the one-call entry point (which
falls back to the three calls when its fused path is off) on small real and
complex inputs, checked against the oracle on the same bytes.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import numpy as np
import torch
import cholesky_spd_solve_amd as spd
import oracle
import spdgen
from helpers import L_TOL, LOGDET_TOL, X_TOL, logdet_rel, rel_err_cols, wide

for dt, n, nrhs, T in [("f64", 1000, 5, 128), ("f64", 1300, 7, 256), ("f64", 2100, 3, 128),
                       ("f32", 1024, 4, 128), ("c128", 700, 3, 64)]:
    print("case", dt, n, nrhs, T, flush=True)
    A = spdgen.make_A(n, dt, 0.5, 7, device="cuda")
    B = spdgen.make_B(n, nrhs, dt, 7, device="cuda")
    A_np, B_np = wide(A), wide(B)
    L, X = spdgen.to_colmajor(A), spdgen.to_colmajor(B)
    ld = torch.zeros(1, dtype=torch.float64, device="cuda")
    info = spd.posv(L, X, T, logdet_out=ld)
    torch.cuda.synchronize()
    assert int(info.item()) == 0, dt
    Lo, info_o = oracle.potrf(A_np)
    assert info_o == 0
    assert np.abs(np.tril(wide(L)) - Lo).max() <= L_TOL[dt] * np.abs(Lo).max(), (dt, n)
    assert rel_err_cols(X, oracle.potrs(Lo, B_np)) <= X_TOL[dt], (dt, n)
    if dt in ("f64", "c128"):
        assert logdet_rel(float(ld.item()), oracle.logdet(Lo)) <= LOGDET_TOL, (dt, n)
print("ok", flush=True)
"""


@pytest.mark.parametrize("env", [{"SPD_LOOKAHEAD": "0"}, {"SPD_TWO_STEP": "0"}], ids=["sequential", "one-step"])
def test_schedule_parity(gpu, env):
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, **env), capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0 and r.stdout.rstrip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]
