"""spd_posv_noalloc, the form of spd_posv that takes its workspace from the
library's fixed per-device scratch buffer, against spd_posv itself.

Two calls in a row share the buffer: the second, on a smaller input, must not
be affected by what the first left there.  Results are compared with
spd_posv's on the same bytes to the parity tolerances (the no-alloc form runs
the sequential schedule, so its rounding order may differ from spd_posv's):
L and x per column 1e-9 relative (fp64 / complex128), log det 1e-11.  Sizes
whose workspace exceeds the buffer are rejected before anything runs.
"""
from __future__ import annotations

import math

import pytest
import torch

import spdgen
from helpers import L_TOL, LOGDET_TOL, X_TOL, logdet_rel, rel_err_cols

pytestmark = pytest.mark.gpu


def solve_both(spd, dt, n, nrhs, T, seed):
    A0 = spdgen.make_A(n, dt, 0.1, seed, device="cuda")
    B0 = spdgen.make_B(n, nrhs, dt, seed, device="cuda")
    out = {}
    for form in ("posv", "noalloc"):
        L, X = spdgen.to_colmajor(A0), spdgen.to_colmajor(B0)
        info = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        ld = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
        if form == "posv":
            spd.posv(L, X, T, info=info, logdet_out=ld)
        else:
            spd.posv_noalloc(L, X, T, info, logdet_out=ld)
        torch.cuda.synchronize()
        out[form] = (int(info.item()), torch.tril(L), X, float(ld.item()))
    (i1, L1, X1, ld1), (i2, L2, X2, ld2) = out["posv"], out["noalloc"]
    assert i1 == 0 and i2 == 0
    err_L = ((L2 - L1).abs().max() / L1.abs().max()).item()
    err_x = rel_err_cols(X2, X1)
    err_ld = logdet_rel(ld2, ld1)
    print(f"{dt} n={n} nrhs={nrhs} T={T}: L {err_L:.2e} x {err_x:.2e} logdet {err_ld:.2e}", flush=True)
    assert err_L <= L_TOL[dt] and err_x <= X_TOL[dt] and err_ld <= LOGDET_TOL
    assert math.isfinite(ld2)


def test_noalloc_matches_posv_two_calls(gpu):
    """A large call (fp64 N = 4096, 16 right-hand sides, T_A = 256: 57 MiB of
    the 64 MiB buffer), then a smaller one, then another dtype."""
    solve_both(gpu, "f64", 4096, 16, 256, 1)
    solve_both(gpu, "f64", 1000, 5, 128, 2)
    solve_both(gpu, "c128", 700, 3, 64, 3)


def test_noalloc_rejects_sizes_beyond_the_buffer(gpu):
    """N = 16384 fp32 with 64 right-hand sides needs 226 MiB: rejected with
    SPD_ERR_SCRATCH, and A, B and info are left as they were."""
    n, nrhs, T = 16384, 64, 512
    assert gpu.workspace_size(torch.float32, n, nrhs, T) > gpu.NOALLOC_SCRATCH_BYTES
    A = spdgen.to_colmajor(torch.eye(n, dtype=torch.float32, device="cuda"))
    B = spdgen.to_colmajor(torch.ones(n, nrhs, dtype=torch.float32, device="cuda"))
    info = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    lib = gpu.load()
    import ctypes
    rc = lib.spd_posv_noalloc(0, n, nrhs, ctypes.c_void_p(A.data_ptr()), n, ctypes.c_void_p(B.data_ptr()), n, T,
                              ctypes.c_void_p(info.data_ptr()), None, None)
    assert rc == gpu.SPD_ERR_SCRATCH
    assert "bytes of workspace" in lib.spd_last_error().decode()
    torch.cuda.synchronize()
    assert int(info.item()) == -7
    assert torch.equal(B, torch.ones_like(B))
    assert torch.equal(torch.diagonal(A), torch.ones(n, dtype=torch.float32, device="cuda"))
