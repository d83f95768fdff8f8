"""The five benchmark workloads against the oracle, element by element.

Every workload runs through both forms of the solve: the one-call entry point
(spd_posv: the factorization with the forward substitution beside it, log
det, the back substitution) and the three calls (spd_potrf, spd_logdet,
spd_potrs).  Each is compared with the CPU oracle run on exactly the same
input bytes (widened to double for the fp32 workload):

  - the whole factor L (lower triangle), max |L - L_oracle| / max |L_oracle|;
  - x in every right-hand-side column, ||x - x_oracle||_2 / ||x_oracle||_2
    (1e-9 for fp64 / complex128, 1e-3 for fp32);
  - log det, 1e-11 relative (fp64 / complex128 workloads, which request it);
  - the normwise backward error of x, 64 N eps of the working precision.

The oracle at N = 32768 is an unblocked left-looking factorization streaming
about 47 TB through the host's memory: several minutes.  It is taken in equal-
work ranges of columns, one test item per range, so that each item reports as
it finishes; the comparison items compute whatever ranges have not run yet,
so any of them can also run alone.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import spdgen
from helpers import EPS, L_TOL, LOGDET_TOL, X_TOL, backward_error, logdet_rel, rel_err_cols, wide

pytestmark = pytest.mark.gpu


def run_gpu(spd, A0, B0, T, mode, want_logdet):
    """Solve on fresh column-major copies; returns (L, X, logdet, info)."""
    L = spdgen.to_colmajor(A0)
    X = spdgen.to_colmajor(B0)
    n, nrhs = X.shape
    work = spd.workspace(L.dtype, n, nrhs, T)
    ld = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    if mode == "posv":
        info = spd.posv(L, X, T, logdet_out=ld if want_logdet else None, work=work)
    else:
        info = spd.potrf(L, T, work=work)
        if want_logdet:
            spd.logdet(L, info, out=ld)
        spd.potrs(L, X, T, info=info, work=work)
    torch.cuda.synchronize()
    return L, X, (float(ld.item()) if want_logdet else None), int(info.item())


def compare(spd, k, mode, A0, B0, Lo, Xo, ldo):
    c = spdgen.CONFIGS[k]
    dt, n, T = c["dtype"], c["n"], c["T_A"]
    L, X, ld, info = run_gpu(spd, A0, B0, T, mode, c["logdet"])
    assert info == 0
    # the whole factor, on the GPU (the oracle's row-major L uploaded once)
    wd = torch.complex128 if Lo.is_complex() else torch.float64
    diff = (torch.tril(L).to(wd) - Lo).abs().max().item()
    err_L = diff / Lo.abs().max().item()
    del L
    err_x = rel_err_cols(X, Xo)
    eta = backward_error(A0, X, B0)
    msg = f"config {k} {mode}: L {err_L:.2e} x {err_x:.2e} eta {eta:.2e}"
    if ld is not None:
        err_ld = logdet_rel(ld, ldo)
        msg += f" logdet {ld:.12g} vs {ldo:.12g} ({err_ld:.2e})"
    print(msg, flush=True)
    assert err_L <= L_TOL[dt], msg
    assert err_x <= X_TOL[dt], msg
    assert eta <= 64 * n * EPS[dt], msg
    if ld is not None:
        assert err_ld <= LOGDET_TOL, msg


class Workload:
    """Inputs of one workload on the GPU and the oracle's results for them."""

    def __init__(self, k, parts=1):
        c = spdgen.CONFIGS[k]
        self.k = k
        self.A0, self.B0, _ = spdgen.make_config(k, 0, device="cuda")
        torch.cuda.synchronize()
        # A is exactly symmetric (Hermitian), so its column-major storage read
        # row-major is A^T = conj(A): the oracle reads the lower triangle of
        # the row-major array it is given, so hand it the transpose view
        # (complex: conjugated) to read A itself without another copy
        a = self.A0.cpu().numpy()
        a = a.T if not np.iscomplexobj(a) else np.conj(a.T)
        self.fact = oracle.Factorization(a)
        self.bounds = oracle.Factorization.equal_work_bounds(c["n"], parts)
        self._results = None

    def advance(self, part):
        info = self.fact.advance(self.bounds[part])
        assert info == 0
        print(f"config {self.k}: oracle columns up to {self.fact.next} of {self.fact.n}", flush=True)

    def results(self):
        """(L_oracle on the GPU, X_oracle, logdet_oracle)"""
        if self._results is None:
            assert self.fact.advance(self.fact.n) == 0
            lo = self.fact.l
            xo = oracle.potrs(lo, wide(self.B0))
            ldo = oracle.logdet(lo)
            self.fact.a = None  # free the host copy of A
            self._results = (torch.from_numpy(lo).cuda(), xo, ldo)
            self.fact.l = None
        return self._results


@pytest.fixture(scope="module")
def config3():
    return Workload(3)


@pytest.fixture(scope="module")
def config4():
    return Workload(4)


CONFIG5_PARTS = 12


@pytest.fixture(scope="module")
def config5():
    return Workload(5, CONFIG5_PARTS)


@pytest.mark.parametrize("mode", ["posv", "three-calls"])
def test_config3_fp32_n16384(gpu, config3, mode):
    """fp32, N = 16384, N_RHS = 64, T_A = 512 (x only; the oracle in double on
    the same fp32 bytes)."""
    compare(gpu, 3, mode, config3.A0, config3.B0, *config3.results())


@pytest.mark.parametrize("mode", ["posv", "three-calls"])
def test_config4_c128_n8192(gpu, config4, mode):
    """complex128, N = 8192, N_RHS = 32, T_A = 256, with log det."""
    compare(gpu, 4, mode, config4.A0, config4.B0, *config4.results())


@pytest.mark.parametrize("part", range(CONFIG5_PARTS))
def test_config5_oracle_columns(gpu, config5, part):
    """The oracle's factorization of the N = 32768 workload, one equal-work
    range of columns per item."""
    config5.advance(part)


@pytest.mark.parametrize("mode", ["posv", "three-calls"])
def test_config5_fp64_n32768(gpu, config5, mode):
    """fp64, N = 32768, N_RHS = 128, T_A = 512 (the benchmark's workload),
    with log det."""
    compare(gpu, 5, mode, config5.A0, config5.B0, *config5.results())
