"""Every kernel variant of the large workloads, element by element against
the oracle, at sizes the oracle finishes in seconds.

The tile shapes and schedules switch with the problem's size (128-row
trailing-update tiles from about 512 of them, deeper operand slices for large
orders, paired steps while many rows remain, 64-row substitution tiles for
tall block updates).  The schedule options move those switches, so each
variant the N = 16384 / 32768 workloads run is reached here at N = 8192 and
compared with the oracle on the same bytes, through the one-call solve and
the three calls:

  default            fp64: 128 x 128 trailing-update tiles with 8-deep
                     slices, one step at a time; 32-row substitution tiles
  pairs              every step paired (the two-panel update of depth 2 T_A)
  deep + tall        also 16-deep (fp64) / 32-deep (fp32) slices and 64-row
                     substitution and panel-product tiles everywhere

plus a ragged order (N = 8191, last tile 511 wide) and complex64 at N = 8192,
and a large ragged order (N = 30001) checked on the outputs the oracle can
compute there in seconds.
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

_cache = {}


def inputs(dt, n, nrhs, delta, seed):
    """GPU inputs and the oracle's (L, X, logdet) on them, computed once."""
    key = (dt, n, nrhs, delta, seed)
    if key not in _cache:
        A0 = spdgen.make_A(n, dt, delta, seed, device="cuda")
        B0 = spdgen.make_B(n, nrhs, dt, seed, device="cuda")
        Lo, info = oracle.potrf(wide(A0))
        assert info == 0
        Xo = oracle.potrs(Lo, wide(B0))
        _cache.clear()  # one input set alive at a time
        _cache[key] = (A0, B0, torch.from_numpy(Lo).cuda(), Xo, oracle.logdet(Lo))
    return _cache[key]


def solve_and_compare(spd, dt, n, nrhs, T, delta, seed, mode, opts):
    A0, B0, Lo, Xo, ldo = inputs(dt, n, nrhs, delta, seed)
    L, X = spdgen.to_colmajor(A0), spdgen.to_colmajor(B0)
    ld = torch.zeros(1, dtype=torch.float64, device="cuda")
    with spd.options(opts):
        work = spd.workspace(L.dtype, n, nrhs, T)
        if mode == "posv":
            info = spd.posv(L, X, T, logdet_out=ld, work=work)
        else:
            info = spd.potrf(L, T, work=work)
            spd.logdet(L, info, out=ld)
            spd.potrs(L, X, T, info=info, work=work)
        torch.cuda.synchronize()
    assert int(info.item()) == 0
    wd = torch.complex128 if Lo.is_complex() else torch.float64
    err_L = (torch.tril(L).to(wd) - Lo).abs().max().item() / Lo.abs().max().item()
    err_x = rel_err_cols(X, Xo)
    eta = backward_error(A0, X, B0)
    err_ld = logdet_rel(float(ld.item()), ldo)
    msg = f"{dt} n={n} nrhs={nrhs} T={T} {mode} {opts}: L {err_L:.2e} x {err_x:.2e} eta {eta:.2e} ld {err_ld:.2e}"
    print(msg, flush=True)
    assert err_L <= L_TOL[dt], msg
    assert err_x <= X_TOL[dt], msg
    assert eta <= 64 * n * EPS[dt], msg
    assert err_ld <= (LOGDET_TOL if dt in ("f64", "c128") else 1e-4), msg


def variants(spd):
    return {
        "default": {},
        "pairs": {spd.OPT_PAIR_ROWS: 0},
        "deep+tall": {spd.OPT_PAIR_ROWS: 0, spd.OPT_SYRK_DEEP_ROWS: 0, spd.OPT_RECT_TALL_ROWS: 0},
    }


@pytest.mark.parametrize("mode", ["posv", "three-calls"])
@pytest.mark.parametrize("variant", ["default", "pairs", "deep+tall"])
def test_fp64_n8192_t512(gpu, variant, mode):
    solve_and_compare(gpu, "f64", 8192, 128, 512, 0.05, 3, mode, variants(gpu)[variant])


@pytest.mark.parametrize("mode", ["posv", "three-calls"])
@pytest.mark.parametrize("variant", ["default", "deep+tall"])
def test_fp32_n8192_t512(gpu, variant, mode):
    solve_and_compare(gpu, "f32", 8192, 64, 512, 1.0, 4, mode, variants(gpu)[variant])


@pytest.mark.parametrize("mode", ["posv", "three-calls"])
@pytest.mark.parametrize("variant", ["default", "pairs"])
def test_fp64_ragged_n8191_t512(gpu, variant, mode):
    """N = 8191: fifteen 512-wide tiles and a last one of 511."""
    solve_and_compare(gpu, "f64", 8191, 128, 512, 0.05, 5, mode, variants(gpu)[variant])


@pytest.mark.parametrize("mode", ["posv", "three-calls"])
def test_c64_n8192_t256(gpu, mode):
    """complex64 at the complex128 workload's shape (N = 8192, 32 right-hand
    sides, T_A = 256), against the complex128 oracle on the same bytes."""
    solve_and_compare(gpu, "c64", 8192, 32, 256, 0.5, 6, mode, {})


@pytest.mark.parametrize("mode", ["posv", "three-calls"])
def test_c128_n4096_pairs(gpu, mode):
    """Complex paired steps: the two-panel update on 64-row complex tiles."""
    solve_and_compare(gpu, "c128", 4096, 16, 256, 0.5, 7, mode, {gpu.OPT_PAIR_ROWS: 0})


def test_fp64_ragged_n30001_sampled(gpu):
    """N = 30001, T_A = 512 (58 whole tiles and a last one of 305), 128
    right-hand sides, through the one-call solve.  The oracle computes the
    leading 2 T_A columns of L exactly (they depend only on the leading
    principal block and the sampled rows); x is checked by its normwise
    backward error against the input, and log det against the oracle's
    value for the leading block plus the factor's remaining diagonal."""
    n, nrhs, T = 30001, 128, 512
    _cache.clear()
    A0 = spdgen.make_A(n, "f64", 0.05, 8, device="cuda")
    B0 = spdgen.make_B(n, nrhs, "f64", 8, device="cuda")
    L, X = spdgen.to_colmajor(A0), spdgen.to_colmajor(B0)
    ld = torch.zeros(1, dtype=torch.float64, device="cuda")
    info = gpu.posv(L, X, T, logdet_out=ld)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    K = 2 * T
    rng = np.random.default_rng(30001)
    R = np.unique(np.concatenate([rng.choice(np.arange(K, n), 96, replace=False), np.arange(n - 5, n)]))
    S = np.concatenate([np.arange(K), R])
    St = torch.from_numpy(S).cuda()
    Lo, info_o = oracle.potrf(wide(A0[St][:, St]))
    assert info_o == 0
    Lg = np.where(np.arange(len(S))[:, None] >= np.arange(K)[None, :], wide(L[St][:, :K]), 0)
    err_L = np.abs(Lg - Lo[:, :K]).max() / np.abs(Lo[:, :K]).max()
    d = wide(torch.diagonal(L))
    ld_ref = oracle.logdet(Lo[:K, :K]) + 2.0 * math.fsum(np.log(d[K:]))
    eta = backward_error(A0, X, B0)
    msg = f"n=30001: L[:, :{K}] {err_L:.2e} eta {eta:.2e} logdet {float(ld.item()):.12g} vs {ld_ref:.12g}"
    print(msg, flush=True)
    assert err_L <= L_TOL["f64"], msg
    assert eta <= 64 * n * EPS["f64"], msg
    assert logdet_rel(float(ld.item()), ld_ref) <= LOGDET_TOL, msg
