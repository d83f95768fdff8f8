"""Accuracy of the pivot square root and reciprocal square root of the leaf
factorization, through the public factorization.

The leaf takes L_jj = sqrt(d) and scales column j by 1/sqrt(d) with
Goldschmidt's coupled iteration (after an exact power-of-four scaling of d
into [1/2, 2) and the hardware reciprocal-square-root estimate).  A
block-diagonal A of 2 x 2 blocks [[d, e], [e, 4]], with e a power of two near
sqrt(d), exposes both results exactly: L(2i, 2i) is the computed sqrt(d) and
L(2i+1, 2i) = e / sqrt(d) is the computed reciprocal times a power of two
(exact).  They are compared with the correctly rounded values (computed in
50-digit decimal arithmetic) over pivots spread log-uniformly across the
whole exponent range of the working precision, including subnormal pivots in
the first tile.  The bound asserted is the one the leaf's design states:
within 2 units in the last place for double and single precision.
"""
from __future__ import annotations

import decimal

import numpy as np
import pytest
import torch

import spdgen

pytestmark = pytest.mark.gpu

ULP_BOUND = 2.0
D = decimal.Decimal


def pivots(dt, count, seed):
    rng = np.random.default_rng(seed)
    if dt == "f64":
        lo, hi, sub = -1000.0, 1000.0, [5e-324, 1e-310, 2.0**-1030]
        ftype = np.float64
    else:
        lo, hi, sub = -120.0, 120.0, [1.4e-45, 1e-40, 2.0**-130]
        ftype = np.float32
    d = np.exp2(rng.uniform(lo, hi, count)).astype(ftype)
    d[: len(sub)] = np.array(sub, dtype=ftype)  # subnormal pivots, in the first tile
    d[len(sub): len(sub) + 4] = np.array([1.0, 2.0, 0.5, 4.0], dtype=ftype)
    return d


def ulps(got: np.ndarray, exact: list, ftype) -> np.ndarray:
    """|got - exact| in units of the last place of the correctly rounded exact value."""
    out = np.empty(len(got))
    for i, (g, x) in enumerate(zip(got, exact)):
        ref = ftype(float(x))
        u = float(np.spacing(ref))
        out[i] = float(abs(D(float(g)) - x) / D(u))
    return out


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_pivot_sqrt_and_reciprocal_within_two_ulps(gpu, dt):
    decimal.getcontext().prec = 50
    tdt = torch.float64 if dt == "f64" else torch.float32
    ftype = np.float64 if dt == "f64" else np.float32
    worst_s, worst_r = 0.0, 0.0
    for call in range(4):
        P = 4096
        n = 2 * P
        d = pivots(dt, P, 100 + call)
        # e = 2^round(log2(d) / 2): e^2 / d in [1/2, 2], so the second pivot 4 - e^2 / d stays in [2, 3.5]
        k = np.round(np.log2(d.astype(np.float64)) / 2.0).astype(np.int64)
        e = np.ldexp(1.0, k).astype(ftype)
        A = torch.zeros(n, n, dtype=tdt, device="cuda")
        idx = torch.arange(0, n, 2, device="cuda")
        A[idx, idx] = torch.from_numpy(d).cuda()
        A[idx + 1, idx] = torch.from_numpy(e).cuda()
        A[idx, idx + 1] = torch.from_numpy(e).cuda()
        A[idx + 1, idx + 1] = 4.0
        L = spdgen.to_colmajor(A)
        info = gpu.potrf(L, 512)
        torch.cuda.synchronize()
        assert int(info.item()) == 0
        sq = L[idx, idx].cpu().numpy()
        rs = (L[idx + 1, idx].cpu().numpy() / e).astype(ftype)  # division by a power of two: exact
        exact_s = [D(float(x)).sqrt() for x in d]
        exact_r = [1 / s for s in exact_s]
        us, ur = ulps(sq, exact_s, ftype), ulps(rs, exact_r, ftype)
        worst_s, worst_r = max(worst_s, us.max()), max(worst_r, ur.max())
        assert us.max() <= ULP_BOUND, (dt, d[int(us.argmax())], us.max())
        assert ur.max() <= ULP_BOUND, (dt, d[int(ur.argmax())], ur.max())
    print(f"{dt}: sqrt within {worst_s:.3f} ulp, 1/sqrt within {worst_r:.3f} ulp over {4 * 4096} pivots", flush=True)
