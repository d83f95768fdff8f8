"""Shared test helpers: tolerances and error measures for parity checks.

Tolerances (per working precision):
  fp64 / c128 : relative error of x <= 1e-9 (per right-hand-side column,
                2-norm, worst column), log det <= 1e-11 relative, normwise
                backward error <= 64 n eps
  fp32 / c64  : relative error of x <= 1e-3 against the double-precision
                oracle run on the same (exactly widened) input, backward error
                <= 64 n eps(float32)
The factor L has no stated tolerance; it is compared as max |L_gpu - L_ref| /
max |L_ref| <= 1e-10 (double) or 1e-3 (single): for these inputs
(condition numbers below 100) the factor's perturbation is of order
kappa * n * eps, far inside both.
"""
from __future__ import annotations

import math

import numpy as np
import torch

X_TOL = {"f64": 1e-9, "c128": 1e-9, "f32": 1e-3, "c64": 1e-3}
L_TOL = {"f64": 1e-10, "c128": 1e-10, "f32": 1e-3, "c64": 1e-3}
LOGDET_TOL = 1e-11
EPS = {"f64": 2.0**-52, "c128": 2.0**-52, "f32": 2.0**-23, "c64": 2.0**-23}
TORCH = {"f32": torch.float32, "f64": torch.float64, "c64": torch.complex64, "c128": torch.complex128}


def dtype_name(t: torch.dtype) -> str:
    return {v: k for k, v in TORCH.items()}[t]


def wide(x) -> np.ndarray:
    x = x.detach().cpu().numpy() if isinstance(x, torch.Tensor) else np.asarray(x)
    return x.astype(np.complex128 if np.iscomplexobj(x) else np.float64)


def rel_err_cols(x, xref) -> float:
    """max over columns of ||x - xref||_2 / ||xref||_2"""
    x, xref = wide(x), wide(xref)
    if x.ndim == 1:
        x, xref = x[:, None], xref[:, None]
    num = np.linalg.norm(x - xref, axis=0)
    den = np.linalg.norm(xref, axis=0)
    return float(np.max(num / np.where(den == 0, 1.0, den))) if x.size else 0.0


def backward_error(A, x, b) -> float:
    """Rigal-Gaches normwise backward error, worst column, in double precision:
    ||b - A x||_inf / (||A||_inf ||x||_inf + ||b||_inf).  A, x, b may be CPU or
    GPU tensors / arrays (GPU: the residual uses torch's own matmul)."""
    if isinstance(A, torch.Tensor) and A.is_cuda:
        wd = torch.complex128 if A.is_complex() else torch.float64
        Aw, xw, bw = A.to(wd), x.to(wd), b.to(wd)
        if xw.dim() == 1:
            xw, bw = xw[:, None], bw[:, None]
        r = bw - Aw @ xw
        nA = Aw.abs().sum(dim=1).max()
        eta = r.abs().amax(dim=0) / (nA * xw.abs().amax(dim=0) + bw.abs().amax(dim=0))
        return float(eta.max().item())
    A, x, b = wide(A), wide(x), wide(b)
    if x.ndim == 1:
        x, b = x[:, None], b[:, None]
    r = b - A @ x
    nA = np.abs(A).sum(axis=1).max()
    eta = np.abs(r).max(axis=0) / (nA * np.abs(x).max(axis=0) + np.abs(b).max(axis=0))
    return float(eta.max())


def logdet_rel(a: float, ref: float) -> float:
    if math.isnan(a) or math.isnan(ref):
        return math.inf
    return abs(a - ref) / max(abs(ref), 1e-300)


def lower(x: np.ndarray) -> np.ndarray:
    return np.tril(x)
