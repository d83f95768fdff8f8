"""Seeded synthetic inputs for the dense SPD/HPD solve.

This module is shared by the oracle's tests and by the GPU path's tests and
benchmark.  It only draws random numbers and assembles the test matrices; it
holds none of the factorization, substitution or log-determinant arithmetic.

Workloads (JAXMg paper, "Performance and scaling"): the paper times its
Cholesky solve on synthetic inputs only.  The five workloads below are
random Gram matrices shifted by a multiple of the identity, so they are
symmetric (Hermitian) positive definite with a Marchenko-Pastur spectrum on
[delta, 4 + delta]:

    A = G G^H / N + delta * I,   G_ij iid N(0, 1)  (complex: (N(0,1) + i N(0,1)) / sqrt 2)
    B_ij iid with the same distribution as G_ij.

The paper's own potrs benchmark input, A = diag(1, ..., N) with b = (1, ..., 1)^T,
is also provided (:func:`diag_benchmark`).

Matrices are returned as torch tensors with *column-major* storage: a logical
(rows, cols) tensor with strides (1, ld).  Random numbers come from NumPy's
PCG64 with ``SeedSequence([seed, stream, block])``; stream 0 draws G and stream
1 draws B, so B does not depend on how G was drawn.  Row blocks of 1024 rows are
drawn from independent child streams so generation can use several threads
and still be reproducible bit for bit.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os

import numpy as np
import torch

# name -> (torch dtype, numpy dtype, is_complex)
DTYPES = {
    "f32": (torch.float32, np.float32, False),
    "f64": (torch.float64, np.float64, False),
    "c64": (torch.complex64, np.complex64, True),
    "c128": (torch.complex128, np.complex128, True),
}

# The five solve workloads: dtype, N, N_RHS, T_A, diagonal shift delta, whether
# the log-determinant is requested.
CONFIGS = {
    1: dict(dtype="f64", n=256, nrhs=1, T_A=64, delta=1.0, logdet=True),
    2: dict(dtype="f64", n=4096, nrhs=16, T_A=256, delta=0.1, logdet=True),
    3: dict(dtype="f32", n=16384, nrhs=64, T_A=512, delta=1.0, logdet=False),
    4: dict(dtype="c128", n=8192, nrhs=32, T_A=256, delta=0.5, logdet=True),
    5: dict(dtype="f64", n=32768, nrhs=128, T_A=512, delta=0.05, logdet=True),
}

_BLOCK_ROWS = 1024


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def gaussian(rows: int, cols: int, is_complex: bool, seed: int, stream: int) -> np.ndarray:
    """Row-major (rows, cols) array of iid standard normals (float64), or
    complex normals (N(0,1) + i N(0,1)) / sqrt(2) (complex128)."""
    out = np.empty((rows, cols), dtype=np.complex128 if is_complex else np.float64)
    nblk = (rows + _BLOCK_ROWS - 1) // _BLOCK_ROWS

    def fill(b: int) -> None:
        r0 = b * _BLOCK_ROWS
        r1 = min(rows, r0 + _BLOCK_ROWS)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, b])))
        if is_complex:
            re = rng.standard_normal((r1 - r0, cols))
            im = rng.standard_normal((r1 - r0, cols))
            out[r0:r1] = (re + 1j * im) * (1.0 / math.sqrt(2.0))
        else:
            out[r0:r1] = rng.standard_normal((r1 - r0, cols))

    if nblk == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def to_colmajor(m: torch.Tensor, ld: int | None = None, pad_value=0.0) -> torch.Tensor:
    """Copy a logical (rows, cols) matrix into column-major storage with leading
    dimension ``ld`` >= rows; rows [rows, ld) of every column hold ``pad_value``."""
    rows, cols = m.shape
    ld = rows if ld is None else int(ld)
    if ld < max(1, rows):
        raise ValueError("ld must be >= max(1, rows)")
    base = torch.full((cols, ld), pad_value, dtype=m.dtype, device=m.device)
    base[:, :rows] = m.t()
    return base.t()[:rows, :]


def is_colmajor(t: torch.Tensor) -> bool:
    return t.dim() == 2 and t.stride(0) == 1 and t.stride(1) >= max(1, t.shape[0])


def _mirror_lower(a: torch.Tensor) -> torch.Tensor:
    """Exactly Hermitian copy of ``a``: keep the lower triangle, write its
    conjugate transpose into the upper one, zero the diagonal's imaginary part."""
    low = torch.tril(a, -1)
    d = torch.diagonal(a)
    if a.is_complex():
        d = d.real.to(a.dtype)
    return low + low.mH + torch.diag_embed(d)


def make_A(n: int, dtype: str, delta: float, seed: int = 0, lda: int | None = None,
           device: str | torch.device = "cpu", pad_value=0.0) -> torch.Tensor:
    """A = G G^H / n + delta I, exactly symmetric/Hermitian, column-major.

    For ``f32``/``c64`` G is rounded to single precision first, the product is
    formed in double precision, rounded once to single, and delta is added in
    single precision.  The same bytes serve the GPU path and the oracle."""
    tdt, _, cplx = DTYPES[dtype]
    single = dtype in ("f32", "c64")
    wide = torch.complex128 if cplx else torch.float64
    g = torch.from_numpy(gaussian(n, n, cplx, seed, 0))
    if single:
        g = g.to(tdt).to(wide)
    g = g.to(device)
    a = (g @ g.mH) * (1.0 / n)
    del g
    a = _mirror_lower(a)
    if single:
        a = a.to(tdt)
        a.diagonal().add_(torch.tensor(delta, dtype=tdt, device=a.device))
    else:
        a.diagonal().add_(delta)
    out = to_colmajor(a, lda, pad_value)
    return out


def make_B(n: int, nrhs: int, dtype: str, seed: int = 0, ldb: int | None = None,
           device: str | torch.device = "cpu", pad_value=0.0) -> torch.Tensor:
    """B with iid (complex) standard normal entries, column-major (n, nrhs)."""
    tdt, _, cplx = DTYPES[dtype]
    b = torch.from_numpy(gaussian(n, nrhs, cplx, seed, 1)).to(tdt).to(device)
    return to_colmajor(b, ldb, pad_value)


def make_herm(n: int, dtype: str, seed: int = 0, lda: int | None = None, device: str | torch.device = "cpu",
              pad_value=0.0) -> torch.Tensor:
    """Symmetric / Hermitian indefinite H = (G + G^H) / sqrt(2 n), exactly
    Hermitian, column-major (the A of a generalized eigenproblem A v = w B v;
    its spectrum fills about [-2, 2])."""
    tdt, _, cplx = DTYPES[dtype]
    wide = torch.complex128 if cplx else torch.float64
    g = torch.from_numpy(gaussian(n, n, cplx, seed, 2)).to(wide).to(device)
    h = (g + g.mH) * (1.0 / math.sqrt(2.0 * n))
    del g
    return to_colmajor(_mirror_lower(h).to(tdt), lda, pad_value)


def make_config(k: int, seed: int = 0, device="cpu"):
    """(A, B, meta) for workload ``k`` (1..5)."""
    c = dict(CONFIGS[k])
    A = make_A(c["n"], c["dtype"], c["delta"], seed, device=device)
    B = make_B(c["n"], c["nrhs"], c["dtype"], seed, device=device)
    c["seed"] = seed
    c["config"] = k
    return A, B, c


def diag_benchmark(n: int, nrhs: int = 1, dtype: str = "f64", device="cpu"):
    """The JAXMg paper's potrs benchmark input (section "Performance and
    scaling"): A = diag(1, ..., n), b = (1, ..., 1)^T, column-major."""
    tdt, _, _ = DTYPES[dtype]
    a = torch.diag(torch.arange(1, n + 1, dtype=torch.float64)).to(tdt).to(device)
    b = torch.ones((n, nrhs), dtype=tdt, device=device)
    return to_colmajor(a), to_colmajor(b)


def random_spd_small(n: int, dtype: str, seed: int, delta: float = 0.5, lda=None, device="cpu",
                     pad_value=0.0):
    """Small well-conditioned workload of the same family, for parity sweeps."""
    return make_A(n, dtype, delta, seed, lda=lda, device=device, pad_value=pad_value)
