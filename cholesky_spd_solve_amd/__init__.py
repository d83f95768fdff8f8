"""Python binding of the gfx950 dense SPD/HPD solver (``libspd_mi355x.so``).

Argument marshalling only: every step of the factorization, the solves and
the log-determinant runs in the library's HIP kernels.  PyTorch supplies the
device memory and the stream.

The operation (JAXMg paper, "Software design", potrs): solve A X = B for a
symmetric (Hermitian) positive-definite A via A = L L^H, optionally returning
log det(A) from the same factor; T_A is the tile size.

Matrices are torch tensors on the GPU in *column-major* storage: a logical
(rows, cols) tensor with ``stride(0) == 1`` and ``stride(1) == ld >= rows``
(for example ``M.t()`` of a row-major tensor, or what ``spdgen`` returns).
Buffers are updated in place, as the C ABI does.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspd_mi355x.so")

SPD_R32, SPD_R64, SPD_C64, SPD_C128 = 0, 1, 2, 3
DTYPE_CODE = {
    torch.float32: SPD_R32,
    torch.float64: SPD_R64,
    torch.complex64: SPD_C64,
    torch.complex128: SPD_C128,
}
SYMBOLS = ("spd_workspace_size", "spd_potrf", "spd_potrs", "spd_posv", "spd_forward_solve", "spd_gp_loglik",
           "spd_logdet",
           "spd_sygst_workspace_size", "spd_sygst", "spd_last_error", "spd_profile_enable", "spd_profile_read",
           "spd_debug_validate", "spd_set_option", "spd_get_option", "spd_release", "spd_posv_noalloc")
SPD_ERR_HIP, SPD_ERR_CHECK, SPD_ERR_SCRATCH = 1, 2, 3
NOALLOC_SCRATCH_BYTES = 64 << 20  # spd_posv_noalloc's fixed per-device buffer
PROF_SYRK, PROF_PANEL, PROF_DIAG, PROF_SOLVE, PROF_UPDATE, PROF_SYRK_AUX = 0, 1, 2, 3, 4, 5
# schedule / tile-shape options (spd_set_option)
OPT_LOOKAHEAD, OPT_TWO_STEP, OPT_PAIR_ROWS, OPT_SYRK_DEEP_ROWS, OPT_RECT_TALL_ROWS = 1, 2, 3, 4, 5
OPT_TILE_LAUNCH, OPT_TILE_WAIT_US, OPT_COLUMN_FIRST_ROWS, OPT_TILE_HOLD_ROWS = 6, 7, 8, 9
OPT_SUBST_LAUNCH, OPT_TILE_UPDATE_ROWS, OPT_TRIPLE_ROWS = 10, 11, 12
OPT_DEFAULT = -(1 << 63)

_lock = threading.Lock()
_lib = None


class LinAlgError(RuntimeError):
    """The matrix is not positive definite: ``info`` is the order of the first
    leading minor that is not."""

    def __init__(self, info: int):
        super().__init__(f"leading minor of order {info} is not positive definite")
        self.info = info


class SpdError(RuntimeError):
    pass


def load():
    """Load the HIP library; raises if it has not been built (there is no
    fallback path)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise SpdError(f"{LIB_PATH} is missing: build it with "
                               "`python -m cholesky_spd_solve_amd.build`")
            lib = ctypes.CDLL(LIB_PATH)
            i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
            i32 = ctypes.c_int
            lib.spd_workspace_size.argtypes = [i32, i64, i64, i64]
            lib.spd_workspace_size.restype = sz
            lib.spd_potrf.argtypes = [i32, i64, vp, i64, i64, vp, vp, sz, vp]
            lib.spd_potrf.restype = i32
            lib.spd_potrs.argtypes = [i32, i64, i64, vp, i64, vp, i64, i64, vp, vp, sz, vp]
            lib.spd_potrs.restype = i32
            lib.spd_posv.argtypes = [i32, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp, sz, vp]
            lib.spd_posv.restype = i32
            lib.spd_posv_noalloc.argtypes = [i32, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp]
            lib.spd_posv_noalloc.restype = i32
            lib.spd_forward_solve.argtypes = [i32, i64, i64, vp, i64, vp, i64, i64, vp, vp, sz, vp]
            lib.spd_forward_solve.restype = i32
            lib.spd_gp_loglik.argtypes = [i32, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp, sz, vp]
            lib.spd_gp_loglik.restype = i32
            lib.spd_logdet.argtypes = [i32, i64, vp, i64, vp, vp, vp]
            lib.spd_logdet.restype = i32
            lib.spd_sygst_workspace_size.argtypes = [i32, i32, i64, i64]
            lib.spd_sygst_workspace_size.restype = sz
            lib.spd_sygst.argtypes = [i32, i32, i64, vp, i64, vp, i64, i64, vp, vp, sz, vp]
            lib.spd_sygst.restype = i32
            lib.spd_last_error.argtypes = []
            lib.spd_last_error.restype = ctypes.c_char_p
            lib.spd_profile_enable.argtypes = [i32]
            lib.spd_profile_enable.restype = i32
            lib.spd_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double),
                                             ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
            lib.spd_profile_read.restype = i32
            lib.spd_debug_validate.argtypes = [i32]
            lib.spd_debug_validate.restype = i32
            lib.spd_set_option.argtypes = [i32, i64]
            lib.spd_set_option.restype = i32
            lib.spd_get_option.argtypes = [i32]
            lib.spd_get_option.restype = i64
            lib.spd_release.argtypes = []
            lib.spd_release.restype = i32
            _lib = lib
    return _lib


def _check(rc: int, what: str):
    if rc == 0:
        return
    if rc < 0:
        raise ValueError(f"{what}: argument {-rc} is invalid")
    msg = load().spd_last_error().decode(errors="replace")
    kind = ("launch validation failed" if rc == SPD_ERR_CHECK else
            "scratch buffer too small" if rc == SPD_ERR_SCRATCH else "HIP error")
    raise SpdError(f"{what}: {kind}: {msg}")


def _code(t: torch.Tensor) -> int:
    try:
        return DTYPE_CODE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _colmajor(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    rows, cols = t.shape
    if cols > 1 and rows > 0 and not (t.stride(0) == 1 and t.stride(1) >= rows):
        raise ValueError(f"{name} must be column-major (stride(0) == 1, stride(1) >= rows)")
    if cols <= 1:
        if rows > 1 and t.stride(0) != 1:
            raise ValueError(f"{name} must be column-major (stride(0) == 1)")
        return max(1, rows)
    return max(1, t.stride(1))


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def workspace_size(dtype: torch.dtype, n: int, nrhs: int, T_A: int) -> int:
    return int(load().spd_workspace_size(DTYPE_CODE[dtype], n, nrhs, T_A))


def workspace(dtype: torch.dtype, n: int, nrhs: int, T_A: int, device="cuda") -> torch.Tensor:
    nbytes = workspace_size(dtype, n, nrhs, T_A)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def potrf(A: torch.Tensor, T_A: int, info: torch.Tensor | None = None, work: torch.Tensor | None = None,
          stream=None) -> torch.Tensor:
    """Factor A = L L^H in place (lower triangle).  Returns the device int32
    ``info`` (0, or the order of the first non-positive-definite minor)."""
    lda = _colmajor(A, "A")
    n = A.shape[0]
    if A.shape[1] != n:
        raise ValueError("A must be square")
    if info is None:
        info = torch.empty(1, dtype=torch.int32, device=A.device)
    if work is None:
        work = workspace(A.dtype, n, 0, T_A, A.device)
    rc = load().spd_potrf(_code(A), n, _ptr(A), lda, int(T_A), _ptr(info), _ptr(work), work.numel(),
                          ctypes.c_void_p(_stream(stream)))
    _check(rc, "spd_potrf")
    return info


def potrs(L: torch.Tensor, B: torch.Tensor, T_A: int, info: torch.Tensor | None = None,
          work: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Overwrite B with the solution of (L L^H) X = B; returns B."""
    lda = _colmajor(L, "L")
    ldb = _colmajor(B, "B")
    n, nrhs = B.shape
    if L.shape != (n, n):
        raise ValueError("L must be n x n with n = B.shape[0]")
    if B.dtype != L.dtype:
        raise TypeError("L and B must have the same dtype")
    if work is None:
        work = workspace(L.dtype, n, nrhs, T_A, L.device)
    rc = load().spd_potrs(_code(L), n, nrhs, _ptr(L), lda, _ptr(B), ldb, int(T_A), _ptr(info), _ptr(work),
                          work.numel(), ctypes.c_void_p(_stream(stream)))
    _check(rc, "spd_potrs")
    return B


def posv(A: torch.Tensor, B: torch.Tensor, T_A: int, info: torch.Tensor | None = None,
         logdet_out: torch.Tensor | None = None, work: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Factor A (in place, as potrf), write log det(A) into ``logdet_out``
    (device float64, optional) and overwrite B with the solution, in one
    call.  Returns the device int32 ``info``."""
    lda = _colmajor(A, "A")
    ldb = _colmajor(B, "B")
    n, nrhs = B.shape
    if A.shape != (n, n):
        raise ValueError("A must be n x n with n = B.shape[0]")
    if B.dtype != A.dtype:
        raise TypeError("A and B must have the same dtype")
    if info is None:
        info = torch.empty(1, dtype=torch.int32, device=A.device)
    if work is None:
        work = workspace(A.dtype, n, nrhs, T_A, A.device)
    rc = load().spd_posv(_code(A), n, nrhs, _ptr(A), lda, _ptr(B), ldb, int(T_A), _ptr(info), _ptr(logdet_out),
                         _ptr(work), work.numel(), ctypes.c_void_p(_stream(stream)))
    _check(rc, "spd_posv")
    return info


def posv_noalloc(A: torch.Tensor, B: torch.Tensor, T_A: int, info: torch.Tensor, logdet_out=None,
                 stream=None) -> torch.Tensor:
    """posv with no workspace argument: the library's fixed per-device
    scratch buffer serves as workspace and nothing is allocated (``info`` and
    ``logdet_out`` are the caller's).  Raises SpdError when the sizes need
    more than NOALLOC_SCRATCH_BYTES of workspace."""
    lda = _colmajor(A, "A")
    ldb = _colmajor(B, "B")
    n, nrhs = B.shape
    if A.shape != (n, n):
        raise ValueError("A must be n x n with n = B.shape[0]")
    if B.dtype != A.dtype:
        raise TypeError("A and B must have the same dtype")
    rc = load().spd_posv_noalloc(_code(A), n, nrhs, _ptr(A), lda, _ptr(B), ldb, int(T_A), _ptr(info),
                                 _ptr(logdet_out), ctypes.c_void_p(_stream(stream)))
    _check(rc, "spd_posv_noalloc")
    return info


def forward_solve(L: torch.Tensor, B: torch.Tensor, T_A: int, info: torch.Tensor | None = None,
                  work: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Overwrite B with L^-1 B (forward substitution only); returns B."""
    lda = _colmajor(L, "L")
    ldb = _colmajor(B, "B")
    n, nrhs = B.shape
    if L.shape != (n, n):
        raise ValueError("L must be n x n with n = B.shape[0]")
    if B.dtype != L.dtype:
        raise TypeError("L and B must have the same dtype")
    if work is None:
        work = workspace(L.dtype, n, nrhs, T_A, L.device)
    rc = load().spd_forward_solve(_code(L), n, nrhs, _ptr(L), lda, _ptr(B), ldb, int(T_A), _ptr(info), _ptr(work),
                                  work.numel(), ctypes.c_void_p(_stream(stream)))
    _check(rc, "spd_forward_solve")
    return B


def gp_loglik(L: torch.Tensor, R: torch.Tensor, T_A: int, info: torch.Tensor | None = None,
              work: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Gaussian-process marginal log-likelihood of each residual column of R
    (R is overwritten by L^-1 R) into a device float64 tensor of R.shape[1]."""
    lda = _colmajor(L, "L")
    ldr = _colmajor(R, "R")
    n, nrhs = R.shape
    if L.shape != (n, n):
        raise ValueError("L must be n x n with n = R.shape[0]")
    if R.dtype != L.dtype:
        raise TypeError("L and R must have the same dtype")
    if work is None:
        work = workspace(L.dtype, n, nrhs, T_A, L.device)
    if out is None:
        out = torch.empty(nrhs, dtype=torch.float64, device=L.device)
    rc = load().spd_gp_loglik(_code(L), n, nrhs, _ptr(L), lda, _ptr(R), ldr, int(T_A), _ptr(info), _ptr(out),
                              _ptr(work), work.numel(), ctypes.c_void_p(_stream(stream)))
    _check(rc, "spd_gp_loglik")
    return out


def logdet(L: torch.Tensor, info: torch.Tensor | None = None, out: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    """log det(A) = 2 sum log Re L_ii into a device float64 scalar tensor."""
    lda = _colmajor(L, "L")
    n = L.shape[0]
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=L.device)
    rc = load().spd_logdet(_code(L), n, _ptr(L), lda, _ptr(info), _ptr(out), ctypes.c_void_p(_stream(stream)))
    _check(rc, "spd_logdet")
    return out


def sygst_workspace_size(dtype: torch.dtype, itype: int, n: int, T_A: int) -> int:
    return int(load().spd_sygst_workspace_size(DTYPE_CODE[dtype], int(itype), n, T_A))


def sygst(itype: int, A: torch.Tensor, L: torch.Tensor, T_A: int, info: torch.Tensor | None = None,
          work: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Reduce the generalized eigenproblem of (A, B = L L^H) to standard form
    in place: the lower triangle of A becomes that of L^-1 A L^-H (itype 1) or
    L^H A L (itypes 2 and 3).  ``info`` is the one potrf returned for B.
    Returns A."""
    lda = _colmajor(A, "A")
    ldl = _colmajor(L, "L")
    n = A.shape[0]
    if A.shape != (n, n) or L.shape != (n, n):
        raise ValueError("A and L must be n x n")
    if A.dtype != L.dtype:
        raise TypeError("A and L must have the same dtype")
    if work is None:
        nbytes = sygst_workspace_size(A.dtype, itype, n, T_A)
        work = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=A.device)
    rc = load().spd_sygst(_code(A), int(itype), n, _ptr(A), lda, _ptr(L), ldl, int(T_A), _ptr(info), _ptr(work),
                          work.numel(), ctypes.c_void_p(_stream(stream)))
    _check(rc, "spd_sygst")
    return A


def solve(A: torch.Tensor, B: torch.Tensor, T_A: int, want_logdet: bool = False, check: bool = True):
    """potrf, then logdet (optional), then potrs, all in place, on the current
    stream; one synchronisation at the end to read ``info``.  Returns X (= B)
    or (X, logdet).  Raises LinAlgError if A is not positive definite."""
    n = A.shape[0]
    nrhs = B.shape[1] if B.dim() == 2 else 1
    work = workspace(A.dtype, n, nrhs, T_A, A.device)
    info = potrf(A, T_A, work=work)
    ld = logdet(A, info) if want_logdet else None
    potrs(A, B, T_A, info=info, work=work)
    if check:
        code = int(info.item())
        if code != 0:
            raise LinAlgError(code)
    if want_logdet:
        return B, float(ld.item())
    return B


def debug_validate(mode: int) -> None:
    """Launch validation: 0 off, 1 replay every launch's addresses on the host
    before enqueueing it, 2 replay only (dry run, no GPU work)."""
    _check(load().spd_debug_validate(int(mode)), "spd_debug_validate")


def set_option(opt: int, value: int) -> None:
    """Set a schedule / tile-shape option (OPT_*; OPT_DEFAULT restores the
    default).  Options select among schedules and tile shapes that compute
    the same result; they are process-wide."""
    _check(load().spd_set_option(int(opt), int(value)), "spd_set_option")


def get_option(opt: int) -> int:
    return int(load().spd_get_option(int(opt)))


class options:
    """Context manager: set options for a block, restore the previous values
    after it, e.g. ``with options({OPT_PAIR_ROWS: 0}): ...``."""

    def __init__(self, values: dict):
        self.values = dict(values)
        self.saved = {}

    def __enter__(self):
        try:
            for k, v in self.values.items():
                prev = get_option(k)
                set_option(k, v)
                self.saved[k] = prev
        except BaseException:
            self.__exit__()
            raise
        return self

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            set_option(k, v)
        return False


def release() -> None:
    """Wait for and destroy this thread's auxiliary streams and events."""
    _check(load().spd_release(), "spd_release")


def profile_enable(mask: int) -> None:
    _check(load().spd_profile_enable(int(mask)), "spd_profile_enable")


def profile_read(kernel_class: int):
    """(milliseconds, launches, flops) of one kernel class since the last read."""
    ms = ctypes.c_double()
    cnt = ctypes.c_int64()
    fl = ctypes.c_double()
    _check(load().spd_profile_read(int(kernel_class), ctypes.byref(ms), ctypes.byref(cnt), ctypes.byref(fl)),
           "spd_profile_read")
    return ms.value, cnt.value, fl.value
