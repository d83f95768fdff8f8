"""CPU-only replay of every kernel launch the solver would make.

With launch validation in dry-run mode (spd_debug_validate(2)) the library
enqueues nothing and instead replays each launch on the host: every thread of
every workgroup computes, with the kernels' own index functions, the addresses
it would touch, and each must fall inside the buffers handed to the entry
point.  The pointers below are never dereferenced; they only fix the address
ranges (and 16-byte alignment, which selects the vectorised load path).
"""
import ctypes

import pytest

import cholesky_spd_solve_amd as spd

ES = {0: 4, 1: 8, 2: 8, 3: 16}
BASE = 1 << 40  # fake device addresses, far apart and 4 KiB aligned


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(spd.LIB_PATH):
        from cholesky_spd_solve_amd import build
        build.build()
    lib = spd.load()
    assert lib.spd_debug_validate(2) == 0
    yield lib
    lib.spd_debug_validate(0)


def dry_solve(lib, dt, n, nrhs, T, lda=None, ldb=None, shift=0):
    """potrf + logdet + potrs on fake buffers; `shift` elements of offset break
    16-byte alignment of A and B."""
    es = ES[dt]
    lda = lda or max(1, n)
    ldb = ldb or max(1, n)
    vp = ctypes.c_void_p
    A = BASE + shift * es
    B = 2 * BASE + shift * es
    info = 3 * BASE
    ld = 3 * BASE + 4096
    work = 4 * BASE
    wbytes = lib.spd_workspace_size(dt, n, nrhs, T)
    rc = lib.spd_potrf(dt, n, vp(A), lda, T, vp(info), vp(work), wbytes, None)
    assert rc == 0, (rc, lib.spd_last_error())
    rc = lib.spd_logdet(dt, n, vp(A), lda, vp(info), vp(ld), None)
    assert rc == 0, (rc, lib.spd_last_error())
    rc = lib.spd_potrs(dt, n, nrhs, vp(A), lda, vp(B), ldb, T, vp(info), vp(work), wbytes, None)
    assert rc == 0, (rc, lib.spd_last_error())


CODE = {"f32": 0, "f64": 1, "c64": 2, "c128": 3}
SHAPES = [
    ("f64", 1, 1, 64), ("f64", 2, 3, 1), ("f64", 63, 2, 16), ("f64", 64, 1, 64), ("f64", 65, 5, 64),
    ("f64", 127, 4, 32), ("f64", 130, 7, 100), ("f64", 300, 16, 128), ("f64", 777, 3, 1000),
    ("f64", 1000, 33, 256), ("f64", 600, 130, 192), ("f64", 520, 40, 128), ("f64", 256, 1, 64),
    ("f32", 65, 2, 64), ("f32", 300, 16, 128), ("f32", 1000, 33, 256), ("f32", 518, 64, 512),
    ("c128", 1, 1, 8), ("c128", 65, 3, 64), ("c128", 300, 16, 100), ("c128", 600, 32, 256),
    ("c64", 130, 4, 64), ("c64", 700, 8, 256),
]


@pytest.mark.parametrize("dt,n,nrhs,T", SHAPES)
def test_dry_run_in_bounds(lib, dt, n, nrhs, T):
    dry_solve(lib, CODE[dt], n, nrhs, T)


@pytest.mark.parametrize("dt,n,nrhs,T", SHAPES[::3])
def test_dry_run_block_step_back_substitution(lib, dt, n, nrhs, T):
    """The back substitution by block steps (SPD_OPT_SUBST_LAUNCH = 0), which
    these sizes otherwise do in one launch."""
    with spd.options({spd.OPT_SUBST_LAUNCH: 0}):
        dry_solve(lib, CODE[dt], n, nrhs, T)


@pytest.mark.parametrize("dt,n,nrhs,T", [("f64", 333, 6, 64), ("c128", 333, 6, 64), ("f32", 300, 9, 128),
                                         ("f64", 1024, 16, 256)])
def test_dry_run_padded_and_unaligned(lib, dt, n, nrhs, T):
    dry_solve(lib, CODE[dt], n, nrhs, T, lda=n + 5, ldb=n + 3)
    dry_solve(lib, CODE[dt], n, nrhs, T, lda=n + 2, ldb=n + 2, shift=1)


@pytest.mark.parametrize("dt,n,nrhs,T", [s for s in SHAPES if s[0] in ("f64", "f32")])
def test_dry_run_forward_solve_and_gp_loglik(lib, dt, n, nrhs, T):
    code, es = CODE[dt], ES[CODE[dt]]
    vp = ctypes.c_void_p
    A, B, info, out, work = BASE, 2 * BASE, 3 * BASE, 3 * BASE + 4096, 4 * BASE
    wbytes = lib.spd_workspace_size(code, n, nrhs, T)
    assert lib.spd_forward_solve(code, n, nrhs, vp(A), n, vp(B), n, T, vp(info), vp(work), wbytes, None) == 0, \
        lib.spd_last_error()
    assert lib.spd_gp_loglik(code, n, nrhs, vp(A), n, vp(B), n, T, vp(info), vp(out), vp(work), wbytes, None) == 0, \
        lib.spd_last_error()


def test_dry_run_real_general_path(lib):
    """A leading dimension past the block-update kernel's 32-bit offsets sends
    real types down the general substitution path; it must stay in bounds."""
    dry_solve(lib, 1, 65, 3, 32, lda=(1 << 24) + 8)


@pytest.mark.parametrize("dt", ["f64", "f32", "c128", "c64"])
def test_dry_run_huge_leading_dimension(lib, dt):
    """Leading dimensions whose 64 or 128 columns span more than 2^32
    elements: the trailing update must address C with 64-bit offsets (the
    replay checks that every offset fits the kernel's offset type)."""
    dry_solve(lib, CODE[dt], 300, 5, 64, lda=1 << 27, ldb=(1 << 27) + 3)


def test_dry_run_detects_a_short_workspace(lib):
    """The validator itself: a workspace one byte too small for the kernels
    (but passed as large enough) must be caught."""
    vp = ctypes.c_void_p
    n, T = 200, 64
    need = lib.spd_workspace_size(1, n, 0, T)
    # claim `need` bytes but place the buffer so that its real extent ends early:
    # register a smaller region by lying about work_bytes is rejected up front,
    # so instead overlap the workspace with the end of A's address range
    rc = lib.spd_potrf(1, n, vp(BASE), n, T, vp(3 * BASE), vp(4 * BASE), need - 1, None)
    assert rc == -8
    rc = lib.spd_potrf(1, n, vp(BASE), n - 1 + 1, T, vp(3 * BASE), vp(4 * BASE), need, None)
    assert rc == 0, lib.spd_last_error()


GST_SHAPES = [("f64", 1, 8), ("f64", 65, 32), ("f64", 200, 64), ("f64", 260, 128), ("f32", 130, 64),
              ("c128", 70, 32), ("c64", 100, 64)]


@pytest.mark.parametrize("itype", [1, 2, 3])
@pytest.mark.parametrize("dt,n,T", GST_SHAPES)
def test_dry_run_sygst(lib, itype, dt, n, T):
    code = CODE[dt]
    vp = ctypes.c_void_p
    A, Lb, info, work = BASE, 2 * BASE, 3 * BASE, 4 * BASE
    wbytes = lib.spd_sygst_workspace_size(code, itype, n, T)
    assert wbytes > 0
    for lda, ldl in ((n, n), (n + 3, n + 5)):
        rc = lib.spd_sygst(code, itype, n, vp(A), lda, vp(Lb), ldl, T, vp(info), vp(work), wbytes, None)
        assert rc == 0, (rc, lib.spd_last_error())


@pytest.mark.parametrize("dt,n,nrhs,T", SHAPES + [("f64", 2000, 7, 128), ("f64", 1300, 130, 128)])
def test_dry_run_posv(lib, dt, n, nrhs, T):
    """The fused solve (the factorization with the forward substitution on a
    second stream where the two-step schedule applies, the three calls
    otherwise), with and without log det."""
    code, es = CODE[dt], ES[CODE[dt]]
    vp = ctypes.c_void_p
    A, B, info, ld, work = BASE, 2 * BASE, 3 * BASE, 3 * BASE + 4096, 4 * BASE
    wbytes = lib.spd_workspace_size(code, n, nrhs, T)
    for logdet in (vp(ld), None):
        rc = lib.spd_posv(code, n, nrhs, vp(A), n, vp(B), n, T, vp(info), logdet, vp(work), wbytes, None)
        assert rc == 0, (rc, lib.spd_last_error())


@pytest.mark.parametrize("dt,n,nrhs,T", [("f64", 2048, 16, 256), ("f64", 1000, 5, 128), ("c128", 700, 3, 64),
                                         ("f32", 65, 2, 64), ("c64", 300, 4, 100)])
def test_dry_run_posv_noalloc(lib, dt, n, nrhs, T):
    """The fixed-scratch solve replays in bounds of the scratch buffer (a
    stand-in address in a dry run), with and without log det."""
    code = CODE[dt]
    vp = ctypes.c_void_p
    A, B, info, ld = BASE, 2 * BASE, 3 * BASE, 3 * BASE + 4096
    for logdet in (vp(ld), None):
        rc = lib.spd_posv_noalloc(code, n, nrhs, vp(A), n, vp(B), n, T, vp(info), logdet, None)
        assert rc == 0, (rc, lib.spd_last_error())


def test_dry_run_posv_noalloc_rejects_large_sizes(lib):
    vp = ctypes.c_void_p
    n, nrhs, T = 16384, 64, 512
    assert lib.spd_workspace_size(0, n, nrhs, T) > (64 << 20)
    rc = lib.spd_posv_noalloc(0, n, nrhs, vp(BASE), n, vp(2 * BASE), n, T, vp(3 * BASE), None, None)
    assert rc == 3
    assert b"bytes of workspace" in lib.spd_last_error()
    assert lib.spd_posv_noalloc(0, 4, 1, vp(BASE), 3, vp(2 * BASE), 4, 2, vp(3 * BASE), None, None) == -5


@pytest.mark.parametrize("triple_rows,pair_rows", [(-1, -1), (1, 0), (1, -1), (0, 0)])
@pytest.mark.parametrize("dt,n,nrhs,T", [("f64", 6001, 3, 128), ("f32", 5120, 2, 128)])
def test_dry_run_step_groups(lib, dt, n, nrhs, T, triple_rows, pair_rows):
    """Orders of 40 tiles and more keep six trailing-update panels and take
    the factorization's steps in threes while the trailing matrix is large;
    every mix of threes, pairs and single steps (a ragged last tile, the
    groups wrapping around the six buffers) replays in bounds, through the
    three calls and the fused solve."""
    code = CODE[dt]
    with spd.options({spd.OPT_TRIPLE_ROWS: triple_rows, spd.OPT_PAIR_ROWS: pair_rows}):
        dry_solve(lib, code, n, nrhs, T)
        vp = ctypes.c_void_p
        A, B, info, ld, work = BASE, 2 * BASE, 3 * BASE, 3 * BASE + 4096, 4 * BASE
        wbytes = lib.spd_workspace_size(code, n, nrhs, T)
        rc = lib.spd_posv(code, n, nrhs, vp(A), n, vp(B), n, T, vp(info), vp(ld), vp(work), wbytes, None)
        assert rc == 0, (rc, lib.spd_last_error())
