"""CPU-only checks of the host side: the C ABI library loads and exports every
entry point its header declares, argument validation rejects bad calls before
any GPU work, the workspace query, and the seeded input generator."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import spdgen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spd.h")


@pytest.fixture(scope="module")
def lib():
    import cholesky_spd_solve_amd as spd
    if not os.path.exists(spd.LIB_PATH):
        from cholesky_spd_solve_amd import build
        build.build()
    return spd.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spd_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in ("spd_potrf", "spd_potrs", "spd_logdet", "spd_workspace_size"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_symbol_list_matches_header():
    import cholesky_spd_solve_amd as spd
    assert sorted(spd.SYMBOLS) == declared_functions()


def test_workspace_size(lib):
    f = lib.spd_workspace_size
    assert f(1, 0, 0, 64) == 0
    assert f(1, -1, 0, 64) == 0
    assert f(1, 10, -1, 64) == 0
    assert f(1, 10, 1, 0) == 0
    assert f(9, 10, 1, 4) == 0
    # INV nt*T*T + four panels (six from 40 tiles on) of (n rounded up to 128) x (T rounded up to 32)
    # + TMP max(T*T, T*nrhs) + a 256-byte counter + the one-launch diagonal
    # tile's 2 nb^2 + 2 flags of 128 bytes each (nb = ceil(T / 64)) rounded up
    # to 256 bytes (16640 bytes at T = 512, 1280 at T = 100); for nrhs > 0 also two
    # buffers for the transposed solved block, (nrhs rounded up to 128) x (T
    # rounded up to 32), two sets of nt*T*T chain products, 8 partial
    # T x nrhs blocks, the one-launch back substitution's two T x nrhs blocks
    # and its 2*nt*nc + 2 counters of 128 bytes each (nc = ceil(nrhs / 64)
    # column pieces, 32 wide when nrhs <= 32); each rounded up to 256 bytes
    n, nrhs, T = 32768, 128, 512
    up = lambda a, b: -(-a // b) * b
    el = (n // T) * T * T + 6 * n * T + T * T  # 64 tiles: six panel buffers
    solve = 2 * 128 * 512 + 2 * (n // T) * T * T + 8 * T * nrhs + 2 * T * nrhs
    sflags = up(4 * 32 * (2 * 64 * 2 + 2), 256)
    assert f(1, n, 0, T) == el * 8 + 256 + 16640
    assert f(1, n, nrhs, T) == (el + solve) * 8 + 256 + 16640 + sflags
    assert f(3, n, nrhs, T) == (el + solve) * 16 + 256 + 16640 + sflags
    n, nrhs, T = 1000, 7, 100
    el = up(10 * 100 * 100, 32) + 4 * up(1024 * 128, 32) + up(100 * 100, 32)
    solve = up(2 * 128 * 128, 32) + 2 * up(10 * 100 * 100, 32) + up(8 * 100 * 7, 32) + up(2 * 100 * 7, 32)
    sflags = up(4 * 32 * (2 * 10 * 1 + 2), 256)
    assert f(1, n, 0, T) == el * 8 + 256 + 1280
    assert f(1, n, nrhs, T) == (el + solve) * 8 + 256 + 1280 + sflags
    # T_A > n is clamped to n
    assert f(1, 100, 1, 1000) == f(1, 100, 1, 100)


def test_sygst_workspace_size(lib):
    f = lib.spd_sygst_workspace_size
    assert f(1, 0, 10, 4) == 0 and f(1, 4, 10, 4) == 0 and f(1, 1, 0, 4) == 0 and f(1, 1, 10, 0) == 0
    assert f(9, 1, 10, 4) == 0
    up = lambda a, b: -(-a // b) * b
    for dt, es in ((1, 8), (3, 16), (0, 4)):
        n, T = 1000, 128
        al = 256 // es
        sq = up(n * n, al)
        # itype 1: M, the substitution workspace for n right-hand sides, two
        # sets of the rank-2k panels P and Q ((n up to 128) x 2 (T up to 32)),
        # Y and V (n x T), two T x T tiles
        solve = lib.spd_workspace_size(dt, n, n, T) // es
        pw = up(up(n, 128) * 2 * up(T, 32), al)
        assert f(dt, 1, n, T) == (sq + up(solve, al) + 4 * pw + 2 * up(n * T, al) + 2 * up(T * T, al)) * es
        # itypes 2 and 3: M, the panels P and Q, two squares of order n up to
        # 128, two sets of nt T x T tiles, two T x n blocks
        nt = -(-n // T)
        sq128 = up(up(n, 128) ** 2, al)
        ref = (sq + 2 * pw + 2 * sq128 + 2 * up(nt * T * T, al) + 2 * up(T * n, al)) * es
        assert f(dt, 2, n, T) == f(dt, 3, n, T) == ref


def test_argument_validation_returns_before_gpu_work(lib):
    vp = ctypes.c_void_p
    dummy = vp(0x1000)  # never dereferenced: every call below is rejected first
    info = vp(0x2000)
    pot = lib.spd_potrf
    assert pot(7, 4, dummy, 4, 2, info, dummy, 1 << 20, None) == -1
    assert pot(1, -1, dummy, 4, 2, info, dummy, 1 << 20, None) == -2
    assert pot(1, 4, None, 4, 2, info, dummy, 1 << 20, None) == -3
    assert pot(1, 4, dummy, 3, 2, info, dummy, 1 << 20, None) == -4
    assert pot(1, 4, dummy, 4, 0, info, dummy, 1 << 20, None) == -5
    assert pot(1, 4, dummy, 4, 2, None, dummy, 1 << 20, None) == -6
    assert pot(1, 4, dummy, 4, 2, info, None, 1 << 20, None) == -7
    assert pot(1, 4, dummy, 4, 2, info, dummy, 8, None) == -8
    prs = lib.spd_potrs
    assert prs(1, 4, -2, dummy, 4, dummy, 4, 2, info, dummy, 1 << 20, None) == -3
    assert prs(1, 4, 2, dummy, 4, dummy, 3, 2, info, dummy, 1 << 20, None) == -7
    assert prs(1, 4, 2, dummy, 4, dummy, 4, 0, info, dummy, 1 << 20, None) == -8
    assert prs(1, 4, 2, dummy, 4, dummy, 4, 2, info, dummy, 8, None) == -11
    ld = lib.spd_logdet
    assert ld(1, 4, dummy, 2, info, dummy, None) == -4
    assert ld(1, 4, dummy, 4, info, None, None) == -6
    fw = lib.spd_forward_solve
    assert fw(7, 4, 2, dummy, 4, dummy, 4, 2, info, dummy, 1 << 20, None) == -1
    assert fw(1, 4, 2, dummy, 4, dummy, 3, 2, info, dummy, 1 << 20, None) == -7
    assert fw(1, 4, 2, dummy, 4, dummy, 4, 2, info, dummy, 8, None) == -11
    gp = lib.spd_gp_loglik
    out = vp(0x3000)
    assert gp(3, 4, 2, dummy, 4, dummy, 4, 2, info, out, dummy, 1 << 20, None) == -1  # complex
    assert gp(2, 4, 2, dummy, 4, dummy, 4, 2, info, out, dummy, 1 << 20, None) == -1
    assert gp(1, 4, 2, dummy, 3, dummy, 4, 2, info, out, dummy, 1 << 20, None) == -5
    assert gp(1, 4, 2, dummy, 4, dummy, 4, 2, info, None, dummy, 1 << 20, None) == -10
    assert gp(1, 4, 2, dummy, 4, dummy, 4, 2, info, out, dummy, 8, None) == -12
    pv = lib.spd_posv
    assert pv(7, 4, 2, dummy, 4, dummy, 4, 2, info, None, dummy, 1 << 20, None) == -1
    assert pv(1, 4, -1, dummy, 4, dummy, 4, 2, info, None, dummy, 1 << 20, None) == -3
    assert pv(1, 4, 2, dummy, 3, dummy, 4, 2, info, None, dummy, 1 << 20, None) == -5
    assert pv(1, 4, 2, dummy, 4, dummy, 3, 2, info, None, dummy, 1 << 20, None) == -7
    assert pv(1, 4, 2, dummy, 4, dummy, 4, 0, info, None, dummy, 1 << 20, None) == -8
    assert pv(1, 4, 2, dummy, 4, dummy, 4, 2, None, None, dummy, 1 << 20, None) == -9
    assert pv(1, 4, 2, dummy, 4, dummy, 4, 2, info, None, dummy, 8, None) == -12
    gst = lib.spd_sygst
    assert gst(7, 1, 4, dummy, 4, dummy, 4, 2, info, dummy, 1 << 20, None) == -1
    assert gst(1, 0, 4, dummy, 4, dummy, 4, 2, info, dummy, 1 << 20, None) == -2
    assert gst(1, 4, 4, dummy, 4, dummy, 4, 2, info, dummy, 1 << 20, None) == -2
    assert gst(1, 1, -1, dummy, 4, dummy, 4, 2, info, dummy, 1 << 20, None) == -3
    assert gst(1, 1, 4, None, 4, dummy, 4, 2, info, dummy, 1 << 20, None) == -4
    assert gst(1, 1, 4, dummy, 3, dummy, 4, 2, info, dummy, 1 << 20, None) == -5
    assert gst(1, 1, 4, dummy, 4, None, 4, 2, info, dummy, 1 << 20, None) == -6
    assert gst(1, 2, 4, dummy, 4, dummy, 3, 2, info, dummy, 1 << 20, None) == -7
    assert gst(1, 3, 4, dummy, 4, dummy, 4, 0, info, dummy, 1 << 20, None) == -8
    assert gst(1, 1, 4, dummy, 4, dummy, 4, 2, info, None, 1 << 20, None) == -10
    assert gst(1, 1, 4, dummy, 4, dummy, 4, 2, info, dummy, 8, None) == -11
    assert gst(1, 1, 0, None, 1, None, 1, 2, info, None, 0, None) == 0  # n == 0: nothing to do


def test_profile_class_validation(lib):
    import cholesky_spd_solve_amd as spd
    with pytest.raises(ValueError):
        spd.profile_read(9)


def test_options_validate_and_restore(lib):
    """spd_set_option checks its option number and value range; the
    default marker restores each option's default."""
    import cholesky_spd_solve_amd as spd
    defaults = {spd.OPT_LOOKAHEAD: 1, spd.OPT_TWO_STEP: 1, spd.OPT_PAIR_ROWS: -1, spd.OPT_SYRK_DEEP_ROWS: -1,
                spd.OPT_RECT_TALL_ROWS: 16384, spd.OPT_TILE_LAUNCH: 1, spd.OPT_TILE_WAIT_US: 2000000,
                spd.OPT_COLUMN_FIRST_ROWS: 8192, spd.OPT_TILE_HOLD_ROWS: 8192, spd.OPT_SUBST_LAUNCH: 2097152, spd.OPT_TILE_UPDATE_ROWS: -1,
                spd.OPT_TRIPLE_ROWS: -1}
    for k, v in defaults.items():
        assert spd.get_option(k) == v
    assert lib.spd_set_option(0, 1) == -1
    assert lib.spd_set_option(13, 1) == -1
    assert lib.spd_get_option(13) == -(1 << 63)
    assert lib.spd_set_option(spd.OPT_LOOKAHEAD, 2) == -2
    assert lib.spd_set_option(spd.OPT_TWO_STEP, -1) == -2
    assert lib.spd_set_option(spd.OPT_PAIR_ROWS, -2) == -2
    assert lib.spd_set_option(spd.OPT_RECT_TALL_ROWS, -1) == -2
    assert lib.spd_set_option(spd.OPT_TILE_LAUNCH, 2) == -2
    assert lib.spd_set_option(spd.OPT_TILE_WAIT_US, -1) == -2
    assert lib.spd_set_option(spd.OPT_COLUMN_FIRST_ROWS, -1) == -2
    assert lib.spd_set_option(spd.OPT_TILE_HOLD_ROWS, -1) == -2
    assert lib.spd_set_option(spd.OPT_SUBST_LAUNCH, -1) == -2
    assert lib.spd_set_option(spd.OPT_TILE_UPDATE_ROWS, -2) == -2
    assert lib.spd_set_option(spd.OPT_TRIPLE_ROWS, -2) == -2
    with spd.options({spd.OPT_PAIR_ROWS: 0, spd.OPT_LOOKAHEAD: 0, spd.OPT_RECT_TALL_ROWS: 7}):
        assert spd.get_option(spd.OPT_PAIR_ROWS) == 0
        assert spd.get_option(spd.OPT_LOOKAHEAD) == 0
        assert spd.get_option(spd.OPT_RECT_TALL_ROWS) == 7
    for k, v in defaults.items():
        assert spd.get_option(k) == v
    # a rejected value inside the block leaves every option as it was
    with pytest.raises(ValueError, match="argument 2"):
        with spd.options({spd.OPT_PAIR_ROWS: 0, spd.OPT_LOOKAHEAD: 5}):
            pass
    for k, v in defaults.items():
        assert spd.get_option(k) == v
    spd.set_option(spd.OPT_SYRK_DEEP_ROWS, 5)
    spd.set_option(spd.OPT_SYRK_DEEP_ROWS, spd.OPT_DEFAULT)
    assert spd.get_option(spd.OPT_SYRK_DEEP_ROWS) == -1
    assert lib.spd_release() == 0  # nothing created on this thread: nothing to do


# ------------------------------------------------------------ generator ---

@pytest.mark.parametrize("dt", ["f64", "f32", "c128", "c64"])
def test_generator_exact_symmetry_and_layout(dt):
    A = spdgen.make_A(96, dt, 0.5, seed=3, lda=100)
    assert A.shape == (96, 96) and A.stride() == (1, 100)
    assert torch.equal(A, A.mH)
    if A.is_complex():
        assert torch.all(torch.diagonal(A).imag == 0)
    ev = torch.linalg.eigvalsh(A.to(torch.complex128 if A.is_complex() else torch.float64))
    assert ev.min() > 0.4  # spectrum shifted by delta = 0.5


def test_generator_reproducible_and_seeded():
    a1 = spdgen.make_A(50, "f64", 0.1, seed=1)
    a2 = spdgen.make_A(50, "f64", 0.1, seed=1)
    a3 = spdgen.make_A(50, "f64", 0.1, seed=2)
    assert torch.equal(a1, a2) and not torch.equal(a1, a3)
    b1 = spdgen.make_B(50, 3, "f64", seed=1)
    assert b1.stride() == (1, 50)
    # B does not depend on how G was drawn
    assert torch.equal(b1, spdgen.make_B(50, 3, "f64", seed=1))


def test_generator_blocks_threads_invariant():
    # more than one 1024-row block: the blocks come from independent child streams
    g = spdgen.gaussian(2100, 3, False, 0, 0)
    g2 = spdgen.gaussian(2100, 3, False, 0, 0)
    assert np.array_equal(g, g2)
    assert abs(g.mean()) < 0.1 and abs(g.std() - 1) < 0.1


def test_config_table():
    assert spdgen.CONFIGS[5] == dict(dtype="f64", n=32768, nrhs=128, T_A=512, delta=0.05, logdet=True)
    assert spdgen.CONFIGS[3]["dtype"] == "f32" and not spdgen.CONFIGS[3]["logdet"]


def test_fp32_workload_rounding():
    # G rounded to fp32, Gram in double, rounded once, then delta added in fp32
    A = spdgen.make_A(40, "f32", 1.0, seed=4)
    assert A.dtype == torch.float32
    g = torch.from_numpy(spdgen.gaussian(40, 40, False, 4, 0)).float().double()
    ref = ((g @ g.T) * (1.0 / 40)).float()
    ref = torch.tril(ref, -1) + torch.tril(ref, -1).T + torch.diag(torch.diagonal(ref))
    ref.diagonal().add_(torch.tensor(1.0, dtype=torch.float32))
    assert torch.equal(A, ref)


def test_diag_benchmark_input():
    A, B = spdgen.diag_benchmark(5, 2)
    assert torch.equal(torch.diagonal(A), torch.arange(1, 6, dtype=torch.float64))
    assert torch.count_nonzero(A) == 5 and torch.all(B == 1)
