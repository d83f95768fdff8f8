// Host-side launch validator of the dense SPD/HPD solver.
//
// When switched on (spd_debug_validate), every kernel launch is first replayed
// on the host: each workgroup and thread of the launch computes, with the same
// index arithmetic the kernel itself uses (tile enumeration, k ranges, the
// loaders' thread-to-element maps, leaf_geom, acc_row), the addresses it would
// read or write, and each access must lie inside one of the buffers the caller
// passed to the entry point (the matrix, the right-hand side, the workspace,
// info, the log-determinant); a write must also be to a buffer the entry point
// may modify.  The first violation stops the call with SPD_ERR_CHECK and a
// message naming the kernel, the workgroup, the thread and the address.
//
// Mode 2 ("dry run") validates without touching the GPU at all, so the whole
// launch sequence of any problem shape can be checked on a machine without a
// GPU.  The replay is exhaustive (every thread of every workgroup), so it is
// meant for small and medium shapes.
#pragma once

#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <string>
#include <vector>

#include "spd_gemm.hpp"
#include "spd_kernels.hpp"
#include "spd_rect.hpp"
#include "spd_subst.hpp"
#include "spd_syrk.hpp"
#include "spd_tile.hpp"

namespace spd {

struct Region {
    uintptr_t lo, hi;
    bool writable;
    const char *name;
};

struct Checker {
    std::vector<Region> regions;
    std::string err;

    void begin()
    {
        regions.clear();
        err.clear();
    }
    void add(const void *p, size_t bytes, bool writable, const char *name)
    {
        if (p != nullptr && bytes > 0)
            regions.push_back({(uintptr_t)p, (uintptr_t)p + bytes, writable, name});
    }
    bool access(const void *p, size_t bytes, bool write, const char *kernel, long wg, long th)
    {
        const uintptr_t a = (uintptr_t)p, b = a + bytes;
        for (const Region &r : regions) {
            if (a >= r.lo && b <= r.hi) {
                if (write && !r.writable)
                    break;
                return true;
            }
        }
        char buf[256];
        snprintf(buf, sizeof buf, "%s: workgroup %ld thread %ld %s %zu bytes at %p outside every %s buffer",
                 kernel, wg, th, write ? "writes" : "reads", bytes, p, write ? "writable" : "");
        err = buf;
        return false;
    }
};

// Replay of gemm_kernel (spd_gemm.hpp): element-wise bounds-checked operand
// loads of the k slices [kbeg, kend), the C prologue (beta) and the epilogue.
template <typename R, bool CPLX, int BM, int BN, int KB, int WM, int WN, bool AT, bool BT>
static bool check_gemm(const GemmArgs &p, dim3 grid, Checker &c)
{
    typedef typename Elem<R, CPLX>::type E;
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int LA = BM * KB / NT, LB = BN * KB / NT;
    const char *kn = "gemm_kernel";
    if (p.info != nullptr && !c.access(p.info, 4, false, kn, 0, 0))
        return false;
    for (unsigned z = 0; z < grid.z; ++z) {
        const int zo = (int)z / p.nb_inner, zi = (int)z - zo * p.nb_inner;
        const E *A = (const E *)p.A + zo * p.sA_out + zi * p.sA_in;
        const E *B = (const E *)p.B + zo * p.sB_out + zi * p.sB_in;
        E *C = (E *)p.C + zo * p.sC_out + zi * p.sC_in;
        for (unsigned b = 0; b < grid.x; ++b) {
            const long wg = (long)z * grid.x + b;
            int I, J;
            const int t = xcd_remap((int)b, p.ntiles);
            if (p.tri) {
                tri_index(t, I, J);
            } else {
                I = t % p.tiles_m;
                J = t / p.tiles_m;
            }
            const int i0 = I * BM, j0 = J * BN, m = p.m, n = p.n;
            int kbeg = 0, kend = p.k;
            switch (p.kmode) {
            case KM_END_BY_J: kend = std::min(kend, j0 + BN); break;
            case KM_BEG_BY_J: kbeg = j0; break;
            case KM_END_BY_I: kend = std::min(kend, i0 + BM); break;
            case KM_BEG_BY_I: kbeg = i0; break;
            default: break;
            }
            kbeg = (kbeg / KB) * KB;
            for (int tid = 0; tid < NT; ++tid) {
                const int lane = tid & 63, wave = tid >> 6;
                const int wm = wave % WM, wn = wave / WM;
                const int li = lane & 15, lk = lane >> 4;
                const int ib = wm * TM, jb = wn * TN;
                for (int k0 = kbeg; k0 < kend; k0 += KB) {
                    for (int q = 0; q < LA; ++q) {
                        const int e = tid + NT * q;
                        const int i = AT ? e / KB : e % BM, kk = AT ? e % KB : e / BM;
                        const int gi = i0 + i, gk = k0 + kk;
                        if (gi < m && gk < kend) {
                            const E *src = AT ? (A + gk + (int64_t)gi * p.lda) : (A + gi + (int64_t)gk * p.lda);
                            if (!c.access(src, sizeof(E), false, kn, wg, tid))
                                return false;
                        }
                    }
                    for (int q = 0; q < LB; ++q) {
                        const int e = tid + NT * q;
                        const int j = BT ? e % BN : e / KB, kk = BT ? e / BN : e % KB;
                        const int gj = j0 + j, gk = k0 + kk;
                        if (gj < n && gk < kend) {
                            const E *src = BT ? (B + gj + (int64_t)gk * p.ldb) : (B + gk + (int64_t)gj * p.ldb);
                            if (!c.access(src, sizeof(E), false, kn, wg, tid))
                                return false;
                        }
                    }
                }
                for (int fi = 0; fi < FM; ++fi)
                    for (int fj = 0; fj < FN; ++fj)
                        for (int q = 0; q < 4; ++q) {
                            const int i = i0 + ib + fi * 16 + li, j = j0 + jb + fj * 16 + acc_row<R>(lk, q);
                            if (p.beta && i < m && j < n &&
                                !c.access(C + i + (int64_t)j * p.ldc, sizeof(E), false, kn, wg, tid))
                                return false;
                            if (i < m && j < n && (!p.tri || i >= j) &&
                                !c.access(C + i + (int64_t)j * p.ldc, sizeof(E), true, kn, wg, tid))
                                return false;
                        }
            }
        }
    }
    return true;
}

// Replay of syrk_kernel (spd_syrk.hpp): whole-tile vector loads of both row
// blocks of W for every slice, and the epilogue's read-modify-write of C.
template <typename R, bool CPLX, int BM, int KB, int WM, int WN, bool BIGLD, bool PK = false>
static bool check_syrk(const SyrkArgs &p, dim3 grid, Checker &c)
{
    typedef typename SyrkOff<BIGLD>::type Off;
    typedef typename Elem<R, CPLX>::type E;
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BM / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    typedef SyrkLoad<R, CPLX, BM, KB, NT> LD;
    const char *kn = "syrk_kernel";
    if (p.info != nullptr && !c.access(p.info, 4, false, kn, 0, 0))
        return false;
    if (p.ldw % BM != 0 || p.kp % KB != 0 || p.kp <= 0) {
        c.err = "syrk_kernel: panel layout is not whole tiles and slices";
        return false;
    }
    for (unsigned b = 0; b < grid.x; ++b) {
        int I, J;
        syrk_tile(p, (int)b, I, J);
        const int i0 = I * BM, j0 = J * BM;
        const bool rectm = p.ncols > 0;
        if (rectm ? (I >= p.tiles || (int64_t)J * BM >= p.ncols || p.krange != SYRK_K_ALL)
                  : (I >= p.tiles || J > I || (p.jt_end > 0 && J >= p.jt_end))) {
            c.err = "syrk_kernel: workgroup maps outside the lower tiles";
            return false;
        }
        const E *W = (const E *)p.W;
        const E *Vc = (const E *)p.V;
        int kb, ke;
        syrk_krange<BM>(p, i0, j0, kb, ke);
        if (kb < 0 || ke > p.kp || kb >= ke || kb % KB != 0 || ke % KB != 0 ||
            (p.kp1 > 0 && (p.kp1 % KB != 0 || p.kp1 >= p.kp || kb != 0))) {
            c.err = "syrk_kernel: depth range outside the panel or not whole slices";
            return false;
        }
        for (int tid = 0; tid < NT; ++tid) {
            for (int k0 = kb; k0 < ke; k0 += KB)
                for (int q = 0; q < LD::L; ++q) {
                    int r, k;
                    LD::coords(tid, q, r, k);
                    const uint32_t off = (uint32_t)(r + (int64_t)k * p.ldw);
                    if (r + LD::V > BM || k >= KB) {
                        c.err = "syrk_kernel: load outside its tile slice";
                        return false;
                    }
                    const bool second = p.kp1 > 0 && k0 >= p.kp1;
                    const E *Wp = second ? (const E *)p.W2 : W, *Vp = second ? (const E *)p.V2 : Vc;
                    const int64_t kk0 = second ? k0 - p.kp1 : k0;
                    if (!c.access(Wp + i0 + kk0 * p.ldw + off, LD::V * sizeof(E), false, kn, b, tid) ||
                        !c.access(Vp + j0 + kk0 * p.ldw + off, LD::V * sizeof(E), false, kn, b, tid))
                        return false;
                }
            const int lane = tid & 63, wave = tid >> 6;
            const int wm = wave % WM, wn = wave / WM;
            const int li = lane & 15, lk = lane >> 4;
            const int ib = wm * TM, jb = wn * TN;
            const bool whole = rectm ? (i0 + BM <= p.m && j0 + BM <= p.ncols) : ((I != J) && (i0 + BM <= p.m));
            E *Ct = (E *)p.C + i0 + (int64_t)j0 * p.ldc;
            constexpr int RA = SyrkPack<R, PK, FM>::value, RB = SyrkPack<R, PK, FN>::value;
            // whole tiles with 16-byte access to C: RA adjacent rows per vector
            const bool vec = RA > 1 && whole && p.vecc;
            for (int fi = 0; fi < FM; ++fi)
                for (int fj = 0; fj < FN; ++fj)
                    for (int q = 0; q < 4; ++q) {
                        const int i = ib + pk_index<RA>(fi, li), j = jb + pk_index<RB>(fj, acc_row<R>(lk, q));
                        if (vec && fi % RA != 0)
                            continue;  // inside the vector of fragment fi - fi % RA
                        if (whole || (i0 + i < p.m && (rectm ? j0 + j < p.ncols : i0 + i >= j0 + j))) {
                            const int64_t full = i + (int64_t)j * p.ldc;
                            if ((int64_t)(Off)full != full) {
                                c.err = "syrk_kernel: offset into C does not fit its type";
                                return false;
                            }
                            E *dst = Ct + (Off)full;
                            const size_t bytes = vec ? RA * sizeof(E) : sizeof(E);
                            if (vec && (uintptr_t)dst % 16 != 0) {
                                c.err = "syrk_kernel: unaligned vector access to C";
                                return false;
                            }
                            if (!c.access(dst, bytes, false, kn, b, tid) || !c.access(dst, bytes, true, kn, b, tid))
                                return false;
                        }
                    }
        }
    }
    return true;
}

// Replay of rect_kernel (spd_rect.hpp): the P loads (whole vectors on the
// fast path, element by element with the row and column masks otherwise), the
// unmasked Q vectors, and the epilogue's read-modify-write of C.
template <typename R, int BM, int BN, int KB, int WM, int WN, bool PT, bool VEC, bool STORE = false>
static bool check_rect(const RectArgs &p, dim3 grid, Checker &c)
{
    constexpr int NT = 64 * WM * WN;
    typedef RectLoad<R, BM, BN, KB, NT, PT> LD;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int V = LD::V;
    const char *kn = "rect_kernel";
    if (p.info != nullptr && !c.access(p.info, 4, false, kn, 0, 0))
        return false;
    if (p.ldq % BN != 0 || p.kp % KB != 0 || p.kp <= 0 || p.kvalid > p.kp || (int64_t)p.tiles_m * BM < p.m ||
        (int64_t)p.ntiles != (int64_t)p.tiles_m * ((p.n + BN - 1) / BN)) {
        c.err = "rect_kernel: operand layout is not whole tiles and slices";
        return false;
    }
    for (unsigned b = 0; b < grid.x; ++b) {
        const int t = xcd_remap((int)b, p.ntiles);
        const int I = t % p.tiles_m, J = t / p.tiles_m;
        const int i0 = I * BM, j0 = J * BN;
        if ((int64_t)j0 >= p.ldq) {
            c.err = "rect_kernel: workgroup maps past the operand buffer";
            return false;
        }
        const bool prows = i0 + BM <= p.m;
        const R *P = (const R *)p.P + (PT ? (int64_t)i0 * p.ldp : (int64_t)i0);
        const R *Q = (const R *)p.Q + j0;
        const int kend = rect_slices<BN, KB, STORE>(p, j0) * KB;
        for (int tid = 0; tid < NT; ++tid) {
            for (int k0 = 0; k0 < kend; k0 += KB) {
                const R *pa = P + (PT ? (int64_t)k0 : (int64_t)k0 * p.ldp);
                const R *qb = Q + (int64_t)k0 * p.ldq;
                const bool fast = prows && k0 + KB <= p.kvalid;
                for (int q = 0; q < LD::LP; ++q) {
                    int r, k;
                    LD::p_coords(tid, q, r, k);
                    const int64_t off = PT ? (k + (int64_t)r * p.ldp) : (r + (int64_t)k * p.ldp);
                    if (fast) {
                        if (VEC && ((uintptr_t)(pa + off)) % 16 != 0) {
                            c.err = "rect_kernel: unaligned vector load of P";
                            return false;
                        }
                        if (!c.access(pa + off, 16, false, kn, b, tid))
                            return false;
                    } else {
                        for (int v = 0; v < V; ++v) {
                            const int i = i0 + r + (PT ? 0 : v), kk = k0 + k + (PT ? v : 0);
                            if (i < p.m && kk < p.kvalid && !c.access(pa + off + v, sizeof(R), false, kn, b, tid))
                                return false;
                        }
                    }
                }
                for (int q = 0; q < LD::LQ; ++q) {
                    int r, k;
                    LD::q_coords(tid, q, r, k);
                    if (!c.access(qb + r + (int64_t)k * p.ldq, 16, false, kn, b, tid))
                        return false;
                }
            }
            const int lane = tid & 63, wave = tid >> 6;
            const int wm = wave % WM, wn = wave / WM;
            const int li = lane & 15, lk = lane >> 4;
            const int ib = wm * TM, jb = wn * TN;
            const bool whole = prows && (j0 + BN <= p.n);
            R *Ct = (R *)p.C + i0 + (int64_t)j0 * p.ldc;
            for (int fi = 0; fi < FM; ++fi)
                for (int fj = 0; fj < FN; ++fj)
                    for (int q = 0; q < 4; ++q) {
                        const int i = ib + fi * 16 + li, j = jb + fj * 16 + acc_row<R>(lk, q);
                        if (whole || (i0 + i < p.m && j0 + j < p.n)) {
                            R *dst = Ct + i + (int64_t)j * p.ldc;
                            if ((!STORE && !c.access(dst, sizeof(R), false, kn, b, tid)) ||
                                !c.access(dst, sizeof(R), true, kn, b, tid))
                                return false;
                        }
                    }
        }
    }
    return true;
}

// panel: the leaf + panel launch (leaf16_kernel<R, true>): every workgroup
// factors the one leaf; workgroup 0 writes it and its inverse, workgroup
// w >= 1 reads and writes rows [64(w-1), 64w) of the p.prows panel rows.
template <typename R, bool CPLX>
static bool check_leaf(const LeafArgs &p, unsigned grid, Checker &c, bool panel = false)
{
    typedef typename Elem<R, CPLX>::type E;
    const char *kn = panel ? "leaf16_kernel (leaf + panel)" : "leaf16_kernel";
    if (p.info != nullptr && !c.access(p.info, 4, p.factor != 0, kn, 0, 0))
        return false;
    if (panel && (p.ctr == nullptr || !c.access(p.ctr, 4, true, kn, 0, 0))) {
        if (c.err.empty())
            c.err = "leaf16_kernel (leaf + panel): no workgroup counter";
        return false;
    }
    for (unsigned g = 0; g < grid; ++g) {
        int64_t c0, ioff;
        int lb;
        if (!leaf_geom(p, panel ? 0 : (int)g, c0, lb, ioff))
            continue;
        const E *A = (const E *)p.A + c0 + c0 * p.lda;
        const E *Inv = (const E *)p.Inv + ioff;
        const bool writes_leaf = true;  // with panel, whichever workgroup finishes last
        for (int col = 0; col < lb; ++col)
            for (int r = 0; r < lb; ++r) {
                if (r >= col) {
                    if (!c.access(A + r + (int64_t)col * p.lda, sizeof(E), false, kn, g, 0))
                        return false;
                    if (writes_leaf && p.factor && !c.access(A + r + (int64_t)col * p.lda, sizeof(E), true, kn, g, 0))
                        return false;
                }
                if (writes_leaf && !c.access(Inv + r + (int64_t)col * p.ldi, sizeof(E), true, kn, g, 0))
                    return false;
            }
        if (panel && g > 0) {
            const E *Pb = A + lb + (int64_t)(g - 1) * LEAF;
            const int prow = std::min<int>(LEAF, p.prows - (int)(g - 1) * LEAF);
            for (int col = 0; col < lb; ++col)
                for (int r = 0; r < prow; ++r)
                    if (!c.access(Pb + r + (int64_t)col * p.lda, sizeof(E), false, kn, g, 0) ||
                        !c.access(Pb + r + (int64_t)col * p.lda, sizeof(E), true, kn, g, 0))
                        return false;
        }
    }
    return true;
}

// Replay of tile_kernel / tile_kernel_c (spd_tile.hpp).  Per role, the
// column segments of the blocks it reads (the diagonal blocks of the inverse
// as whole squares) and writes (each segment one contiguous access), the
// flags it waits for and raises, and the order: every flag a workgroup waits
// for must be raised by exactly one workgroup of a smaller id (so that waits
// only ever point back to workgroups dispatched before them).
template <typename R, bool CPLX>
static bool check_tile(const TileArgs &p, unsigned grid, Checker &c)
{
    typedef typename Elem<R, CPLX>::type E;
    const char *kn = CPLX ? "tile_kernel_c" : "tile_kernel";
    const int nb = p.nb;
    if (nb < 1 || nb * LEAF < p.tk || (nb - 1) * LEAF >= p.tk || grid != (unsigned)tile_groups(nb)) {
        c.err = "tile_kernel: block count does not match the tile order";
        return false;
    }
    if (p.info != nullptr && !c.access(p.info, 4, true, kn, 0, 0))
        return false;
    const int nflags = tile_flag_ints(nb);
    if (!c.access(p.flags, 4 * (size_t)nflags, true, kn, 0, 0))
        return false;
    // producer of every flag: L blocks at i nb + j, inverse blocks at nb^2 + i nb + b
    std::vector<int> prod(2 * nb * nb, -1);
    auto raise = [&](int f, int g) {
        if (prod[f] >= 0) {
            c.err = "tile_kernel: a flag is raised by two workgroups";
            return false;
        }
        prod[f] = g;
        return true;
    };
    for (unsigned g = 0; g < grid; ++g) {
        int i, j;
        const int kind = tile_role(nb, (int)g, i, j);
        if (kind == TILE_D) {
            if (j > 0 && !raise(i * nb + j - 1, (int)g))
                return false;
            if (!raise(i * nb + i, (int)g))
                return false;
        } else if (kind == TILE_O) {
            if (!raise(i * nb + j, (int)g))
                return false;
        } else if (kind == TILE_X) {
            if (!raise(nb * nb + i * nb + j, (int)g))
                return false;
        } else {
            c.err = "tile_kernel: a workgroup without a role";
            return false;
        }
    }
    const E *A = (const E *)p.D, *Iv = (const E *)p.Inv;
    auto nrows = [&](int b) { return std::min(LEAF, p.tk - b * LEAF); };
    // columns [0, nc) of block (bi, bj) of M (ld), rows [0, nr) (lower: rows >= column)
    auto blk = [&](const E *M, int64_t ld, int bi, int bj, int nr, int nc, bool lower, bool write, unsigned g) {
        for (int col = 0; col < nc; ++col) {
            const int r0 = lower ? col : 0;
            if (r0 >= nr)
                continue;
            const E *e = M + (int64_t)bi * LEAF + r0 + ((int64_t)bj * LEAF + col) * ld;
            if (!c.access(e, sizeof(E) * (size_t)(nr - r0), write, kn, g, 0))
                return false;
        }
        return true;
    };
    auto waits = [&](unsigned g, int f) {
        if (f < 0 || f >= 2 * nb * nb || prod[f] < 0 || prod[f] >= (int)g) {
            char buf[160];
            snprintf(buf, sizeof buf, "tile_kernel: workgroup %u waits for flag %d, raised by workgroup %d", g, f,
                     (f >= 0 && f < 2 * nb * nb) ? prod[f] : -2);
            c.err = buf;
            return false;
        }
        return true;
    };
    // the tile's own trailing update: rows [0, nr) of block b of W, columns [0, wk)
    const E *Wp = (const E *)p.W;
    auto wblk = [&](int b, int nr, unsigned g) {
        for (int col = 0; col < p.wk; ++col)
            if (!c.access(Wp + (int64_t)b * LEAF + (int64_t)col * p.ldw, sizeof(E) * (size_t)nr, false, kn, g, 0))
                return false;
        return true;
    };
    if (p.wk > 0 && (Wp == nullptr || p.ldw < p.tk)) {
        c.err = "tile_kernel: the previous panel does not cover the tile";
        return false;
    }
    for (unsigned g = 0; g < grid; ++g) {
        int i, j;
        const int kind = tile_role(nb, (int)g, i, j);
        const int nr = nrows(i);
        if (p.wk > 0 && kind == TILE_D && (!wblk(j, nr, g) || (j > 0 && !wblk(j - 1, LEAF, g))))
            return false;
        if (p.wk > 0 && kind == TILE_O && (!wblk(i, nr, g) || !wblk(j, LEAF, g)))
            return false;
        if (kind == TILE_D) {
            if (!blk(A, p.lda, j, j, nr, nr, true, false, g) || !blk(A, p.lda, j, j, nr, nr, true, true, g) ||
                !blk(Iv, p.ldi, j, j, nr, nr, false, true, g))
                return false;
            if (j > 0) {
                if (!blk(A, p.lda, j, j - 1, nr, LEAF, false, false, g) ||
                    !blk(A, p.lda, j, j - 1, nr, LEAF, false, true, g) || !waits(g, (j - 1) * nb + j - 1) ||
                    !blk(Iv, p.ldi, j - 1, j - 1, LEAF, LEAF, false, false, g))
                    return false;
            }
            for (int l = 0; l + 1 < j; ++l)
                if (!waits(g, j * nb + l) || !waits(g, (j - 1) * nb + l) ||
                    !blk(A, p.lda, j, l, nr, LEAF, false, false, g) ||
                    !blk(A, p.lda, j - 1, l, LEAF, LEAF, false, false, g))
                    return false;
        } else if (kind == TILE_O) {
            if (!blk(A, p.lda, i, j, nr, LEAF, false, false, g) || !blk(A, p.lda, i, j, nr, LEAF, false, true, g) ||
                !waits(g, j * nb + j) || !blk(Iv, p.ldi, j, j, LEAF, LEAF, false, false, g))
                return false;
            for (int l = 0; l < j; ++l)
                if (!waits(g, i * nb + l) || !waits(g, j * nb + l) ||
                    !blk(A, p.lda, i, l, nr, LEAF, false, false, g) ||
                    !blk(A, p.lda, j, l, LEAF, LEAF, false, false, g))
                    return false;
        } else {
            const int b = j;
            if (!waits(g, i * nb + i) || !blk(Iv, p.ldi, i, i, nr, nr, false, false, g) ||
                !blk(Iv, p.ldi, i, b, nr, LEAF, false, true, g))
                return false;
            for (int k = b; k < i; ++k)
                if (!waits(g, i * nb + k) || !waits(g, k == b ? b * nb + b : nb * nb + k * nb + b) ||
                    !blk(A, p.lda, i, k, nr, LEAF, false, false, g) ||
                    !blk(Iv, p.ldi, k, b, LEAF, LEAF, false, false, g))
                    return false;
        }
    }
    return true;
}

// Replay of subst_kernel (spd_subst.hpp): the piece of every workgroup, the
// column segments each one reads and writes (the operand loads are masked to
// them), and that every counter a workgroup waits for is advanced only by
// workgroups of its own or later tile rows (each counter of (i, ct) by
// exactly the row pieces of tile row i), with the tile rows in id order from
// the last.
template <typename R, bool CPLX, int TC>
static bool check_subst(const SubstArgs &p, unsigned grid, Checker &c)
{
    typedef typename Elem<R, CPLX>::type E;
    const char *kn = "subst_kernel";
    if (p.nt < 1 || p.T < 1 || p.n < 1 || p.nrhs < 1 || (int64_t)(p.nt - 1) * p.T >= p.n ||
        (int64_t)p.nt * p.T < p.n || p.nr != (p.T + SUB_TR - 1) / SUB_TR || p.nc != (p.nrhs + TC - 1) / TC ||
        p.ldz < p.T || p.ldb < p.n || p.lda < p.n || grid != (unsigned)subst_groups(p)) {
        c.err = "subst_kernel: launch shape does not match the problem";
        return false;
    }
    if (p.info != nullptr && !c.access(p.info, 4, false, kn, 0, 0))
        return false;
    if (p.status != nullptr && !c.access(p.status, 4, true, kn, 0, 0))
        return false;
    if (!c.access(p.flags, 4 * (size_t)subst_flag_ints(p.nt, p.nc), true, kn, 0, 0))
        return false;
    // per (i, ct): pieces counted by the counters; per tile row: the ids it
    // spans
    std::vector<int> count(p.nt * p.nc, 0), row_lo(p.nt, INT32_MAX), row_hi(p.nt, -1);
    std::vector<char> seen((size_t)p.nt * p.nr * p.nc, 0);
    for (unsigned g = 0; g < grid; ++g) {
        int i, rt, ct;
        subst_piece(p, (int)g, i, rt, ct);
        if (i < 0 || i >= p.nt || rt < 0 || rt >= subst_rows(p, i) || ct < 0 || ct >= p.nc) {
            c.err = "subst_kernel: a workgroup without a piece";
            return false;
        }
        char &once = seen[(size_t)(i * p.nr + rt) * p.nc + ct];
        if (once) {
            c.err = "subst_kernel: two workgroups take the same piece";
            return false;
        }
        once = 1;
        ++count[i * p.nc + ct];
        row_lo[i] = std::min(row_lo[i], (int)g);
        row_hi[i] = std::max(row_hi[i], (int)g);
    }
    for (int i = 0; i < p.nt; ++i) {
        if (i + 1 < p.nt && row_lo[i] <= row_hi[i + 1]) {
            c.err = "subst_kernel: tile rows are not in id order from the last";
            return false;
        }
        for (int ct = 0; ct < p.nc; ++ct)
            if (count[i * p.nc + ct] != subst_rows(p, i)) {
                c.err = "subst_kernel: a counter does not count every row piece";
                return false;
            }
    }
    const E *A = (const E *)p.A, *Iv = (const E *)p.Inv, *G = (const E *)p.G;
    const E *B = (const E *)p.B, *Z = (const E *)p.Z;
    auto rows = [&](int ti) { return std::min(p.T, p.n - ti * p.T); };
    // rows [r0, r0 + nr) of columns [c0, c0 + nc) of M (ld)
    auto seg = [&](const E *M, int64_t ld, int64_t r0, int nr, int64_t c0, int nc, bool write, unsigned g) {
        for (int col = 0; col < nc && nr > 0; ++col)
            if (!c.access(M + r0 + (c0 + col) * ld, sizeof(E) * (size_t)nr, write, kn, g, 0))
                return false;
        return true;
    };
    // a counter of tile row j awaited by workgroup g of tile row i: j > i, or
    // j = i for the Z counter (the R parts of row i wait for later rows only)
    auto from = [&](unsigned g, int i, int j, bool same_row_ok) {
        if (j < i || (j == i && !same_row_ok)) {
            char buf[128];
            snprintf(buf, sizeof buf, "subst_kernel: workgroup %u (tile row %d) waits for tile row %d", g, i, j);
            c.err = buf;
            return false;
        }
        return true;
    };
    for (unsigned g = 0; g < grid; ++g) {
        int i, rt, ct;
        subst_piece(p, (int)g, i, rt, ct);
        const int tki = rows(i), r0 = rt * SUB_TR, c0 = ct * TC;
        const int nrow = std::min(SUB_TR, tki - r0), ncol = std::min(TC, p.nrhs - c0);
        const int64_t row0 = (int64_t)i * p.T;
        const E *Zi = Z + (i & 1) * p.ldz * p.nrhs;
        // R part
        if (!seg(B, p.ldb, row0 + r0, nrow, c0, ncol, false, g) || !seg(Zi, p.ldz, r0, nrow, c0, ncol, true, g))
            return false;
        // the last term (j = i + 2) is also the wait that frees buffer i % 2
        for (int j = p.nt - 1; j > i + 1; --j) {
            const int64_t rj = (int64_t)j * p.T;
            if (!from(g, i, j, false) || !seg(A, p.lda, rj, rows(j), row0 + r0, nrow, false, g) ||
                !seg(B, p.ldb, rj, rows(j), c0, ncol, false, g))
                return false;
        }
        // C part
        if (!from(g, i, i, true) || !seg(Iv + (int64_t)i * p.T * p.T, p.T, r0, tki - r0, r0, nrow, false, g) ||
            !seg(Zi, p.ldz, r0, tki - r0, c0, ncol, false, g) || !seg(B, p.ldb, row0 + r0, nrow, c0, ncol, true, g))
            return false;
        if (i + 1 < p.nt &&
            (!from(g, i, i + 1, false) ||
             !seg(G + (int64_t)(i + 1) * p.T * p.T, p.T, 0, rows(i + 1), r0, nrow, false, g) ||
             !seg(B, p.ldb, row0 + p.T, rows(i + 1), c0, ncol, false, g)))
            return false;
    }
    // a wait that runs out: the last workgroup fills X with NaN
    return seg(B, p.ldb, 0, p.n, 0, p.nrhs, true, 0);
}

// dst(0:m, 0:n) written, src(0:m, 0:n) read (either may be null)
template <typename E>
static bool check_2d(const char *kn, E *dst, int64_t ldd, const E *src, int64_t lds, int64_t m, int64_t n,
                     const int *info, Checker &c)
{
    if (info != nullptr && !c.access(info, 4, false, kn, 0, 0))
        return false;
    for (int64_t j = 0; j < n; ++j)
        for (int64_t i = 0; i < m; ++i) {
            if (dst != nullptr && !c.access(dst + i + j * ldd, sizeof(E), true, kn, 0, 0))
                return false;
            if (src != nullptr && !c.access(src + i + j * lds, sizeof(E), false, kn, 0, 0))
                return false;
        }
    return true;
}

// copy_t_kernel: dst(0:m, 0:n) and src(0:m, 0:n) as check_2d, and qt(j, i)
// for i < kp, j < n
template <typename E>
static bool check_copy_t(E *dst, int64_t ldd, E *qt, int64_t ldq, const E *src, int64_t lds, int64_t m,
                         int64_t n, int64_t kp, const int *info, Checker &c)
{
    const char *kn = "copy_t_kernel";
    if (!check_2d<E>(kn, dst, ldd, src, lds, m, n, info, c))
        return false;
    for (int64_t i = 0; i < kp; ++i)
        for (int64_t j = 0; j < n; ++j)
            if (!c.access(qt + j + i * ldq, sizeof(E), true, kn, 0, 0))
                return false;
    return true;
}

// reduce_copy_t_kernel: S partial blocks read, dst and qt as copy_t
template <typename E>
static bool check_reduce_copy_t(E *dst, int64_t ldd, E *qt, int64_t ldq, const E *part, int64_t ldp, int64_t sp,
                                int S, int64_t m, int64_t n, int64_t kp, const int *info, Checker &c)
{
    const char *kn = "reduce_copy_t_kernel";
    for (int z = 0; z < S; ++z)
        if (!check_2d<E>(kn, z == 0 ? dst : nullptr, ldd, part + z * sp, ldp, m, n, info, c))
            return false;
    for (int64_t i = 0; i < kp; ++i)
        for (int64_t j = 0; j < n; ++j)
            if (!c.access(qt + j + i * ldq, sizeof(E), true, kn, 0, 0))
                return false;
    return true;
}

// gp_loglik_kernel: Y(0:n, 0:nrhs) and the diagonal of L read, out written
template <typename R>
static bool check_gp_loglik(const R *Y, int64_t ldy, const R *L, int64_t lda, int64_t n, int64_t nrhs,
                            const int *info, double *out, Checker &c)
{
    const char *kn = "gp_loglik_kernel";
    if (!check_2d<R>(kn, nullptr, 0, Y, ldy, n, nrhs, info, c))
        return false;
    for (int64_t i = 0; i < n; ++i)
        if (!c.access(L + i * (1 + lda), sizeof(R), false, kn, 0, 0))
            return false;
    for (int64_t j = 0; j < nrhs; ++j)
        if (!c.access(out + j, sizeof(double), true, kn, j, 0))
            return false;
    return true;
}

// Generalized-eigenproblem helpers: element maps of herm_full_kernel,
// tril_kernel, copy_lower_kernel and the tile pairs of conj_transpose_kernel.
template <typename E>
static bool check_expand(const char *kn, const E *src, int64_t lds, E *dst, int64_t ldd, int64_t n, bool mirror,
                         Checker &c)
{
    for (int64_t j = 0; j < n; ++j)
        for (int64_t i = 0; i < n; ++i) {
            if (i >= j && !c.access(src + i + j * lds, sizeof(E), false, kn, 0, 0))
                return false;
            if (mirror && i < j && !c.access(src + j + i * lds, sizeof(E), false, kn, 0, 0))
                return false;
            if (!c.access(dst + i + j * ldd, sizeof(E), true, kn, 0, 0))
                return false;
        }
    return true;
}

template <typename E>
static bool check_copy_lower(E *A, int64_t lda, const E *M, int64_t ldm, int64_t n, const int *info, Checker &c)
{
    const char *kn = "copy_lower_kernel";
    if (info != nullptr && !c.access(info, 4, false, kn, 0, 0))
        return false;
    for (int64_t j = 0; j < n; ++j)
        for (int64_t i = j; i < n; ++i)
            if (!c.access(M + i + j * ldm, sizeof(E), false, kn, 0, 0) ||
                !c.access(A + i + j * lda, sizeof(E), true, kn, 0, 0))
                return false;
    return true;
}

template <typename E>
static bool check_conj_transpose(E *M, int64_t ldm, int64_t n, unsigned grid, const int *info, Checker &c)
{
    const char *kn = "conj_transpose_kernel";
    constexpr int TB = 32;
    if (info != nullptr && !c.access(info, 4, false, kn, 0, 0))
        return false;
    const int64_t tt = (n + TB - 1) / TB;
    if ((int64_t)grid != tt * (tt + 1) / 2) {
        c.err = "conj_transpose_kernel: grid is not the lower tile pairs";
        return false;
    }
    for (unsigned b = 0; b < grid; ++b) {
        int I, J;
        tri_index((int)b, I, J);
        const int64_t i0 = (int64_t)I * TB, j0 = (int64_t)J * TB;
        for (int cc = 0; cc < TB; ++cc)
            for (int t = 0; t < TB; ++t) {
                if (i0 + t < n && j0 + cc < n &&
                    (!c.access(M + (i0 + t) + (j0 + cc) * ldm, sizeof(E), false, kn, b, t) ||
                     !c.access(M + (i0 + t) + (j0 + cc) * ldm, sizeof(E), true, kn, b, t)))
                    return false;
                if (j0 + t < n && i0 + cc < n &&
                    (!c.access(M + (j0 + t) + (i0 + cc) * ldm, sizeof(E), false, kn, b, t) ||
                     !c.access(M + (j0 + t) + (i0 + cc) * ldm, sizeof(E), true, kn, b, t)))
                    return false;
            }
    }
    return true;
}

// Element maps of the blocked-reduction helpers: every element a thread of
// these grid-stride kernels touches, in each buffer.
template <typename E>
static bool check_region(const char *kn, const E *base, int64_t ld, int64_t rows, int64_t cols, bool write,
                         Checker &c)
{
    for (int64_t j = 0; j < cols; ++j)
        for (int64_t i = 0; i < rows; ++i)
            if (!c.access(base + i + j * ld, sizeof(E), write, kn, 0, 0))
                return false;
    return true;
}

template <typename E>
static bool check_gst_pack(const E *Y, int64_t ldy, const E *V, int64_t ldv, const E *L, int64_t ldl, E *P, E *Q,
                           int64_t ldw, E *X, int64_t ldx, int64_t m, int64_t tk, int64_t kh, Checker &c)
{
    const char *kn = "gst_pack_kernel";
    if (m > ldw || tk > kh) {
        c.err = "gst_pack_kernel: panel larger than its buffer";
        return false;
    }
    return check_region(kn, Y, ldy, m, tk, false, c) && check_region(kn, V, ldv, m, tk, false, c) &&
           check_region(kn, L, ldl, m, tk, false, c) && check_region(kn, X, ldx, m, tk, true, c) &&
           check_region(kn, P, ldw, ldw, 2 * kh, true, c) && check_region(kn, Q, ldw, ldw, 2 * kh, true, c);
}

template <typename E>
static bool check_lower_read(const char *kn, const E *L, int64_t ldl, int64_t n, Checker &c)
{
    for (int64_t j = 0; j < n; ++j)
        for (int64_t i = j; i < n; ++i)
            if (!c.access(L + i + j * ldl, sizeof(E), false, kn, 0, 0))
                return false;
    return true;
}

template <typename E>
static bool check_gst_lh(const E *L, int64_t ldl, E *X, int64_t ldx, int64_t n, Checker &c)
{
    const char *kn = "gst_lh_kernel";
    if (ldx < n || ldx % 32 != 0) {
        c.err = "gst_lh_kernel: leading dimension below n or not whole 32 x 32 tiles";
        return false;
    }
    return check_region(kn, X, ldx, ldx, ldx, true, c) && check_lower_read(kn, L, ldl, n, c);
}

template <typename E>
static bool check_gst_diag_tril(const E *L, int64_t ldl, E *D, int64_t n, int64_t T, int64_t nt, Checker &c)
{
    const char *kn = "gst_diag_tril_kernel";
    if (!check_region(kn, D, T * T, T * T, nt, true, c))
        return false;
    for (int64_t t = 0; t < nt; ++t)
        for (int64_t j = 0; j < T; ++j)
            for (int64_t i = j; i < T && t * T + i < n; ++i)
                if (!c.access(L + (t * T + i) + (t * T + j) * ldl, sizeof(E), false, kn, 0, 0))
                    return false;
    return true;
}

template <typename E>
static bool check_gst_half(E *W, int64_t ldw, const E *V, E *X, int64_t ldv, int64_t rows, int64_t p, Checker &c)
{
    const char *kn = "gst_half_kernel";
    return check_region(kn, W, ldw, rows, p, false, c) && check_region(kn, W, ldw, rows, p, true, c) &&
           check_region(kn, V, ldv, rows, p, false, c) && check_region(kn, X, ldv, rows, p, true, c);
}

template <typename E>
static bool check_panel_pack(const E *S0, int64_t ld0, const E *S1, int64_t ld1, E *D, int64_t ldw, int64_t m,
                             int64_t tk, int64_t kh, int halves, Checker &c)
{
    const char *kn = "panel_pack_kernel";
    if (m > ldw || tk > kh || halves < 1 || halves > 2) {
        c.err = "panel_pack_kernel: panel larger than its buffer";
        return false;
    }
    return check_region(kn, D, ldw, ldw, kh * halves, true, c) && check_region(kn, S0, ld0, m, tk, false, c) &&
           (halves == 1 || check_region(kn, S1, ld1, m, tk, false, c));
}

}  // namespace spd
