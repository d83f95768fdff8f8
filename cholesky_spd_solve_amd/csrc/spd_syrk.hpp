// Trailing update of the right-looking blocked Cholesky factorization on the
// gfx950 matrix cores (JAXMg paper, "Software design": the potrf step of
// potrs; this is the symmetric rank-T_A update that carries almost all of its
// flops):
//
//     C(i, j) -= sum_k W(i, k) * conj(W(j, k))      for 0 <= j <= i < m
//
// The same kernel computes C -/+= W V^H over the lower tiles for two
// different operands laid out alike (the rank-2k updates of the
// generalized-eigenproblem reduction), optionally with a per-tile depth range
// where the operands are known to be zero outside it.
//
// W is the freshly solved panel L21 (m x T_A), staged in the workspace with a
// layout this kernel can read without any bounds logic:
//   - leading dimension ldw is a multiple of the tile size BM, and rows
//     [m, ldw) are zero, so every row block of W is whole;
//   - the number of columns kp is a multiple of the slice depth KB, and columns
//     beyond the panel width are zero.
// Only C needs bounds: the tiles on the diagonal and those that cross row m.
//
// A workgroup owns one BM x BM tile (I, J), I >= J, of the lower triangle of
// C (of all of it, or of its first jt_end tile columns only), split over
// WM x WN wave64s; each wave holds (BM/WM) x (BM/WN) of C as
// 16x16 accumulator blocks of v_mfma_*_16x16x4.  W is consumed KB columns at
// a time: the next slice is loaded from HBM into registers (16-byte vector
// loads, 32-bit offsets from a uniform tile origin) while the current slice is
// read from LDS by the matrix cores; one barrier per slice.  Within a slice the
// operands of the next k-step are read from LDS ahead of the current one's
// matrix-core instructions.  C is read and
// written once, in the epilogue, one 16-row block at a time.
//
// Complex types keep real and imaginary parts in separate LDS planes and use
// four real MFMAs per complex multiply-add.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spd_gemm.hpp"

namespace spd {

struct SyrkArgs {
    const void *W;  // panel, column-major, leading dimension ldw (see above)
    const void *V;  // column operand, same layout (V == W: the symmetric update)
    const void *W2; // kp1 > 0: depth [kp1, kp) comes from W2 and V2 (depth 0 at
    const void *V2; // their column 0), same leading dimension: two panels side by side
    int kp1;
    int64_t ldw;
    void *C;        // trailing matrix, column-major, leading dimension ldc
    int64_t ldc;
    int m;          // order of C
    int kp;         // columns of W (a multiple of KB)
    int tiles;      // tile rows = ceil(m / BM)
    int jt_end;     // 0: every lower tile; > 0: only tile columns J < jt_end
    int tskip;      // lower triangle (jt_end = ncols = 0): the first tskip tiles of the row
                    // order are left alone (tskip = s (s + 1) / 2 leaves the leading
                    // s x s tiles, the diagonal tile the next launch updates itself)
    int ncols;      // 0: the lower triangle of the m x m C; > 0: every tile of the
                    // m x ncols C (rows of W against rows of V, no triangle)
    int ntiles;     // number of tiles updated (workgroups)
    int krange;     // depth range of tile (I, J): SYRK_K_ALL [0, kp), SYRK_K_ROW [i0, kp),
                    // SYRK_K_BAND [j0, i0 + BM) (the operands are zero outside it)
    int add;        // 1: C += W V^H instead of C -= W V^H
    int vecc;       // 1: C is 16-byte aligned with a leading dimension that keeps
                    // every column so (the packed-row kernel then moves whole
                    // tiles of C with 16-byte vectors)
    const int *info;  // if non-null and *info != 0 the kernel does nothing
};

enum { SYRK_K_ALL = 0, SYRK_K_ROW = 1, SYRK_K_BAND = 2 };

__device__ inline double fma_r(double a, double b, double c) { return __builtin_fma(a, b, c); }
__device__ inline float fma_r(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

// Depth range [kb, ke) of the tile at rows i0, columns j0 (multiples of BM,
// hence of the slice depth); shared with the host-side launch validator.
template <int BM>
__host__ __device__ inline void syrk_krange(const SyrkArgs &p, int i0, int j0, int &kb, int &ke)
{
    kb = 0;
    ke = p.kp;
    if (p.krange == SYRK_K_ROW) {
        kb = i0;
    } else if (p.krange == SYRK_K_BAND) {
        kb = j0;
        ke = i0 + BM < p.kp ? i0 + BM : p.kp;
    }
}

// Tile (I, J) of workgroup b: with ncols > 0 every tile of the rectangle in
// column order; otherwise the whole lower triangle in row order (past its
// first tskip tiles), or, with
// jt_end > 0, the first jt_end tile columns in column order (column J holds
// tiles I = J .. tiles - 1).  Workgroup ids are first remapped so consecutive
// tiles share an XCD.  Shared with the host-side launch validator.
__host__ __device__ inline void syrk_tile(const SyrkArgs &p, int b, int &I, int &J)
{
    int t = xcd_remap(b, p.ntiles);
    if (p.ncols > 0) {  // rectangle, column by column
        I = t % p.tiles;
        J = t / p.tiles;
        return;
    }
    if (p.jt_end <= 0) {
        tri_index(t + p.tskip, I, J);
        return;
    }
    J = 0;
    while (J + 1 < p.jt_end && t >= p.tiles - J) {
        t -= p.tiles - J;
        ++J;
    }
    I = J + t;
}

// Elements per 16-byte vector load and the loader's thread -> element map,
// shared with the host-side launch validator.
template <typename R, bool CPLX, int BM, int KB, int NT>
struct SyrkLoad {
    typedef typename Elem<R, CPLX>::type E;
    static constexpr int V = (int)(16 / sizeof(E));  // elements per vector
    static constexpr int NCH = BM / V;               // vectors per column of a tile
    static constexpr int L = BM * KB / (V * NT);     // vector loads per thread per operand
    static_assert(BM % V == 0 && (BM * KB) % (V * NT) == 0, "tile does not divide into vector loads");

    // row r (first of V) and column k of load q of thread tid, within a tile slice
    __host__ __device__ static inline void coords(int tid, int q, int &r, int &k)
    {
        const int e = tid + NT * q;
        r = (e % NCH) * V;
        k = e / NCH;
    }
};

// Offsets into C within a tile: 32-bit while BM columns of C span fewer than
// 2^32 elements, 64-bit beyond (BIGLD).
template <bool BIGLD> struct SyrkOff { typedef uint32_t type; };
template <> struct SyrkOff<true> { typedef int64_t type; };
constexpr int64_t SYRK_LD32 = INT64_C(1) << 24;  // leading dimensions below this use 32-bit offsets

// Packed rows.  Within a wave's TM x TN block of C, fragment f (of 16 rows,
// or of 16 columns) and lane index l (0..15) address row (column)
//     pk_index<RP>(f, l) = (f / RP) * 16 RP + RP l + f % RP,
// so the RP fragments f = RP g .. RP g + RP - 1 of one lane hold RP adjacent
// rows: one 16-byte LDS read gives a lane its operands for all of them, and
// the epilogue moves RP adjacent elements of a column of C per vector.
// RP = 1 is the plain layout (row 16 f + l).  Only which lane holds which row
// changes, not what is summed or in which order, so the results are the same
// bits for every RP.  Shared with the host-side launch validator.
template <int RP>
__host__ __device__ inline int pk_index(int f, int l)
{
    return (f / RP) * 16 * RP + RP * l + f % RP;
}

// Rows per 16-byte operand read: RP adjacent rows of W fill one vector, up to
// the number of fragments.
template <typename R, bool PK, int F>
struct SyrkPack {
    static constexpr int V = (int)(16 / sizeof(R));
    static constexpr int value = !PK ? 1 : (V < F ? V : F);
};

template <typename R, bool CPLX, int BM, int KB, int WM, int WN, bool BIGLD = false, bool PK = false>
__global__ void __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(PK ? 4 : 2)))
syrk_kernel(const SyrkArgs p)
{
    typedef typename SyrkOff<BIGLD>::type Off;
    typedef typename Elem<R, CPLX>::type E;
    typedef typename AccT<R>::type V4;
    typedef SyrkLoad<R, CPLX, BM, KB, 64 * WM * WN> LD;
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BM / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int NP = CPLX ? 2 : 1;
    constexpr int V = LD::V, L = LD::L;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(KB % 4 == 0, "KB must be a multiple of 4");
    static_assert(!(PK && CPLX), "packed rows are for real types");
    constexpr int RA = SyrkPack<R, PK, FM>::value, RB = SyrkPack<R, PK, FN>::value;
    static_assert(FM % RA == 0 && FN % RB == 0, "fragments do not pack");

    __shared__ __align__(16) R As[2][NP][KB][BM];  // As[.][.][k][r] = W(i0 + r, k0 + k)
    __shared__ __align__(16) R Bs[2][NP][KB][BM];  // Bs[.][.][k][r] = conj(W(j0 + r, k0 + k))

    int I, J;
    syrk_tile(p, (int)blockIdx.x, I, J);
    const int i0 = I * BM, j0 = J * BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int li = lane & 15, lk = lane >> 4;
    const int ib = wm * TM, jb = wn * TN;

    // per-thread element offsets inside a slice (identical for both operands)
    uint32_t off[L];
    int rr[L], kk[L];
#pragma unroll
    for (int q = 0; q < L; ++q) {
        LD::coords(tid, q, rr[q], kk[q]);
        off[q] = (uint32_t)(rr[q] + (int64_t)kk[q] * p.ldw);
    }

    int kb, ke;
    syrk_krange<BM>(p, i0, j0, kb, ke);
    const E *__restrict__ wa = (const E *)p.W + i0 + (int64_t)kb * p.ldw;  // slice origin, row block of C
    const E *__restrict__ wb = (const E *)p.V + j0 + (int64_t)kb * p.ldw;  // slice origin, column block
    const int64_t step = (int64_t)KB * p.ldw;

    R ra[L][V][NP], rb[L][V][NP];
    auto load = [&](const E *__restrict__ oa, const E *__restrict__ ob) {
#pragma unroll
        for (int q = 0; q < L; ++q) {
            if constexpr (CPLX && V == 1) {
                Elem<R, true>::load(oa + off[q], ra[q][0][0], ra[q][0][NP - 1]);
                Elem<R, true>::load(ob + off[q], rb[q][0][0], rb[q][0][NP - 1]);
            } else if constexpr (CPLX) {
                // two complex elements in one 16-byte vector
                typedef R vt __attribute__((ext_vector_type(4)));
                const vt x = *(const vt *)(oa + off[q]);
                const vt y = *(const vt *)(ob + off[q]);
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    ra[q][v][0] = x[2 * v];
                    ra[q][v][NP - 1] = x[2 * v + 1];
                    rb[q][v][0] = y[2 * v];
                    rb[q][v][NP - 1] = y[2 * v + 1];
                }
            } else {
                typedef R vt __attribute__((ext_vector_type(V)));
                const vt x = *(const vt *)(oa + off[q]);
                const vt y = *(const vt *)(ob + off[q]);
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    ra[q][v][0] = x[v];
                    rb[q][v][0] = y[v];
                }
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int q = 0; q < L; ++q)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                As[buf][0][kk[q]][rr[q] + v] = ra[q][v][0];
                Bs[buf][0][kk[q]][rr[q] + v] = rb[q][v][0];
                if constexpr (CPLX) {
                    As[buf][1][kk[q]][rr[q] + v] = ra[q][v][1];
                    Bs[buf][1][kk[q]][rr[q] + v] = -rb[q][v][1];  // conj(W(j, k))
                }
            }
    };

    V4 acc[NP][FM][FN];
#pragma unroll
    for (int c = 0; c < NP; ++c)
#pragma unroll
        for (int fi = 0; fi < FM; ++fi)
#pragma unroll
            for (int fj = 0; fj < FN; ++fj)
                acc[c][fi][fj] = V4{0, 0, 0, 0};

    load(wa, wb);
    // status word read alongside the first slice (the panel is valid whatever
    // it holds; nothing is written before it)
    if (p.info != nullptr && *p.info != 0)
        return;
    store(0);
    __syncthreads();
    int cur = 0;
    for (int k0 = kb; k0 < ke; k0 += KB) {
        const bool more = k0 + KB < ke;
        if (more) {
            if (k0 + KB == p.kp1) {  // second panel pair
                wa = (const E *)p.W2 + i0;
                wb = (const E *)p.V2 + j0;
            } else {
                wa += step;
                wb += step;
            }
            load(wa, wb);
        }
        // Operand fragments are double-buffered in registers: those of k-step
        // s+1 are read from LDS before the matrix-core instructions of k-step s
        // are issued, so the LDS latency hides behind them.
        R fa[2][NP][FM], fb[2][NP][FN];
        auto frag = [&](int kr, R (&a)[NP][FM], R (&b)[NP][FN]) {
            if constexpr (RA > 1 || RB > 1) {
                typedef R va __attribute__((ext_vector_type(RA)));
                typedef R vb __attribute__((ext_vector_type(RB)));
#pragma unroll
                for (int g = 0; g < FM / RA; ++g) {
                    const va x = *(const va *)&As[cur][0][kr][ib + pk_index<RA>(g * RA, li)];
#pragma unroll
                    for (int u = 0; u < RA; ++u)
                        a[0][g * RA + u] = x[u];
                }
#pragma unroll
                for (int g = 0; g < FN / RB; ++g) {
                    const vb y = *(const vb *)&Bs[cur][0][kr][jb + pk_index<RB>(g * RB, li)];
#pragma unroll
                    for (int u = 0; u < RB; ++u)
                        b[0][g * RB + u] = y[u];
                }
            } else {
#pragma unroll
                for (int c = 0; c < NP; ++c) {
#pragma unroll
                    for (int fi = 0; fi < FM; ++fi)
                        a[c][fi] = As[cur][c][kr][ib + fi * 16 + li];
#pragma unroll
                    for (int fj = 0; fj < FN; ++fj)
                        b[c][fj] = Bs[cur][c][kr][jb + fj * 16 + li];
                }
            }
        };
        frag(lk, fa[0], fb[0]);
#pragma unroll
        for (int s = 0; s < KB / 4; ++s) {
            if (s + 1 < KB / 4)
                frag((s + 1) * 4 + lk, fa[(s + 1) & 1], fb[(s + 1) & 1]);
            const R(&a)[NP][FM] = fa[s & 1];
            const R(&b)[NP][FN] = fb[s & 1];
#pragma unroll
            for (int fi = 0; fi < FM; ++fi)
#pragma unroll
                for (int fj = 0; fj < FN; ++fj) {
                    if constexpr (!CPLX) {
                        acc[0][fi][fj] = mfma16(b[0][fj], a[0][fi], acc[0][fi][fj]);
                    } else {
                        // re += br*ar - bi*ai ; im += bi*ar + br*ai
                        acc[0][fi][fj] = mfma16(b[0][fj], a[0][fi], acc[0][fi][fj]);
                        acc[0][fi][fj] = mfma16(-b[1][fj], a[1][fi], acc[0][fi][fj]);
                        acc[1][fi][fj] = mfma16(b[1][fj], a[0][fi], acc[1][fi][fj]);
                        acc[1][fi][fj] = mfma16(b[0][fj], a[1][fi], acc[1][fi][fj]);
                    }
                }
        }
        if (more)
            store(cur ^ 1);
        __syncthreads();
        cur ^= 1;
    }

    // ---- epilogue: C -= acc (C += acc when p.add), one 16-row block at a time;
    // fma(-1, acc, c) rounds exactly as c - acc
    const R sg = p.add ? R(1) : R(-1);
    E *__restrict__ Ct = (E *)p.C + i0 + (int64_t)j0 * p.ldc;
    const bool rectm = p.ncols > 0;
    const bool whole = rectm ? (i0 + BM <= p.m && j0 + BM <= p.ncols)
                             : ((I != J) && (i0 + BM <= p.m));  // every element of the tile is updated
    if constexpr (RA > 1) {
        if (whole && p.vecc) {
            // RA adjacent rows of one column of C per 16-byte vector
            typedef R va __attribute__((ext_vector_type(RA)));
#pragma unroll
            for (int g = 0; g < FM / RA; ++g) {
                const int i = ib + pk_index<RA>(g * RA, li);
#pragma unroll
                for (int fj = 0; fj < FN; ++fj) {
                    va cv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int j = jb + pk_index<RB>(fj, acc_row<R>(lk, q));
                        cv[q] = *(const va *)(Ct + (Off)(i + (int64_t)j * p.ldc));
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int j = jb + pk_index<RB>(fj, acc_row<R>(lk, q));
                        va o;
#pragma unroll
                        for (int u = 0; u < RA; ++u)
                            o[u] = fma_r(sg, acc[0][g * RA + u][fj][q], cv[q][u]);
                        *(va *)(Ct + (Off)(i + (int64_t)j * p.ldc)) = o;
                    }
                }
            }
            return;
        }
    }
#pragma unroll
    for (int fi = 0; fi < FM; ++fi) {
        const int i = ib + pk_index<RA>(fi, li);
        R cr[FN][4], ci[FN][4];
        if (whole) {
#pragma unroll
            for (int fj = 0; fj < FN; ++fj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = jb + pk_index<RB>(fj, acc_row<R>(lk, q));
                    ci[fj][q] = 0;
                    Elem<R, CPLX>::load(Ct + (Off)(i + (int64_t)j * p.ldc), cr[fj][q], ci[fj][q]);
                }
#pragma unroll
            for (int fj = 0; fj < FN; ++fj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = jb + pk_index<RB>(fj, acc_row<R>(lk, q));
                    Elem<R, CPLX>::store(Ct + (Off)(i + (int64_t)j * p.ldc),
                                         fma_r(sg, acc[0][fi][fj][q], cr[fj][q]),
                                         CPLX ? fma_r(sg, acc[NP - 1][fi][fj][q], ci[fj][q]) : R(0));
                }
        } else {
#pragma unroll
            for (int fj = 0; fj < FN; ++fj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = jb + pk_index<RB>(fj, acc_row<R>(lk, q));
                    if (i0 + i < p.m && (rectm ? j0 + j < p.ncols : i0 + i >= j0 + j)) {
                        E *dst = Ct + (Off)(i + (int64_t)j * p.ldc);
                        R xr, xi = 0;
                        Elem<R, CPLX>::load(dst, xr, xi);
                        Elem<R, CPLX>::store(dst, fma_r(sg, acc[0][fi][fj][q], xr),
                                             CPLX ? fma_r(sg, acc[NP - 1][fi][fj][q], xi) : R(0));
                    }
                }
        }
    }
}

}  // namespace spd
