// Block update of the blocked triangular solves on the gfx950 matrix cores
// (JAXMg paper, "Software design": the forward and back substitutions of
// potrs), real types:
//
//     C(i, j) -= sum_k P(i, k) * Q(j, k)        0 <= i < m, 0 <= j < n
//
// P is a block of the factor, read where it lies in A:
//   - forward substitution, B(below) -= L(below, k) X_k:  P(i, k) = P[i + k*ldp]
//   - back substitution, B(above) -= L(k, above)^T X_k (PT):  P(i, k) = P[k + i*ldp]
// Rows i >= m and columns k >= kvalid of P are never read (taken as zero).
// Q is the solved block X_k, transposed into the workspace by copy_t_kernel:
// Q(j, k) = Q[j + k*ldq] with ldq a multiple of BN, rows [n, ldq) and columns
// [kvalid, kp) zero, so it needs no bounds logic.
//
// The tile machinery is that of the trailing update (spd_syrk.hpp): a BM x BN
// tile of C per workgroup over WM x WN wave64s of v_mfma_*_16x16x4
// accumulators, KB-deep slices staged through registers with 16-byte loads
// into double-buffered LDS, operand fragments double-buffered in registers,
// one barrier per slice.  Whole tiles take unmasked (vector) loads; only
// tiles that cross row m or column kvalid of P load element by element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "spd_gemm.hpp"

namespace spd {

struct RectArgs {
    const void *P;  // factor block (see above)
    int64_t ldp;
    const void *Q;  // transposed solved block, ldq x kp, zero padded
    int64_t ldq;
    void *C;        // right-hand-side block, column-major, ldc
    int64_t ldc;
    int m, n;       // C is m x n
    int kp;         // columns of Q (a multiple of KB)
    int kvalid;     // columns of P that exist (<= kp)
    int tiles_m;    // ceil(m / BM); workgroup t -> tile (t % tiles_m, t / tiles_m)
    int ntiles;
    const int *info;  // if non-null and *info != 0 the kernel does nothing
};

// Thread -> element maps of the slice loads, shared with the host-side launch
// validator.  V elements per 16-byte vector.
//   Q, and P without PT: vectors run down the rows of a column
//                        (row r .. r+V-1 of slice column k);
//   P with PT:           vectors run along the slice columns of one row
//                        (row r, slice columns k .. k+V-1).
template <typename R, int BM, int BN, int KB, int NT, bool PT>
struct RectLoad {
    static constexpr int V = (int)(16 / sizeof(R));
    static constexpr int LP = BM * KB / (V * NT);  // P vectors per thread per slice
    static constexpr int LQ = BN * KB / (V * NT);  // Q vectors per thread per slice
    static_assert(LP >= 1 && LQ >= 1 && (BM * KB) % (V * NT) == 0 && (BN * KB) % (V * NT) == 0,
                  "tile does not divide into vector loads");
    static_assert(KB % V == 0, "slice depth must hold whole vectors");

    __host__ __device__ static inline void p_coords(int tid, int q, int &r, int &k)
    {
        const int e = tid + NT * q;
        if (PT) {
            r = e % BM;
            k = (e / BM) * V;
        } else {
            r = (e % (BM / V)) * V;
            k = e / (BM / V);
        }
    }
    __host__ __device__ static inline void q_coords(int tid, int q, int &r, int &k)
    {
        const int e = tid + NT * q;
        r = (e % (BN / V)) * V;
        k = e / (BN / V);
    }
};

// VEC: P may be read with 16-byte vectors (the host checked the alignment);
// otherwise the same elements are read one by one.  The arithmetic is the
// same either way, so results do not depend on the leading dimension.
// DEPTH: slices of P and Q in flight from memory (1: the next one; 2: the
// next two, in two register sets, for more bytes in flight per CU).
// STORE: C = P Q^T (C is not read) instead of C -= P Q^T.
// Slices of depth KB a workgroup whose tile starts at column j0 multiplies.
// STORE (the factorization's panel W = P inv(L_kk)^T, Q = inv(L_kk) lower
// triangular): Q(j, k) = 0 for k > j, so columns [j0, j0 + BN) need depth
// j0 + BN only; otherwise the whole depth kp.
template <int BN, int KB, bool STORE>
__host__ __device__ inline int rect_slices(const RectArgs &p, int j0)
{
    const int all = p.kp / KB;
    if (!STORE)
        return all;
    const int need = (j0 + BN + KB - 1) / KB;
    return need < all ? need : all;
}

template <typename R, int BM, int BN, int KB, int WM, int WN, bool PT, bool VEC, int DEPTH = 1, bool STORE = false>
__global__ void __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2)))
rect_kernel(const RectArgs p)
{
    typedef typename AccT<R>::type V4;
    constexpr int NT = 64 * WM * WN;
    typedef RectLoad<R, BM, BN, KB, NT, PT> LD;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int V = LD::V, LP = LD::LP, LQ = LD::LQ;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(KB % 4 == 0, "KB must be a multiple of 4");
    typedef R vt __attribute__((ext_vector_type(V)));

    __shared__ R As[2][KB][BM];  // As[.][k][r] = P(i0 + r, k0 + k)
    __shared__ R Bs[2][KB][BN];  // Bs[.][k][r] = Q(j0 + r, k0 + k)

    const int t = xcd_remap((int)blockIdx.x, p.ntiles);
    const int I = t % p.tiles_m, J = t / p.tiles_m;
    const int i0 = I * BM, j0 = J * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int li = lane & 15, lk = lane >> 4;
    const int ib = wm * TM, jb = wn * TN;

    int pr[LP], pk[LP], qr[LQ], qk[LQ];
    uint32_t poff[LP], qoff[LQ];
#pragma unroll
    for (int q = 0; q < LP; ++q) {
        LD::p_coords(tid, q, pr[q], pk[q]);
        poff[q] = PT ? (uint32_t)(pk[q] + (int64_t)pr[q] * p.ldp) : (uint32_t)(pr[q] + (int64_t)pk[q] * p.ldp);
    }
#pragma unroll
    for (int q = 0; q < LQ; ++q) {
        LD::q_coords(tid, q, qr[q], qk[q]);
        qoff[q] = (uint32_t)(qr[q] + (int64_t)qk[q] * p.ldq);
    }

    // slice origins: P(i0, k0) and Q(j0, k0)
    const R *__restrict__ pa = (const R *)p.P + (PT ? (int64_t)i0 * p.ldp : (int64_t)i0);
    const R *__restrict__ qb = (const R *)p.Q + j0;
    const int64_t pstep = PT ? (int64_t)KB : (int64_t)KB * p.ldp;
    const int64_t qstep = (int64_t)KB * p.ldq;
    const bool prows = i0 + BM <= p.m;  // every row of the P block exists

    static_assert(DEPTH == 1 || DEPTH == 2, "one or two slices in flight");
    R rga[DEPTH][LP][V], rgb[DEPTH][LQ][V];
    auto load = [&](R (&ra)[LP][V], R (&rb)[LQ][V], const R *__restrict__ oa, const R *__restrict__ ob, int k0) {
        if (prows && k0 + KB <= p.kvalid) {
#pragma unroll
            for (int q = 0; q < LP; ++q) {
                if constexpr (VEC) {
                    const vt x = *(const vt *)(oa + poff[q]);
#pragma unroll
                    for (int v = 0; v < V; ++v)
                        ra[q][v] = x[v];
                } else {
#pragma unroll
                    for (int v = 0; v < V; ++v)
                        ra[q][v] = oa[poff[q] + v];
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < LP; ++q)
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const int i = i0 + pr[q] + (PT ? 0 : v), k = k0 + pk[q] + (PT ? v : 0);
                    ra[q][v] = (i < p.m && k < p.kvalid) ? oa[poff[q] + v] : R(0);
                }
        }
#pragma unroll
        for (int q = 0; q < LQ; ++q) {
            const vt y = *(const vt *)(ob + qoff[q]);
#pragma unroll
            for (int v = 0; v < V; ++v)
                rb[q][v] = y[v];
        }
    };
    auto store = [&](const R (&ra)[LP][V], const R (&rb)[LQ][V], int buf) {
#pragma unroll
        for (int q = 0; q < LP; ++q)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                if (PT)
                    As[buf][pk[q] + v][pr[q]] = ra[q][v];
                else
                    As[buf][pk[q]][pr[q] + v] = ra[q][v];
            }
#pragma unroll
        for (int q = 0; q < LQ; ++q)
#pragma unroll
            for (int v = 0; v < V; ++v)
                Bs[buf][qk[q]][qr[q] + v] = rb[q][v];
    };

    V4 acc[FM][FN];
#pragma unroll
    for (int fi = 0; fi < FM; ++fi)
#pragma unroll
        for (int fj = 0; fj < FN; ++fj)
            acc[fi][fj] = V4{0, 0, 0, 0};

    const int nsl = rect_slices<BN, KB, STORE>(p, j0);
    load(rga[0], rgb[0], pa, qb, 0);
    if (DEPTH == 2 && nsl > 1)
        load(rga[DEPTH - 1], rgb[DEPTH - 1], pa + pstep, qb + qstep, KB);
    // status word read alongside the first slice (the operands are valid
    // whatever it holds; nothing is written before it)
    if (p.info != nullptr && *p.info != 0)
        return;
    store(rga[0], rgb[0], 0);
    __syncthreads();
    // Slice sl is read from LDS buffer sl % 2.  With DEPTH 2 the registers of
    // set sl % 2 are refilled with slice sl + 2 while slice sl is multiplied,
    // and set (sl + 1) % 2 (slice sl + 1, loaded one slice earlier) goes to LDS
    // after it; with DEPTH 1 slice sl + 1 is loaded and stored within it.
    auto body = [&](int sl, auto par) {
        constexpr int P = decltype(par)::value;  // sl % 2
        if (DEPTH == 2) {
            if (sl + 2 < nsl)
                load(rga[P % DEPTH], rgb[P % DEPTH], pa + (sl + 2) * pstep, qb + (sl + 2) * qstep, (sl + 2) * KB);
        } else if (sl + 1 < nsl) {
            load(rga[0], rgb[0], pa + (sl + 1) * pstep, qb + (sl + 1) * qstep, (sl + 1) * KB);
        }
        R fa[2][FM], fb[2][FN];
        auto frag = [&](int kr, R (&a)[FM], R (&b)[FN]) {
#pragma unroll
            for (int fi = 0; fi < FM; ++fi)
                a[fi] = As[P][kr][ib + fi * 16 + li];
#pragma unroll
            for (int fj = 0; fj < FN; ++fj)
                b[fj] = Bs[P][kr][jb + fj * 16 + li];
        };
        frag(lk, fa[0], fb[0]);
#pragma unroll
        for (int s = 0; s < KB / 4; ++s) {
            if (s + 1 < KB / 4)
                frag((s + 1) * 4 + lk, fa[(s + 1) & 1], fb[(s + 1) & 1]);
#pragma unroll
            for (int fi = 0; fi < FM; ++fi)
#pragma unroll
                for (int fj = 0; fj < FN; ++fj)
                    acc[fi][fj] = mfma16(fb[s & 1][fj], fa[s & 1][fi], acc[fi][fj]);
        }
        if (sl + 1 < nsl)
            store(rga[(P + 1) % DEPTH], rgb[(P + 1) % DEPTH], P ^ 1);
        __syncthreads();
    };
    for (int sl = 0; sl < nsl; sl += 2) {
        body(sl, std::integral_constant<int, 0>());
        if (sl + 1 < nsl)
            body(sl + 1, std::integral_constant<int, 1>());
    }

    // epilogue: C -= acc (or C = acc), one 16-row block at a time
    R *__restrict__ Ct = (R *)p.C + i0 + (int64_t)j0 * p.ldc;
    const bool whole = prows && (j0 + BN <= p.n);
    if constexpr (STORE) {
#pragma unroll
        for (int fi = 0; fi < FM; ++fi)
#pragma unroll
            for (int fj = 0; fj < FN; ++fj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = ib + fi * 16 + li, j = jb + fj * 16 + acc_row<R>(lk, q);
                    if (whole || (i0 + i < p.m && j0 + j < p.n))
                        Ct[i + (int64_t)j * p.ldc] = acc[fi][fj][q];
                }
        return;
    }
#pragma unroll
    for (int fi = 0; fi < FM; ++fi) {
        const int i = ib + fi * 16 + li;
        R cr[FN][4];
#pragma unroll
        for (int fj = 0; fj < FN; ++fj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = jb + fj * 16 + acc_row<R>(lk, q);
                cr[fj][q] = (whole || (i0 + i < p.m && j0 + j < p.n)) ? Ct[i + (int64_t)j * p.ldc] : R(0);
            }
#pragma unroll
        for (int fj = 0; fj < FN; ++fj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = jb + fj * 16 + acc_row<R>(lk, q);
                if (whole || (i0 + i < p.m && j0 + j < p.n))
                    Ct[i + (int64_t)j * p.ldc] = cr[fj][q] - acc[fi][fj][q];
            }
    }
}

// dst(0:m, 0:n) = src(0:m, 0:n) and qt(j, i) = src(i, j): the solved block
// goes back into B and, transposed, into the update's operand buffer; columns
// [m, kp) of qt are zeroed so the update reads no stale values past the block.
template <typename E>
__global__ void __launch_bounds__(256) copy_t_kernel(E *dst, int64_t ldd, E *qt, int64_t ldq, const E *src,
                                                     int64_t lds, int64_t m, int64_t n, int64_t kp, const int *info)
{
    if (info != nullptr && *info != 0)
        return;
    const int64_t total = kp * n;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e % kp, j = e / kp;
        if (i < m) {
            const E v = src[i + j * lds];
            dst[i + j * ldd] = v;
            qt[j + i * ldq] = v;
        } else {
            qt[j + i * ldq] = E{};
        }
    }
}

// dst(0:m, 0:n) = sum_{z < S} part_z(0:m, 0:n), summed in the order
// z = 0, 1, ..., S-1 (so the result is the same bits on every run), with
// part_z = part + z * sp (leading dimension ldp); qt(j, i) gets the same value
// transposed and columns [m, kp) of qt are zeroed, as copy_t_kernel does.
template <typename E>
__global__ void __launch_bounds__(256) reduce_copy_t_kernel(E *dst, int64_t ldd, E *qt, int64_t ldq, const E *part,
                                                            int64_t ldp, int64_t sp, int S, int64_t m, int64_t n,
                                                            int64_t kp, const int *info)
{
    if (info != nullptr && *info != 0)
        return;
    const int64_t total = kp * n;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e % kp, j = e / kp;
        if (i < m) {
            E v = part[i + j * ldp];
            for (int z = 1; z < S; ++z)
                v += part[z * sp + i + j * ldp];
            dst[i + j * ldd] = v;
            qt[j + i * ldq] = v;
        } else {
            qt[j + i * ldq] = E{};
        }
    }
}

}  // namespace spd
