// Non-GEMM kernels of the dense SPD/HPD solve on gfx950: the LDS-resident
// leaf factorization / inversion, the deterministic log-determinant and the
// small data-movement helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "spd_gemm.hpp"

namespace spd {

constexpr int LEAF = 64;  // largest diagonal block factored inside LDS

struct LeafArgs {
    void *A;        // matrix base (column-major, lda)
    int64_t lda;
    void *Inv;      // inverse storage base
    int64_t ldi;    // leading dimension of one inverse tile
    int64_t sInv;   // elements between consecutive inverse tiles
    int n;          // matrix order
    int T;          // tile size (leaves never straddle a tile boundary)
    int lpt;        // leaves per tile = ceil(T / LEAF)
    int factor;     // 1: factor the leaf and invert it; 0: L is given, invert only
    int *info;      // factor mode: set to (col0 + first failing column + 1)
    int col0;       // global column of A[0, 0] (for info)
};

// Leaf handled by workgroup g: its first global column c0 (relative to the
// matrix base), its order lb and the element offset of its inverse from Inv.
// False when the workgroup has no leaf (ragged last tile).
__host__ __device__ inline bool leaf_geom(const LeafArgs &p, int g, int64_t &c0, int &lb, int64_t &ioff)
{
    const int t = g / p.lpt, b = g - t * p.lpt;
    const int64_t tc = (int64_t)t * p.T;
    if (tc >= p.n)
        return false;
    const int tk = (int)((p.T < p.n - tc) ? p.T : p.n - tc);
    if (b * LEAF >= tk)
        return false;
    lb = (LEAF < tk - b * LEAF) ? LEAF : tk - b * LEAF;
    c0 = tc + (int64_t)b * LEAF;
    ioff = (int64_t)t * p.sInv + (int64_t)b * LEAF * (1 + p.ldi);
    return true;
}

// One workgroup per leaf.  Leaf w lies in tile t = w / lpt at leaf slot
// b = w % lpt: columns c = t*T + b*LEAF ... of the matrix.
//
// factor = 1: right-looking unblocked Cholesky of the leaf's lower triangle in
// LDS (pivot from the real part of the diagonal; a pivot that is not > 0,
// including NaN, stops the factorization and records info), then L is written
// back over the lower triangle (diagonal imaginary parts set to 0) and inv(L)
// is written to the inverse storage with explicit zeros above the diagonal.
// The inverse is built alongside: L X = I is solved row by row, row j of X
// being final once column j of L is, and then removed from the rows below.
//
// factor = 0: the leaf already holds L; only inv(L) is produced.
//
// Thread (r, g) = (tid % 64, tid / 64) owns row r of the leaf and of its
// inverse, columns g, g + 4, g + 8, ...: every column step is a few LDS
// read-modify-writes per thread with no index division, and the values of
// column j a wave needs are the same for all its lanes (LDS broadcasts).
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) leaf_kernel(const LeafArgs p)
{
    typedef typename Elem<R, CPLX>::type E;
    constexpr int NP = CPLX ? 2 : 1;
    constexpr int LD = LEAF + 1;
    constexpr int G = 4;           // column phases (waves)
    __shared__ R S[NP][LEAF][LD];  // S[.][c][r] = L(r, c)
    __shared__ R X[NP][LEAF][LD];  // X[.][c][r] = inv(L)(r, c)
    __shared__ R dg[LEAF];

    if (p.info != nullptr && *p.info != 0)
        return;
    int64_t c0, ioff;
    int lb;
    if (!leaf_geom(p, (int)blockIdx.x, c0, lb, ioff))
        return;
    E *A = (E *)p.A + c0 + c0 * p.lda;
    E *Inv = (E *)p.Inv + ioff;
    const int tid = threadIdx.x;
    const int r = tid & (LEAF - 1), g = tid / LEAF;

    for (int c = g; c < lb; c += G) {
        R re = 0, im = 0;
        if (r < lb && r >= c)
            Elem<R, CPLX>::load(A + r + (int64_t)c * p.lda, re, im);
        if (r == c)
            im = 0;
        S[0][c][r] = re;
        if constexpr (CPLX) S[NP - 1][c][r] = im;
        X[0][c][r] = (r == c) ? R(1) : R(0);
        if constexpr (CPLX) X[NP - 1][c][r] = 0;
    }
    __syncthreads();

    for (int j = 0; j < lb; ++j) {
        R ljj;
        if (p.factor) {
            const R d = S[0][j][j];
            if (!(d > R(0))) {  // uniform: every thread read the same pivot
                if (tid == 0)
                    atomicCAS(p.info, 0, (int)(p.col0 + c0 + j + 1));
                return;
            }
            ljj = sqrt(d);
        } else {
            ljj = S[0][j][j];
        }
        const R rinv = R(1) / ljj;
        // column j of L below the diagonal (phase 0), row j of inv(L) (phase 1)
        if (g == 0 && p.factor && r > j && r < lb) {
            S[0][j][r] *= rinv;
            if constexpr (CPLX) S[NP - 1][j][r] *= rinv;
        }
        if (g == 1 && r <= j) {
            X[0][r][j] *= rinv;
            if constexpr (CPLX) X[NP - 1][r][j] *= rinv;
        }
        if (p.factor && tid == 0)
            dg[j] = ljj;
        __syncthreads();
        if (r > j && r < lb) {
            const R ar = S[0][j][r];
            const R ai = CPLX ? S[NP - 1][j][r] : R(0);
            if (p.factor) {
                // trailing lower triangle: S(r, c) -= L(r, j) conj(L(c, j)), j < c <= r
                for (int c = j + 1 + g; c <= r; c += G) {
                    const R br = S[0][j][c];
                    if constexpr (CPLX) {
                        const R bi = S[1][j][c];
                        S[0][c][r] -= ar * br + ai * bi;
                        S[1][c][r] -= ai * br - ar * bi;
                    } else {
                        S[0][c][r] -= ar * br;
                    }
                }
            }
            // rows below j of inv(L): X(r, c) -= L(r, j) X(j, c), c <= j < r
            for (int c = g; c <= j; c += G) {
                const R xr = X[0][c][j];
                if constexpr (CPLX) {
                    const R xi = X[1][c][j];
                    X[0][c][r] -= ar * xr - ai * xi;
                    X[1][c][r] -= ar * xi + ai * xr;
                } else {
                    X[0][c][r] -= ar * xr;
                }
            }
        }
        __syncthreads();
    }

    for (int c = g; c < lb; c += G) {
        if (r >= lb)
            continue;
        if (p.factor && r >= c) {
            if (r == c)
                Elem<R, CPLX>::store(A + r + (int64_t)c * p.lda, dg[c], R(0));
            else
                Elem<R, CPLX>::store(A + r + (int64_t)c * p.lda, S[0][c][r], CPLX ? S[NP - 1][c][r] : R(0));
        }
        if (r >= c)
            Elem<R, CPLX>::store(Inv + r + (int64_t)c * p.ldi, X[0][c][r], CPLX ? X[NP - 1][c][r] : R(0));
        else
            Elem<R, CPLX>::store(Inv + r + (int64_t)c * p.ldi, R(0), R(0));
    }
}

// log det A = 2 * sum_i log(Re L_ii), accumulated in double.  One workgroup;
// thread t owns the diagonal entries i = t, t + 1024, ... and the partial sums
// are combined by a fixed binary tree, so the result is the same bits on every
// run.  NaN if the factorization reported a failure.
template <typename R, bool CPLX>
__global__ void __launch_bounds__(1024) logdet_kernel(const void *Lv, int64_t lda, int64_t n,
                                                      const int *info, double *out)
{
    typedef typename Elem<R, CPLX>::type E;
    const E *L = (const E *)Lv;
    __shared__ double red[1024];
    const int tid = threadIdx.x;
    double s = 0.0;
    for (int64_t i = tid; i < n; i += 1024) {
        R re, im;
        Elem<R, CPLX>::load(L + i * (1 + lda), re, im);
        s += log((double)re);
    }
    red[tid] = s;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if (tid < w)
            red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0)
        *out = (info != nullptr && *info != 0) ? __longlong_as_double(0x7ff8000000000000LL) : 2.0 * red[0];
}

__global__ void set_int_kernel(int *p, int v) { *p = v; }

// dst(0:m, 0:n) = src(0:m, 0:n)
template <typename E>
__global__ void __launch_bounds__(256) copy2d_kernel(E *dst, int64_t ldd, const E *src, int64_t lds,
                                                     int64_t m, int64_t n, const int *info)
{
    if (info != nullptr && *info != 0)
        return;
    const int64_t total = m * n;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e % m, j = e / m;
        dst[i + j * ldd] = src[i + j * lds];
    }
}

// dst(0:m, 0:n) = 0 (all bits zero)
template <typename E>
__global__ void __launch_bounds__(256) zero2d_kernel(E *dst, int64_t ldd, int64_t m, int64_t n)
{
    const int64_t total = m * n;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e % m, j = e / m;
        E z;
        memset(&z, 0, sizeof(E));
        dst[i + j * ldd] = z;
    }
}

// If the factorization failed, every entry of the solution is NaN.
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) nan_fill_kernel(void *Bv, int64_t ldb, int64_t m, int64_t n,
                                                       const int *info)
{
    typedef typename Elem<R, CPLX>::type E;
    if (info == nullptr || *info == 0)
        return;
    E *B = (E *)Bv;
    const R qnan = (R)__longlong_as_double(0x7ff8000000000000LL);
    const int64_t total = m * n;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e % m, j = e / m;
        Elem<R, CPLX>::store(B + i + j * ldb, qnan, qnan);
    }
}

}  // namespace spd
