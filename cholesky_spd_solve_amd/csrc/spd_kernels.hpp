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
    int prows;      // leaf + panel launch only: rows of the panel below the leaf
    int *ctr;       // leaf + panel launch only: workgroup counter, 0 between launches
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

// ---------------------------------------------------------------------------
// Leaf kernels: one workgroup per leaf.  Leaf w lies in tile t = w / lpt at
// leaf slot b = w % lpt: columns c = t*T + b*LEAF ... of the matrix.
//
// factor = 1: Cholesky factorization of the leaf's lower triangle (pivots from
// the real part of the diagonal; a pivot that is not > 0, NaN included,
// records info and the leaf is not written back), then L is written back
// over the lower triangle (diagonal imaginary parts 0) and inv(L) to the
// inverse storage with explicit zeros above the diagonal.
// factor = 0: the leaf already holds L; only inv(L) is produced.
//
// Blocked leaf for real types, with 16 x 16 sub-blocks:
//
//   for b = 0..3:  factor and invert the diagonal block (b, b)        (one wave)
//                  L(i, b) = A(i, b) inv(L(b, b))^T         i > b      (MFMA)
//                  A(i, j) -= L(i, b) L(j, b)^T        b < j <= i      (MFMA)
//   inv(L)(i, b) = -inv(L(i, i)) sum_{b<=k<i} L(i, k) inv(L)(k, b)    (MFMA,
//                  by increasing i - b)
//
// The 16 x 16 diagonal blocks are done in registers by one wave with no LDS
// traffic inside the column sweep: lane c holds column c of the symmetric
// block (which is also row c) and column c of the inverse; the entries L(r, j)
// reach the other lanes through DPP row broadcasts.  Every
// 16 x 16 x 16 product is four v_mfma_*_16x16x4 with operands read from LDS.
// Padding beyond lb is the identity.

// Value of x in lane `lane` of the wave (lane wave-uniform).
__device__ __forceinline__ double lane_value(double x, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float lane_value(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}
// Value of x in lane N of this lane's row of 16 lanes (DPP row_newbcast:N).
template <int N>
__device__ __forceinline__ double row_value(double x)
{
    const long long b = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(long long, x), 0x150 + N, 0xf, 0xf, true);
    return __builtin_bit_cast(double, b);
}
template <int N>
__device__ __forceinline__ float row_value(float x)
{
    const int b = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, true);
    return __builtin_bit_cast(float, b);
}
// acc += A B for 16 x 16 blocks in LDS: A(r, k) = pa[k * ak + r * ar],
// B(k, c) = pb[k * bk + c * bc].  Lane (li, lk) = (lane % 16, lane / 16) ends
// with C(li, acc_row(lk, q)) in acc[q].
template <typename R>
__device__ __forceinline__ typename AccT<R>::type mma16(const R *pa, int ak, int ar, const R *pb, int bk, int bc,
                                                        typename AccT<R>::type acc)
{
    const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int k = 4 * s + lk;
        const R a = pa[k * ak + li * ar];
        const R b = pb[k * bk + li * bc];
        acc = mfma16(b, a, acc);
    }
    return acc;
}

constexpr int LB16 = 16;         // sub-block order
constexpr int LDL = LEAF + 1;    // LDS row length of the leaf arrays

// 1/sqrt(d) for finite d > 0 (and sqrt(d) in sq), without branches.  With
// d = f 2^e (f in [1/2, 1)) and k = floor(e / 2), m = d 4^-k lies in [1/2, 2):
// the hardware reciprocal square root estimate y of m is refined by
// Goldschmidt's square-root iteration (R. E. Goldschmidt, "Applications of
// division by convergence", MIT, 1964; in the coupled form of P. Markstein,
// "Software division and square root using Goldschmidt's algorithms", RNC 6,
// 2004): g = m y -> sqrt(m) and h = y / 2 -> 1 / (2 sqrt(m)) are updated
// together by r = 1/2 - g h, g += g r, h += h r, each step squaring the
// relative error; the powers of two are then put back exactly.  Both results
// are within 2 units in the last place (checked against correctly rounded
// values over the whole exponent range by the factorization's tests).
__device__ __forceinline__ double rsqrt_refined(double d, double &sq)
{
    const int k = __builtin_amdgcn_frexp_exp(d) >> 1;
    const double m = __builtin_amdgcn_ldexp(d, -2 * k);
    const double y = __builtin_amdgcn_rsq(m);
    double g = m * y, h = 0.5 * y;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const double r = fma(-g, h, 0.5);
        g = fma(g, r, g);
        h = fma(h, r, h);
    }
    sq = __builtin_amdgcn_ldexp(g, k);
    return __builtin_amdgcn_ldexp(h + h, -k);
}
__device__ __forceinline__ float rsqrt_refined(float d, float &sq)
{
    const int k = __builtin_amdgcn_frexp_expf(d) >> 1;
    const float m = __builtin_amdgcn_ldexpf(d, -2 * k);
    const float y = __builtin_amdgcn_rsqf(m);
    float g = m * y, h = 0.5f * y;
    const float r = fmaf(-g, h, 0.5f);
    g = fmaf(g, r, g);
    h = fmaf(h, r, h);
    sq = __builtin_amdgcn_ldexpf(g, k);
    return __builtin_amdgcn_ldexpf(h + h, -k);
}

// b[r] = L(r, J) for r = R0 .. 15, each from lane r's a[J].
template <typename R, int J, int R0>
__device__ __forceinline__ void diag16_bcast(const R *a, R *b)
{
    if constexpr (R0 < LB16) {
        b[R0] = row_value<R0>(a[J]);
        diag16_bcast<R, J, R0 + 1>(a, b);
    }
}

// Scale of pivot column J: s = 1/L(J, J) and ljj = L(J, J) from the pivot
// lane J's a[J].  A pivot that is not > 0 (NaN included) is replaced by 1 and
// the first such column kept in bad; every lane sees the same pivot, so
// nothing diverges.
template <typename R, bool FACTOR, int J>
__device__ __forceinline__ void diag16_pivot(const R *a, R &s, R &ljj, int &bad)
{
    R d = row_value<J>(a[J]);
    if constexpr (FACTOR) {
        const bool ok = d > R(0);
        bad = (!ok && bad < 0) ? J : bad;
        d = ok ? d : R(1);
        s = rsqrt_refined(d, ljj);
    } else {
        ljj = d;
        s = R(1) / d;
    }
}

// Column J of the sweep below (its pivot scale s, ljj already known), then
// the columns after it.  The next pivot is computed right after row J + 1 is
// updated, ahead of the other rows, so its dependent chain overlaps them.
template <typename R, bool FACTOR, int J>
__device__ __forceinline__ void diag16_step(R *a, R *x, int c, R s, R ljj, int &bad)
{
    if constexpr (J < LB16) {
        if constexpr (FACTOR)
            a[J] = (c == J) ? ljj : a[J] * s;
        x[J] *= s;
        R s1 = R(0), l1 = R(0);
        if constexpr (J + 1 < LB16) {
            const R lrj = row_value<J + 1>(a[J]);  // L(J + 1, J)
            if constexpr (FACTOR)
                a[J + 1] -= lrj * a[J];
            x[J + 1] -= lrj * x[J];
            diag16_pivot<R, FACTOR, J + 1>(a, s1, l1, bad);
        }
        // The broadcasts of the column all go out first (into registers of
        // their own, pinned so the compiler cannot fold them back onto one),
        // so no update waits on the broadcast just before it.
        R b[LB16];
        diag16_bcast<R, J, J + 2>(a, b);
#pragma unroll
        for (int r = J + 2; r < LB16; ++r)
            asm volatile("" : "+v"(b[r]));
#pragma unroll
        for (int r = J + 2; r < LB16; ++r) {
            if constexpr (FACTOR)
                a[r] -= b[r] * a[J];
            x[r] -= b[r] * x[J];
        }
        // Pin the column's results for the rows past the next pivot here:
        // left alone, the compiler moves the updates of x past the later
        // columns and keeps all of their broadcasts live at once.
#pragma unroll
        for (int r = J + 2; r < LB16; ++r)
            asm volatile("" : "+v"(a[r]), "+v"(x[r]));
        diag16_step<R, FACTOR, J + 1>(a, x, c, s1, l1, bad);
    }
}

// Factor (FACTOR) and invert, or only invert, the 16 x 16 diagonal block at
// (o, o) of S (S[c][r] = element (r, c), lower triangle); L goes back to S
// (zeros above the diagonal), inv(L) to X.  One wave; lanes 16..63 repeat
// the work of lanes 0..15 and store nothing.  A pivot that is not > 0 records
// info (columns < lb only), sets *failed and is replaced by 1.
//
// Lane c keeps a[r] = A(r, c) = A(c, r) for all r.  Step j: the pivot is lane
// j's a[j]; every lane scales its a[j] by 1/L(j, j), which leaves L(c, j) in
// lane c; then A(r, c) -= L(r, j) L(c, j) for r > j with L(r, j) read from
// lane r.  The inverse is the forward substitution L x = e_c in lane c, which
// needs the same L(r, j) at the same step.
template <typename R, bool FACTOR>
__device__ void diag16(R (*S)[LDL], R (*X)[LDL], int o, int lb, int gcol, int *info, int *failed)
{
    const int lane = threadIdx.x & 63, c = lane & 15;
    R a[LB16], x[LB16];
#pragma unroll
    for (int r = 0; r < LB16; ++r) {
        a[r] = (r >= c) ? S[o + c][o + r] : S[o + r][o + c];
        x[r] = (r == c) ? R(1) : R(0);
    }
    int bad = -1;
    R s0, l0;
    diag16_pivot<R, FACTOR, 0>(a, s0, l0, bad);
    diag16_step<R, FACTOR, 0>(a, x, c, s0, l0, bad);
    if (FACTOR && bad >= 0 && lane == 0 && o + bad < lb) {
        if (info != nullptr)
            atomicCAS(info, 0, gcol + o + bad + 1);
        *failed = 1;
    }
    if (lane < LB16) {
#pragma unroll
        for (int r = 0; r < LB16; ++r) {
            if constexpr (FACTOR)
                S[o + r][o + c] = (r <= c) ? a[r] : R(0);  // row c of L
            X[o + c][o + r] = (r >= c) ? x[r] : R(0);      // column c of inv(L)
        }
    }
}

// Factor (factor) and invert, or only invert, the 64 x 64 block held in S
// (S[c][r] = element (r, c); lower triangle read; identity beyond lb): L
// goes back to S (zeros above the diagonal), inv(L) to X, which must hold
// zeros on entry.  All 256 threads of the workgroup take part (wave 0 sweeps
// the 16 x 16 diagonal blocks, the four waves share the 16 x 16 products);
// the block is in S and X and *failed is 0 before the call (with a barrier
// after the stores), and the results are there after it.  A pivot that is
// not > 0 records info at column gcol + its index (columns < lb only) and
// sets *failed.
template <typename R>
__device__ __forceinline__ void leaf_lds(R (*S)[LDL], R (*X)[LDL], R (*Tm)[LB16][LB16 + 1], bool factor, int lb,
                                         int gcol, int *info, int *failed)
{
    typedef typename AccT<R>::type V4;
    constexpr int NB = LEAF / LB16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lk = lane >> 4;
    // store the 16 x 16 accumulator block (lane layout of mma16) at (ro, co)
    // of M, scaled by sg; lower part only when low
    auto put = [&](R (*M)[LDL], int ro, int co, const V4 &acc, R sg, bool low) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int rr = li, cc = acc_row<R>(lk, qq);
            if (!low || rr >= cc)
                M[co + cc][ro + rr] = sg * acc[qq];
        }
    };

    // acc += sum_{k0 <= k < k1} L(i, k) X(k, b)
    auto tsum = [&](int i, int b, int k0, int k1, V4 &acc) {
        for (int k = k0; k < k1; ++k)
            acc = mma16<R>(&S[k * LB16][i * LB16], LDL, 1, &X[b * LB16][k * LB16], 1, LDL, acc);
    };
    // T to this wave's scratch (Tm[c][r] = T(r, c)), and back
    auto stage = [&](const V4 &acc) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
            Tm[wave][acc_row<R>(lk, qq)][li] = acc[qq];
    };
    auto unstage = [&](V4 &acc) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
            acc[qq] = Tm[wave][acc_row<R>(lk, qq)][li];
    };
    // X(i, b) = -inv(L(i, i)) T, T staged
    auto apply = [&](int i, int b) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS stores done before reading them back
        __builtin_amdgcn_wave_barrier();
        V4 acc2 = {0, 0, 0, 0};
        acc2 = mma16<R>(&X[i * LB16][i * LB16], LDL, 1, &Tm[wave][0][0], 1, LB16 + 1, acc2);
        put(X, i * LB16, b * LB16, acc2, R(-1), false);
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
    };
    static_assert(NB == 4, "the inverse schedule below is written for four sub-blocks");

    for (int b = 0; b < NB; ++b) {
        const int o = b * LB16;
        if (wave == 0) {
            if (factor)
                diag16<R, true>(S, X, o, lb, gcol, info, failed);
            else
                diag16<R, false>(S, X, o, lb, gcol, info, failed);
        } else if (b == 2 && wave == 1) {
            // beside the sweeps, the inverse blocks whose inputs are final
            // (partial sums of the last block row wait in the wave's scratch)
            V4 t = {0, 0, 0, 0};
            tsum(1, 0, 0, 1, t);
            stage(t);
            apply(1, 0);
        } else if (b == 3 && wave == 1) {
            V4 t = {0, 0, 0, 0};
            tsum(2, 1, 1, 2, t);
            stage(t);
            apply(2, 1);
            V4 t31 = {0, 0, 0, 0};
            tsum(3, 1, 1, 3, t31);
            stage(t31);
        } else if (b == 3 && wave == 2) {
            V4 t = {0, 0, 0, 0};
            tsum(2, 0, 0, 2, t);
            stage(t);
            apply(2, 0);
        } else if (b == 3 && wave == 3) {
            V4 t30 = {0, 0, 0, 0};
            tsum(3, 0, 0, 2, t30);
            stage(t30);
        }
        __syncthreads();
        if (factor) {
            // L(i, b) = A(i, b) inv(L(b, b))^T, one block per wave
            const int i = b + 1 + wave;
            if (i < NB) {
                V4 acc = {0, 0, 0, 0};
                acc = mma16<R>(&S[o][i * LB16], LDL, 1, &X[o][o], LDL, 1, acc);
                put(S, i * LB16, o, acc, R(1), false);
            }
            __syncthreads();
            // A(i, j) -= L(i, b) L(j, b)^T, b < j <= i
            for (int t = wave; t < (NB - 1 - b) * (NB - b) / 2; t += 4) {
                int ti, tj;
                tri_index(t, ti, tj);
                const int i2 = b + 1 + ti, j2 = b + 1 + tj;
                V4 acc = {0, 0, 0, 0};
                acc = mma16<R>(&S[o][i2 * LB16], LDL, 1, &S[o][j2 * LB16], LDL, 1, acc);
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int rr = li, cc = acc_row<R>(lk, qq);
                    if (i2 != j2 || rr >= cc)
                        S[j2 * LB16 + cc][i2 * LB16 + rr] -= acc[qq];
                }
            }
            __syncthreads();
        }
    }

    // the last block row of the inverse: X(3, b) = -inv(L(3, 3)) sum_k L(3, k) X(k, b)
    // (rows 1 and 2 and the partial sums above were formed beside the sweeps,
    // each sum in the order of k)
    if (wave == 0) {
        V4 t = {0, 0, 0, 0};
        tsum(3, 2, 2, 3, t);
        stage(t);
        apply(3, 2);
    } else if (wave == 1) {
        apply(3, 1);
    } else if (wave == 3) {
        V4 t = {0, 0, 0, 0};
        unstage(t);
        tsum(3, 0, 2, 3, t);
        stage(t);
        apply(3, 0);
    }
    __syncthreads();

}

// At most 256 registers per lane, so that a leaf fits in the registers one
// finishing trailing-update workgroup gives back.
//
// PANEL: one launch factors a single leaf and solves the panel below it,
// L(i, leaf) = A(i, leaf) inv(L_leaf)^T for the p.prows rows that follow the
// leaf.  Every workgroup factors and inverts the leaf in its own LDS (the same
// bits); workgroup w >= 1 also multiplies rows [64(w-1), 64w) of the panel by
// inv(L_leaf)^T in place.  L may only replace A's leaf once no workgroup still
// has to read it, so each workgroup counts itself out on p.ctr when done and
// the last one stores L and inv(L) and resets the counter (no workgroup waits
// for another).  Only workgroup 0 records info.  The panel rows are loaded
// together with the leaf.
template <typename R, bool PANEL = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) leaf16_kernel(const LeafArgs p)
{
    typedef typename AccT<R>::type V4;
    constexpr int NB = LEAF / LB16;  // 4 sub-blocks
    __shared__ R S[LEAF][LDL];       // S[c][r] = L(r, c)
    __shared__ R X[LEAF][LDL];       // X[c][r] = inv(L)(r, c)
    __shared__ R Tm[4][LB16][LB16 + 1];  // per-wave 16 x 16 scratch
    __shared__ int failed;

    int64_t c0, ioff;
    int lb;
    const int w = PANEL ? (int)blockIdx.x : 0;  // panel block of this workgroup (0: none)
    if (!leaf_geom(p, PANEL ? 0 : (int)blockIdx.x, c0, lb, ioff))
        return;
    R *A = (R *)p.A + c0 + c0 * p.lda;
    R *Inv = (R *)p.Inv + ioff;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, lk = lane >> 4;
    const int r = tid & (LEAF - 1), g = tid / LEAF;
    int *const info = (w == 0) ? p.info : nullptr;
    R *const Pb = A + lb + (int64_t)(w - 1) * LEAF;  // panel block w: rows lb + 64(w-1) + r
    const int prow = p.prows - (w - 1) * LEAF;       // its rows that exist

    // all loads of the leaf (and of the panel block) are in flight together
    // (one memory round trip), and the status word is read alongside them
    R v[LEAF / 4], pv[PANEL ? LEAF / 4 : 1];
#pragma unroll
    for (int k = 0; k < LEAF / 4; ++k) {
        const int c = g + 4 * k;
        v[k] = (r == c) ? R(1) : R(0);
        if (r < lb && c < lb && r >= c)
            v[k] = A[r + (int64_t)c * p.lda];
        if constexpr (PANEL) {
            pv[k] = R(0);
            if (w > 0 && r < prow && c < lb)
                pv[k] = Pb[r + (int64_t)c * p.lda];
        }
    }
    if (p.info != nullptr && *p.info != 0)
        return;
#pragma unroll
    for (int k = 0; k < LEAF / 4; ++k) {
        S[g + 4 * k][r] = v[k];
        X[g + 4 * k][r] = R(0);
    }
    if (tid == 0)
        failed = 0;
    __syncthreads();

    leaf_lds<R>(S, X, Tm, p.factor != 0, lb, p.col0 + (int)c0, info, &failed);

    if (failed)
        return;
    // L and inv(L) into registers first (every LDS read, then the global
    // stores back to back; and the panel block may take S's place)
    R sv[LEAF / 4], xv[LEAF / 4];
#pragma unroll
    for (int k = 0; k < LEAF / 4; ++k) {
        sv[k] = S[g + 4 * k][r];
        xv[k] = X[g + 4 * k][r];
    }
    if constexpr (PANEL) {
        if (w > 0) {
            // panel block B (rows of this workgroup) into S, then
            // P = B inv(L)^T: wave v owns the 16-row block v, P(v, j) =
            // sum_{k <= j} B(v, k) inv(L)(j, k) over 16 x 16 blocks
            __syncthreads();
#pragma unroll
            for (int k = 0; k < LEAF / 4; ++k)
                S[g + 4 * k][r] = pv[k];
            __syncthreads();
#pragma unroll
            for (int bj = 0; bj < NB; ++bj) {
                V4 acc = {0, 0, 0, 0};
                for (int bk = 0; bk <= bj; ++bk)
                    acc = mma16<R>(&S[bk * LB16][wave * LB16], LDL, 1, &X[bk * LB16][bj * LB16], LDL, 1, acc);
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int rr = wave * LB16 + li, cc = bj * LB16 + acc_row<R>(lk, qq);
                    if (rr < prow && cc < lb)
                        Pb[rr + (int64_t)cc * p.lda] = acc[qq];
                }
            }
        }
        // count out; the last workgroup stores the leaf
        __shared__ int last;
        __syncthreads();
        if (tid == 0) {
            last = atomicAdd(p.ctr, 1) == (int)gridDim.x - 1;
            if (last)
                atomicExch(p.ctr, 0);
        }
        __syncthreads();
        if (!last)
            return;
    }
#pragma unroll
    for (int k = 0; k < LEAF / 4; ++k) {
        const int c = g + 4 * k;
        if (r < lb && c < lb) {
            if (p.factor && r >= c)
                A[r + (int64_t)c * p.lda] = sv[k];
            Inv[r + (int64_t)c * p.ldi] = (r >= c) ? xv[k] : R(0);
        }
    }
}

// ---------------------------------------------------------------------------
// Blocked leaf for complex types: leaf16_kernel's scheme with real and
// imaginary parts in separate LDS planes.
//
//   for b = 0..3:  factor and invert the diagonal block (b, b)        (one wave)
//                  L(i, b) = A(i, b) inv(L(b, b))^H         i > b      (MFMA)
//                  A(i, j) -= L(i, b) L(j, b)^H        b < j <= i      (MFMA)
//   inv(L)(i, b) = -inv(L(i, i)) sum_{b<=k<i} L(i, k) inv(L)(k, b)
//
// The diagonal block sweep gives each of the wave's four rows of 16 lanes one
// real plane: lane 16 g + c holds the real (g = 0) and imaginary (g = 1)
// parts of row c of the Hermitian block, and those of column c of the
// inverse (g = 2, 3).  Step j: the pivot is row 0's lane j; every lane
// scales its entry j by 1/L(j, j), which leaves L(c, j) in lane c of rows 0
// and 1; then A(c, r) -= L(c, j) conj(L(r, j)) and x[r] -= L(r, j) x[j] for
// r > j are one real update y[r] -= P Re L(r, j) + Q Im L(r, j) in every
// lane, with P its own entry j and Q the partner plane's (signed).  Every
// complex 16 x 16 x 16 product is sixteen v_mfma_*_16x16x4 (four per complex
// multiply-add).
//
// LDS: one array S per plane holds L in its lower triangle (S[c][r] =
// L(r, c), r >= c) and the strict lower triangle of inv(L) in its upper one
// (S[r][c] = inv(L)(r, c), r > c); inv(L)'s diagonal is kept apart.  That is
// 85 KB in all, so a leaf fits on a CU beside one trailing-update workgroup.

// acc += A B for complex 16 x 16 blocks whose elements come from fa(r, k, re,
// im) and fb(k, c, re, im).  Lane layout as mma16.
template <typename R, typename FA, typename FB>
__device__ __forceinline__ void mma16c(FA fa, FB fb, typename AccT<R>::type &cr, typename AccT<R>::type &ci)
{
    const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int k = 4 * s + lk;
        R a0, a1, b0, b1;
        fa(li, k, a0, a1);
        fb(k, li, b0, b1);
        cr = mfma16(b0, a0, cr);
        cr = mfma16(-b1, a1, cr);
        ci = mfma16(b1, a0, ci);
        ci = mfma16(b0, a1, ci);
    }
}

// As mma16c with A's operands already in registers: a*[s] = A(li, 4 s + lk).
template <typename R, typename FB>
__device__ __forceinline__ void mma16c_ra(const R (&ar)[4], const R (&ai)[4], FB fb, typename AccT<R>::type &cr,
                                          typename AccT<R>::type &ci)
{
    const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        R b0, b1;
        fb(4 * s + lk, li, b0, b1);
        cr = mfma16(b0, ar[s], cr);
        cr = mfma16(-b1, ai[s], cr);
        ci = mfma16(b1, ar[s], ci);
        ci = mfma16(b0, ai[s], ci);
    }
}

// Exchanges between the four rows of 16 lanes (gfx950 permlane swaps):
// row_pairs gives e = [v0, v0, v2, v2] and o = [v1, v1, v3, v3] (row by
// row), low_half [x0, x1, x0, x1]; lane_value the value of lane N.
__device__ __forceinline__ double f64_of(unsigned lo, unsigned hi)
{
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
__device__ __forceinline__ void row_pairs(double v, double &e, double &o)
{
    const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
    const auto l = __builtin_amdgcn_permlane16_swap((unsigned)b, (unsigned)b, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((unsigned)(b >> 32), (unsigned)(b >> 32), false, false);
    e = f64_of(l[0], h[0]);
    o = f64_of(l[1], h[1]);
}
__device__ __forceinline__ void row_pairs(float v, float &e, float &o)
{
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto l = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    e = __builtin_bit_cast(float, (unsigned)l[0]);
    o = __builtin_bit_cast(float, (unsigned)l[1]);
}
__device__ __forceinline__ double low_half(double x)
{
    const unsigned long long b = __builtin_bit_cast(unsigned long long, x);
    const auto l = __builtin_amdgcn_permlane32_swap((unsigned)b, (unsigned)b, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((unsigned)(b >> 32), (unsigned)(b >> 32), false, false);
    return f64_of(l[0], h[0]);
}
__device__ __forceinline__ float low_half(float x)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto l = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)l[0]);
}
template <int N>
__device__ __forceinline__ double lane_value(double x)
{
    const unsigned long long b = __builtin_bit_cast(unsigned long long, x);
    return f64_of((unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, N),
                  (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), N));
}
template <int N>
__device__ __forceinline__ float lane_value(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), N));
}

// y += ur(lane N) m + ui(lane N) q, lane N of this lane's row read by the
// multiply-adds themselves (DPP row_newbcast on the first source; the
// compiler does not fold a broadcast into a 64-bit multiply-add by itself).
// FIRST: ur and ui were just written by other VALU instructions, and a DPP
// read of a VGPR must come at least two cycles after its write.
template <int N, bool FIRST>
__device__ __forceinline__ void fmac_pair(double &y, double ur, double ui, double m, double q)
{
    if constexpr (FIRST)
        asm("s_nop 1\n\tv_fmac_f64_dpp %0, %1, %2 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f64_dpp %0, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
            : "+v"(y)
            : "v"(ur), "v"(m), "v"(ui), "v"(q), "n"(N));
    else
        asm("v_fmac_f64_dpp %0, %1, %2 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f64_dpp %0, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
            : "+v"(y)
            : "v"(ur), "v"(m), "v"(ui), "v"(q), "n"(N));
}
template <int N, bool FIRST>
__device__ __forceinline__ void fmac_pair(float &y, float ur, float ui, float m, float q)
{
    if constexpr (FIRST)
        asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %0, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
            : "+v"(y)
            : "v"(ur), "v"(m), "v"(ui), "v"(q), "n"(N));
    else
        asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %0, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
            : "+v"(y)
            : "v"(ur), "v"(m), "v"(ui), "v"(q), "n"(N));
}
// y[r] += L_re(r, J) m + L_im(r, J) q for r = N .. 15 (ur, ui: rows 0 and
// 1 of column J in every row)
template <typename R, int N, bool FIRST>
__device__ __forceinline__ void diag16c_update(R *y, R ur, R ui, R m, R q)
{
    if constexpr (N < LB16) {
        fmac_pair<N, FIRST>(y[N], ur, ui, m, q);
        diag16c_update<R, N + 1, false>(y, ur, ui, m, q);
    }
}

// Scale of pivot column J from its value d = Re A(J, J) (uniform), as
// diag16_pivot.
template <typename R, bool FACTOR, int J>
__device__ __forceinline__ void diag16c_pivot(R d, R &s, R &ljj, int &bad)
{
    if constexpr (FACTOR) {
        const bool ok = d > R(0);
        bad = (!ok && bad < 0) ? J : bad;
        d = ok ? d : R(1);
        s = rsqrt_refined(d, ljj);
    } else {
        ljj = d;
        s = R(1) / d;
    }
}

// Column J of the complex sweep (pivot scale s, ljj already known), then the
// columns after it.  y, c, g as in diag16c; sg = -1 in rows 1 and 2.  The
// column is scaled (rows 0 and 1 only when FACTOR: otherwise they hold the
// given L), L(r, J) = row 0's and row 1's y[J] in lane r is copied into
// every row, then y[r] -= P Re L(r, J) + Q Im L(r, J) for r > J, row J + 1
// first so that the next pivot's chain overlaps the other rows.
template <typename R, bool FACTOR, int J>
__device__ __forceinline__ void diag16c_step(R *y, int c, int g, R sg, R s, R ljj, int &bad)
{
    if constexpr (J < LB16) {
        if constexpr (FACTOR)
            y[J] = (g < 2 && c == J) ? (g == 0 ? ljj : R(0)) : y[J] * s;
        else
            y[J] = (g < 2) ? y[J] : y[J] * s;
        R e, od;
        row_pairs(y[J], e, od);
        R P = y[J], Q = sg * ((g & 1) ? e : od);  // Q: the partner plane's entry J
        if constexpr (!FACTOR) {
            P = (g < 2) ? R(0) : P;
            Q = (g < 2) ? R(0) : Q;
        }
        const R ur = low_half(e), ui = low_half(od);
        R s1 = R(0), l1 = R(0);
        if constexpr (J + 1 < LB16) {
            y[J + 1] = __builtin_fma(-Q, row_value<J + 1>(ui), __builtin_fma(-P, row_value<J + 1>(ur), y[J + 1]));
            diag16c_pivot<R, FACTOR, J + 1>(lane_value<J + 1>(y[J + 1]), s1, l1, bad);
        }
        if constexpr (J + 2 < LB16)
            diag16c_update<R, J + 2, true>(y, ur, ui, -P, -Q);
        diag16c_step<R, FACTOR, J + 1>(y, c, g, sg, s1, l1, bad);
    }
}

// Factor (FACTOR) and invert, or only invert, the complex 16 x 16 diagonal
// block at (o, o) of S0 + i S1 (S*[c][r] = element (r, c), lower triangle);
// L goes back to S's lower triangle (real diagonal), inv(L) to S's upper
// triangle and Xd (its diagonal).  One wave: lane 16 g + c keeps y[r] = Re
// A(c, r), Im A(c, r), Re inv(L)(r, c), Im inv(L)(r, c) for g = 0 .. 3.
template <typename R, bool FACTOR>
__device__ __forceinline__ void diag16c(R (*S0)[LDL], R (*S1)[LDL], R *Xd0, R *Xd1, int o, int lb, int gcol, int *info,
                                        int *failed)
{
    const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
    R(*const Sp)[LDL] = (g & 1) ? S1 : S0;
    R y[LB16];
#pragma unroll
    for (int r = 0; r < LB16; ++r) {  // row c of A, the upper part as conj(A(r, c)); e_c
        const R v = (r <= c) ? Sp[o + r][o + c] : Sp[o + c][o + r];
        y[r] = g == 0 ? v : g == 1 ? ((r <= c) ? v : -v) : (g == 2 && r == c) ? R(1) : R(0);
    }
    const R sg = (g == 1 || g == 2) ? R(-1) : R(1);
    int bad = -1;
    R s0, l0;
    diag16c_pivot<R, FACTOR, 0>(lane_value<0>(y[0]), s0, l0, bad);
    diag16c_step<R, FACTOR, 0>(y, c, g, sg, s0, l0, bad);
    if (FACTOR && bad >= 0 && lane == 0 && o + bad < lb) {
        if (info != nullptr)
            atomicCAS(info, 0, gcol + o + bad + 1);
        *failed = 1;
    }
    R *const Xp = (g & 1) ? Xd1 : Xd0;
#pragma unroll
    for (int r = 0; r < LB16; ++r) {
        if (g < 2 ? (FACTOR && r <= c) : r > c)  // row c of L; column c of inv(L) below its diagonal
            Sp[o + r][o + c] = y[r];
        if (g >= 2 && r == c)
            Xp[o + c] = y[r];
    }
}

// Element (row, col) of inv(L) kept by the complex leaf (strict lower part in
// the upper triangle of S, the diagonal in Xd, zero above the diagonal).
template <typename R>
__device__ __forceinline__ void leafc_xget(const R (*S)[LEAF][LDL], const R (*Xd)[LEAF], int row, int col, R &re, R &im)
{
    re = row > col ? S[0][row][col] : row == col ? Xd[0][row] : R(0);
    im = row > col ? S[1][row][col] : row == col ? Xd[1][row] : R(0);
}

// Factor (factor) and invert, or only invert, the complex 64 x 64 block held
// in the planes S[0] + i S[1] (S*[c][r] = element (r, c); lower triangle
// read, real diagonal; identity beyond lb): L goes to S's lower triangle,
// inv(L) below its diagonal to S's upper triangle (transposed) and its
// diagonal to Xd.  All 256 threads take part; the block is in S and *failed
// is 0 before the call (with a barrier after the stores), and the results are
// there after it.  A pivot that is not > 0 records info at column gcol + its
// index (columns < lb only) and sets *failed.
template <typename R>
__device__ __forceinline__ void leafc_lds(R (*S)[LEAF][LDL], R (*Xd)[LEAF], R (*Tm)[2][LB16][LB16 + 1], bool factor,
                                          int lb, int gcol, int *info, int *failed)
{
    typedef typename AccT<R>::type V4;
    constexpr int NB = LEAF / LB16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lk = lane >> 4;
    // operand fetchers: element (row, col) of L (lower triangle), of inv(L)
    // (zero above its diagonal) and of conj(inv(L))^T
    auto lget = [&](int row, int col, R &re, R &im) {
        re = S[0][col][row];
        im = S[1][col][row];
    };
    auto xget = [&](int row, int col, R &re, R &im) {
        re = row > col ? S[0][row][col] : row == col ? Xd[0][row] : R(0);
        im = row > col ? S[1][row][col] : row == col ? Xd[1][row] : R(0);
    };
    // store the 16 x 16 accumulator blocks (lane layout of mma16) as rows ro..,
    // columns co.. of L (lower part) or, below its diagonal, of inv(L), scaled by sg
    auto put = [&](bool inv, int ro, int co, const V4 &cr, const V4 &ci, R sg) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int rr = ro + li, cc = co + acc_row<R>(lk, qq);
            const int i0 = inv ? rr : cc, i1 = inv ? cc : rr;
            S[0][i0][i1] = sg * cr[qq];
            S[1][i0][i1] = sg * ci[qq];
        }
    };

    // T += sum_{k0 <= k < k1} L(i, k) X(k, b)
    auto tsum = [&](int i, int b, int k0, int k1, V4 &cr, V4 &ci) {
        for (int k = k0; k < k1; ++k)
            mma16c<R>([&](int rr, int kk, R &re, R &im) { lget(i * LB16 + rr, k * LB16 + kk, re, im); },
                      [&](int kk, int cc, R &re, R &im) { xget(k * LB16 + kk, b * LB16 + cc, re, im); }, cr, ci);
    };
    // T to this wave's scratch (Tm[.][c][r] = T(r, c)), and back
    auto stage = [&](const V4 &cr, const V4 &ci) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            Tm[wave][0][acc_row<R>(lk, qq)][li] = cr[qq];
            Tm[wave][1][acc_row<R>(lk, qq)][li] = ci[qq];
        }
    };
    auto unstage = [&](V4 &cr, V4 &ci) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            cr[qq] = Tm[wave][0][acc_row<R>(lk, qq)][li];
            ci[qq] = Tm[wave][1][acc_row<R>(lk, qq)][li];
        }
    };
    // X(i, b) = -inv(L(i, i)) T, T staged
    auto apply = [&](int i, int b) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS stores done before reading them back
        __builtin_amdgcn_wave_barrier();
        V4 c2r = {0, 0, 0, 0}, c2i = {0, 0, 0, 0};
        mma16c<R>([&](int rr, int kk, R &re, R &im) { xget(i * LB16 + rr, i * LB16 + kk, re, im); },
                  [&](int kk, int cc, R &re, R &im) {
                      re = Tm[wave][0][cc][kk];
                      im = Tm[wave][1][cc][kk];
                  },
                  c2r, c2i);
        put(true, i * LB16, b * LB16, c2r, c2i, R(-1));
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
    };
    static_assert(NB == 4, "the inverse schedule below is written for four sub-blocks");

    for (int b = 0; b < NB; ++b) {
        const int o = b * LB16;
        if (wave == 0) {
            if (factor)
                diag16c<R, true>(S[0], S[1], Xd[0], Xd[1], o, lb, gcol, info, failed);
            else
                diag16c<R, false>(S[0], S[1], Xd[0], Xd[1], o, lb, gcol, info, failed);
        } else if (b == 2 && wave == 1) {
            // beside the sweeps, the inverse blocks whose inputs are final
            // (partial sums of the last block row wait in the wave's scratch)
            V4 tr = {0, 0, 0, 0}, ti = {0, 0, 0, 0};
            tsum(1, 0, 0, 1, tr, ti);
            stage(tr, ti);
            apply(1, 0);
        } else if (b == 3 && wave == 1) {
            V4 tr = {0, 0, 0, 0}, ti = {0, 0, 0, 0};
            tsum(2, 1, 1, 2, tr, ti);
            stage(tr, ti);
            apply(2, 1);
            V4 ur = {0, 0, 0, 0}, ui = {0, 0, 0, 0};
            tsum(3, 1, 1, 3, ur, ui);
            stage(ur, ui);
        } else if (b == 3 && wave == 2) {
            V4 tr = {0, 0, 0, 0}, ti = {0, 0, 0, 0};
            tsum(2, 0, 0, 2, tr, ti);
            stage(tr, ti);
            apply(2, 0);
        } else if (b == 3 && wave == 3) {
            V4 tr = {0, 0, 0, 0}, ti = {0, 0, 0, 0};
            tsum(3, 0, 0, 2, tr, ti);
            stage(tr, ti);
        }
        __syncthreads();
        if (factor) {
            // L(i, b) = A(i, b) inv(L(b, b))^H, one block per wave
            // (each wave reads and then writes only its own block of column b)
            const int i = b + 1 + wave;
            if (i < NB) {
                V4 cr = {0, 0, 0, 0}, ci = {0, 0, 0, 0};
                mma16c<R>([&](int rr, int k, R &re, R &im) { lget(i * LB16 + rr, o + k, re, im); },
                          [&](int k, int cc, R &re, R &im) {
                              xget(o + cc, o + k, re, im);
                              im = -im;
                          },
                          cr, ci);
                put(false, i * LB16, o, cr, ci, R(1));
            }
            __syncthreads();
            // A(i, j) -= L(i, b) L(j, b)^H, b < j <= i
            for (int t = wave; t < (NB - 1 - b) * (NB - b) / 2; t += 4) {
                int ti, tj;
                tri_index(t, ti, tj);
                const int i2 = b + 1 + ti, j2 = b + 1 + tj;
                V4 dr = {0, 0, 0, 0}, di = {0, 0, 0, 0};
                mma16c<R>([&](int rr, int k, R &re, R &im) { lget(i2 * LB16 + rr, o + k, re, im); },
                          [&](int k, int cc, R &re, R &im) {
                              lget(j2 * LB16 + cc, o + k, re, im);
                              im = -im;
                          },
                          dr, di);
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int rr = li, cc = acc_row<R>(lk, qq);
                    if (i2 != j2 || rr >= cc) {
                        S[0][j2 * LB16 + cc][i2 * LB16 + rr] -= dr[qq];
                        S[1][j2 * LB16 + cc][i2 * LB16 + rr] -= di[qq];
                    }
                }
            }
            __syncthreads();
        }
    }

    // the last block row of the inverse: X(3, b) = -inv(L(3, 3)) sum_k L(3, k) X(k, b)
    // (rows 1 and 2 and the partial sums above were formed beside the sweeps,
    // each sum in the order of k)
    if (wave == 0) {
        V4 tr = {0, 0, 0, 0}, ti = {0, 0, 0, 0};
        tsum(3, 2, 2, 3, tr, ti);
        stage(tr, ti);
        apply(3, 2);
    } else if (wave == 1) {
        apply(3, 1);
    } else if (wave == 3) {
        V4 tr = {0, 0, 0, 0}, ti = {0, 0, 0, 0};
        unstage(tr, ti);
        tsum(3, 0, 2, 3, tr, ti);
        stage(tr, ti);
        apply(3, 0);
    }
    __syncthreads();
}

// PANEL: one launch factors a single leaf and solves the p.prows panel rows
// below it, L(i, leaf) = A(i, leaf) inv(L_leaf)^H, as leaf16_kernel's PANEL
// mode: every workgroup factors and inverts the leaf in its own LDS (the same
// bits), workgroup w >= 1 multiplies rows [64(w-1), 64w) of the panel in place,
// reading them straight into the matrix-core operand registers (no LDS), and
// the last workgroup to count itself out on p.ctr stores L and inv(L) and
// resets the counter.  Only workgroup 0 records info.
template <typename R, bool PANEL = false>
__global__ void __launch_bounds__(256) leaf16c_kernel(const LeafArgs p)
{
    typedef typename AccT<R>::type V4;
    typedef typename Elem<R, true>::type E;
    constexpr int NB = LEAF / LB16;
    __shared__ R S[2][LEAF][LDL];           // L below the diagonal, inv(L) above (see above)
    __shared__ R Xd[2][LEAF];               // diagonal of inv(L)
    __shared__ R Tm[4][2][LB16][LB16 + 1];  // per-wave 16 x 16 scratch
    __shared__ int failed;

    int64_t c0, ioff;
    int lb;
    const int w = PANEL ? (int)blockIdx.x : 0;  // panel block of this workgroup (0: none)
    if (!leaf_geom(p, PANEL ? 0 : (int)blockIdx.x, c0, lb, ioff))
        return;
    E *A = (E *)p.A + c0 + c0 * p.lda;
    E *Inv = (E *)p.Inv + ioff;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, lk = lane >> 4;
    const int r = tid & (LEAF - 1), g = tid / LEAF;
    int *const info = (w == 0) ? p.info : nullptr;

    // all loads in flight together, the status word alongside them; the
    // diagonal's imaginary part is taken as 0 and padding beyond lb is the
    // identity
    R vr[LEAF / 4], vi[LEAF / 4];
#pragma unroll
    for (int k = 0; k < LEAF / 4; ++k) {
        const int c = g + 4 * k;
        vr[k] = (r == c) ? R(1) : R(0);
        vi[k] = R(0);
        if (r < lb && c < lb && r >= c)
            Elem<R, true>::load(A + r + (int64_t)c * p.lda, vr[k], vi[k]);
        if (r == c)
            vi[k] = R(0);
    }
    if (p.info != nullptr && *p.info != 0)
        return;
#pragma unroll
    for (int k = 0; k < LEAF / 4; ++k) {
        S[0][g + 4 * k][r] = vr[k];
        S[1][g + 4 * k][r] = vi[k];
    }
    if (tid == 0)
        failed = 0;
    __syncthreads();

    leafc_lds<R>(S, Xd, Tm, p.factor != 0, lb, p.col0 + (int)c0, info, &failed);
    auto xget = [&](int row, int col, R &re, R &im) { leafc_xget<R>(S, Xd, row, col, re, im); };

    if (failed)
        return;
    if constexpr (PANEL) {
        if (w > 0) {
            // wave v owns panel rows 16v .. 16v + 15 of this block:
            // P(v, j) = sum_{k <= j} B(v, k) conj(inv(L)(j, k)) over 16 x 16 blocks,
            // B read from global in the operand layout of mma16c (lane (li, lk)
            // holds B(16v + li, 16 bk + 4 s + lk) in br[bk][s] + i bi[bk][s])
            E *const Pb = A + lb + (int64_t)(w - 1) * LEAF;  // rows lb + 64(w-1) .. of the leaf's columns
            const int prow = p.prows - (w - 1) * LEAF;       // its rows that exist
            const int row = wave * LB16 + li;
            R br[NB][4], bi[NB][4];
#pragma unroll
            for (int bk = 0; bk < NB; ++bk)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k = bk * LB16 + 4 * q + lk;
                    br[bk][q] = R(0);
                    bi[bk][q] = R(0);
                    if (row < prow && k < lb)
                        Elem<R, true>::load(Pb + row + (int64_t)k * p.lda, br[bk][q], bi[bk][q]);
                }
            // every block of the row is read before any is overwritten (the
            // rows belong to this wave alone)
#pragma unroll
            for (int bj = 0; bj < NB; ++bj) {
                V4 cr = {0, 0, 0, 0}, ci = {0, 0, 0, 0};
#pragma unroll
                for (int bk = 0; bk <= bj; ++bk)
                    mma16c_ra<R>(br[bk], bi[bk],
                                 [&](int kk, int cc, R &re, R &im) {
                                     xget(bj * LB16 + cc, bk * LB16 + kk, re, im);
                                     im = -im;
                                 },
                                 cr, ci);
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int cc = bj * LB16 + acc_row<R>(lk, qq);
                    if (row < prow && cc < lb)
                        Elem<R, true>::store(Pb + row + (int64_t)cc * p.lda, cr[qq], ci[qq]);
                }
            }
        }
        // count out; the last workgroup stores the leaf
        __shared__ int last;
        __syncthreads();
        if (tid == 0) {
            last = atomicAdd(p.ctr, 1) == (int)gridDim.x - 1;
            if (last)
                atomicExch(p.ctr, 0);
        }
        __syncthreads();
        if (!last)
            return;
    }
#pragma unroll
    for (int k = 0; k < LEAF / 4; ++k) {
        const int c = g + 4 * k;
        if (r < lb && c < lb) {
            if (p.factor && r >= c)
                Elem<R, true>::store(A + r + (int64_t)c * p.lda, S[0][c][r], r == c ? R(0) : S[1][c][r]);
            R xr = R(0), xi = R(0);
            xget(r, c, xr, xi);
            Elem<R, true>::store(Inv + r + (int64_t)c * p.ldi, xr, xi);
        }
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

// Gaussian-process marginal log-likelihood per right-hand-side column (JAXMg
// paper, "Research Impact Statement", "Cholesky solve (potrs)"): with Y = L^-1 R
// already in place of R,
//     out[j] = -1/2 |Y(:, j)|^2 - sum_i log L_ii - (n/2) log(2 pi)
// (the middle term is 1/2 log det A).  One workgroup per column; both sums are
// accumulated in double by a fixed reduction tree, so the result is the same
// bits on every run.  NaN if the factorization reported a failure.
template <typename R>
__global__ void __launch_bounds__(256) gp_loglik_kernel(const R *Y, int64_t ldy, const R *L, int64_t lda, int64_t n,
                                                        const int *info, double *out)
{
    __shared__ double red[2][256];
    const int tid = threadIdx.x, j = blockIdx.x;
    double ss = 0.0, ld = 0.0;
    for (int64_t i = tid; i < n; i += 256) {
        const double y = (double)Y[i + (int64_t)j * ldy];
        ss += y * y;
        ld += log((double)L[i * (1 + lda)]);
    }
    red[0][tid] = ss;
    red[1][tid] = ld;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) {
            red[0][tid] += red[0][tid + w];
            red[1][tid] += red[1][tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        const double two_pi = 6.283185307179586476925286766559;
        out[j] = (info != nullptr && *info != 0) ? __longlong_as_double(0x7ff8000000000000LL)
                                                 : -0.5 * red[0][0] - red[1][0] - 0.5 * (double)n * log(two_pi);
    }
}

// Reduction of the generalized eigenproblem (helpers).  M (n x n, ldm) gets
// the full Hermitian matrix whose lower triangle is stored in A: M(i, j) =
// A(i, j) for i >= j and conj(A(j, i)) above; only A's lower triangle is
// read, and the imaginary part of the diagonal is taken as zero.  One
// workgroup (32 x 8 threads) per pair of 32 x 32 tiles (I, J), I >= J: tile
// (I, J) of A is staged in LDS, written to M(I, J) and, conjugate-transposed,
// to M(J, I), both down columns.
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) herm_full_kernel(const void *Av, int64_t lda, void *Mv, int64_t ldm, int64_t n)
{
    typedef typename Elem<R, CPLX>::type E;
    constexpr int TB = 32;
    __shared__ R t[2][TB][TB + 1];  // t[.][c][r] = A(i0 + r, j0 + c)
    const E *A = (const E *)Av;
    E *M = (E *)Mv;
    int I, J;
    tri_index((int)blockIdx.x, I, J);
    const int64_t i0 = (int64_t)I * TB, j0 = (int64_t)J * TB;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int c = ty; c < TB; c += 8) {
        R re = 0, im = 0;
        if (i0 + tx < n && j0 + c < n && (I != J || tx >= c))
            Elem<R, CPLX>::load(A + (i0 + tx) + (j0 + c) * lda, re, im);
        t[0][c][tx] = re;
        t[1][c][tx] = (I == J && tx == c) ? R(0) : im;
    }
    __syncthreads();
    for (int c = ty; c < TB; c += 8) {
        if (i0 + tx < n && j0 + c < n) {  // M(I, J)
            const bool low = I != J || tx >= c;
            Elem<R, CPLX>::store(M + (i0 + tx) + (j0 + c) * ldm, low ? t[0][c][tx] : t[0][tx][c],
                                 low ? t[1][c][tx] : -t[1][tx][c]);
        }
        if (I != J && j0 + tx < n && i0 + c < n)  // M(J, I)(r, c) = conj(A(I, J)(c, r))
            Elem<R, CPLX>::store(M + (j0 + tx) + (i0 + c) * ldm, t[0][tx][c], -t[1][tx][c]);
    }
}

// M <- M^H in place for square n x n M: one workgroup per pair of 32 x 32
// tiles (I, J), I >= J, staged through LDS so that reads and writes run down
// columns.
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) conj_transpose_kernel(void *Mv, int64_t ldm, int64_t n, const int *info)
{
    typedef typename Elem<R, CPLX>::type E;
    constexpr int TB = 32;
    __shared__ R a[2][TB][TB + 1], b[2][TB][TB + 1];  // [part][col][row]
    if (info != nullptr && *info != 0)
        return;
    E *M = (E *)Mv;
    int I, J;
    tri_index((int)blockIdx.x, I, J);
    const int64_t i0 = (int64_t)I * TB, j0 = (int64_t)J * TB;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    for (int c = ty; c < TB; c += 8) {
        R re = 0, im = 0;
        if (i0 + tx < n && j0 + c < n)
            Elem<R, CPLX>::load(M + (i0 + tx) + (j0 + c) * ldm, re, im);  // tile (I, J)
        a[0][c][tx] = re;
        a[1][c][tx] = im;
        re = 0;
        im = 0;
        if (j0 + tx < n && i0 + c < n)
            Elem<R, CPLX>::load(M + (j0 + tx) + (i0 + c) * ldm, re, im);  // tile (J, I)
        b[0][c][tx] = re;
        b[1][c][tx] = im;
    }
    __syncthreads();
    for (int c = ty; c < TB; c += 8) {
        // new (I, J)(r, c) = conj(old (J, I)(c, r)); new (J, I)(r, c) = conj(old (I, J)(c, r))
        if (i0 + tx < n && j0 + c < n)
            Elem<R, CPLX>::store(M + (i0 + tx) + (j0 + c) * ldm, b[0][tx][c], -b[1][tx][c]);
        if (I != J && j0 + tx < n && i0 + c < n)
            Elem<R, CPLX>::store(M + (j0 + tx) + (i0 + c) * ldm, a[0][tx][c], -a[1][tx][c]);
    }
}

// A(i, j) = M(i, j) for i >= j (the lower triangle only), the diagonal's
// imaginary part set to zero (the result is Hermitian); NaN there instead when
// info reports a failure.
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) copy_lower_kernel(void *Av, int64_t lda, const void *Mv, int64_t ldm,
                                                         int64_t n, const int *info)
{
    typedef typename Elem<R, CPLX>::type E;
    const bool bad = info != nullptr && *info != 0;
    const R qnan = (R)__longlong_as_double(0x7ff8000000000000LL);
    E *A = (E *)Av;
    const E *M = (const E *)Mv;
    const int64_t total = n * n;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e % n, j = e / n;
        if (i < j)
            continue;
        R re = qnan, im = qnan;
        if (!bad) {
            Elem<R, CPLX>::load(M + i + j * ldm, re, im);
            if (i == j)
                im = 0;
        }
        Elem<R, CPLX>::store(A + i + j * lda, re, im);
    }
}

// X (n x n, ldx) = the lower triangle of L with zeros above it (the diagonal's
// imaginary part taken as zero); only L's lower triangle is read.
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) tril_kernel(const void *Lv, int64_t ldl, void *Xv, int64_t ldx, int64_t n)
{
    typedef typename Elem<R, CPLX>::type E;
    const E *L = (const E *)Lv;
    E *X = (E *)Xv;
    const int64_t total = n * n;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e % n, j = e / n;
        R re = 0, im = 0;
        if (i >= j) {
            Elem<R, CPLX>::load(L + i + j * ldl, re, im);
            if (i == j)
                im = 0;
        }
        Elem<R, CPLX>::store(X + i + j * ldx, re, im);
    }
}

// ---- blocked reduction of the generalized eigenproblem (helpers) ----

// One step of the type-1 reduction, after Y = A21 inv(L11)^H and V = L21 C11
// (m x tk each): Z = Y - V/2 goes into P[:, 0:tk) and Q[:, kh:kh+tk), L21 into
// P[:, kh:kh+tk) and Q[:, 0:tk), and X = Y - V back into the matrix (the block
// column under the diagonal block).  P and Q (ldw x 2 kh) are written whole,
// zero outside those columns and below row m, so that the rank-2k update
// C -= P Q^H = Z L21^H + L21 Z^H reads them without bounds.
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) gst_pack_kernel(const void *Yv, int64_t ldy, const void *Vv, int64_t ldv,
                                                       const void *Lv, int64_t ldl, void *Pv, void *Qv, int64_t ldw,
                                                       void *Xv, int64_t ldx, int64_t m, int64_t tk, int64_t kh)
{
    typedef typename Elem<R, CPLX>::type E;
    const E *Y = (const E *)Yv, *V = (const E *)Vv, *L = (const E *)Lv;
    E *P = (E *)Pv, *Q = (E *)Qv, *X = (E *)Xv;
    const int64_t total = ldw * kh;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e % ldw, k = e / ldw;
        R zr = 0, zi = 0, lr = 0, li = 0;
        if (i < m && k < tk) {
            R yr, yi = 0, vr, vi = 0;
            Elem<R, CPLX>::load(Y + i + k * ldy, yr, yi);
            Elem<R, CPLX>::load(V + i + k * ldv, vr, vi);
            Elem<R, CPLX>::load(L + i + k * ldl, lr, li);
            zr = yr - R(0.5) * vr;
            zi = yi - R(0.5) * vi;
            Elem<R, CPLX>::store(X + i + k * ldx, yr - vr, yi - vi);
        }
        Elem<R, CPLX>::store(P + i + k * ldw, zr, zi);
        Elem<R, CPLX>::store(P + i + (kh + k) * ldw, lr, li);
        Elem<R, CPLX>::store(Q + i + k * ldw, lr, li);
        Elem<R, CPLX>::store(Q + i + (kh + k) * ldw, zr, zi);
    }
}

// D (ldw x halves*kh) = [S0 | S1] as zero-padded column panels: columns
// [0, tk) of half h hold rows [0, m) of S_h (ld ld_h), everything else is 0.
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) panel_pack_kernel(const void *S0v, int64_t ld0, const void *S1v, int64_t ld1,
                                                         void *Dv, int64_t ldw, int64_t m, int64_t tk, int64_t kh,
                                                         int halves)
{
    typedef typename Elem<R, CPLX>::type E;
    const E *S0 = (const E *)S0v, *S1 = (const E *)S1v;
    E *D = (E *)Dv;
    const int64_t total = ldw * kh * halves;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e % ldw, c = e / ldw, h = c / kh, k = c % kh;
        R re = 0, im = 0;
        if (i < m && k < tk)
            Elem<R, CPLX>::load((h == 0 ? S0 + i + k * ld0 : S1 + i + k * ld1), re, im);
        Elem<R, CPLX>::store(D + e, re, im);
    }
}

// X (ldx x ldx, zero padded) = L^H restricted to the entries (i, j) with
// j >= i (strict = 0: the whole upper triangle of L^H) or with column j in a
// later T-block than row i (strict = 1); L's lower triangle is read, the
// diagonal's imaginary part taken as zero.  One workgroup per pair of 32 x 32
// tiles (I, J), I >= J, of the ldx x ldx square: tile (I, J) of L is staged in
// LDS and written conjugate-transposed to X(J, I); X(I, J) below the diagonal
// gets zeros.
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) gst_lh_kernel(const void *Lv, int64_t ldl, void *Xv, int64_t ldx, int64_t n,
                                                     int64_t T, int strict)
{
    typedef typename Elem<R, CPLX>::type E;
    constexpr int TB = 32;
    __shared__ R t[2][TB][TB + 1];  // t[.][c][r] = L(i0 + r, j0 + c)
    const E *L = (const E *)Lv;
    E *X = (E *)Xv;
    int I, J;
    tri_index((int)blockIdx.x, I, J);
    const int64_t i0 = (int64_t)I * TB, j0 = (int64_t)J * TB;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int c = ty; c < TB; c += 8) {
        R re = 0, im = 0;
        if (i0 + tx < n && j0 + c < n && (I != J || tx >= c))
            Elem<R, CPLX>::load(L + (i0 + tx) + (j0 + c) * ldl, re, im);
        t[0][c][tx] = re;
        t[1][c][tx] = (I == J && tx == c) ? R(0) : im;
    }
    __syncthreads();
    for (int c = ty; c < TB; c += 8) {
        // X(J, I)(r, c): i = j0 + r, j = i0 + c, value conj(L(j, i)) = conj(t[r][c])
        const int64_t i = j0 + tx, j = i0 + c;
        R re = 0, im = 0;
        if (i < n && j < n && (strict ? j / T > i / T : j >= i)) {
            re = t[0][tx][c];
            im = -t[1][tx][c];
        }
        Elem<R, CPLX>::store(X + i + j * ldx, re, im);
        if (I != J)  // strictly below the diagonal of X
            Elem<R, CPLX>::store(X + (i0 + tx) + (j0 + c) * ldx, R(0), R(0));
    }
}

// Ld: the lower triangles of L's T x T diagonal blocks, zeros above (tile t
// at t*T*T, ld T; the ragged last block zero padded), the diagonal's
// imaginary part zero.
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) gst_diag_tril_kernel(const void *Lv, int64_t ldl, void *Dv, int64_t n,
                                                            int64_t T, int64_t nt)
{
    typedef typename Elem<R, CPLX>::type E;
    const E *L = (const E *)Lv;
    E *D = (E *)Dv;
    const int64_t total = nt * T * T;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t t = e / (T * T), r = e % (T * T), i = r % T, j = r / T, c0 = t * T;
        R re = 0, im = 0;
        if (i >= j && c0 + i < n) {
            Elem<R, CPLX>::load(L + (c0 + i) + (c0 + j) * ldl, re, im);
            if (i == j)
                im = 0;
        }
        Elem<R, CPLX>::store(D + e, re, im);
    }
}

// For a rows x p block: W += V/2, then X = W + V/2 (V and X with ld ldv).
template <typename R, bool CPLX>
__global__ void __launch_bounds__(256) gst_half_kernel(void *Wv, int64_t ldw, const void *Vv, void *Xv, int64_t ldv,
                                                       int64_t rows, int64_t p)
{
    typedef typename Elem<R, CPLX>::type E;
    E *W = (E *)Wv, *X = (E *)Xv;
    const E *V = (const E *)Vv;
    const int64_t total = rows * p;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e % rows, j = e / rows;
        R wr, wi = 0, vr, vi = 0;
        Elem<R, CPLX>::load(W + i + j * ldw, wr, wi);
        Elem<R, CPLX>::load(V + i + j * ldv, vr, vi);
        wr += R(0.5) * vr;
        wi += R(0.5) * vi;
        Elem<R, CPLX>::store(W + i + j * ldw, wr, wi);
        Elem<R, CPLX>::store(X + i + j * ldv, wr + R(0.5) * vr, wi + R(0.5) * vi);
    }
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
