// MFMA tile kernel for the dense SPD/HPD solve on gfx950 (CDNA4).
//
// One kernel template covers every dense contraction of the blocked Cholesky
// solve (JAXMg paper, "Software design": potrs = potrf then potrs):
//   - the trailing update  A22 -= L21 L21^H  (lower tiles only),
//   - the panel solve      L21 = A21 L11^-H  as a product with inv(L11),
//   - the doubling steps that build inv(L11) from inverted leaf blocks,
//   - the blocked forward / back substitution updates of the right-hand side.
//
//   C = beta * C + s * opA * opB,     s = -1 if neg else +1,  beta in {0, 1}
//
// opA is m x k and opB is k x n.  Operand storage (column-major, leading
// dimension ld):
//   AT = false : opA(i, k) = A[i + k*lda]
//   AT = true  : opA(i, k) = conj(A[k + i*lda])
//   BT = false : opB(k, j) = B[k + j*ldb]
//   BT = true  : opB(k, j) = conj(B[j + k*ldb])
// (conj only matters for complex types.)
//
// Tiling: a workgroup owns a BM x BN tile of C, split over WM x WN wave64s.
// Each wave owns (BM/WM) x (BN/WN) as 16x16 MFMA blocks (v_mfma_*_16x16x4).
// k is consumed in KB-deep slices staged through double-buffered LDS; global
// loads for slice s+1 are in flight while slice s feeds the matrix cores.
// The MFMA's A-source is fed from opB and its B-source from opA, so that a
// lane's four accumulator registers hold four C columns of one row and each
// 16-lane group reads/writes one contiguous 16-element column segment of C
// (which four columns depends on the instruction, see acc_row).
//
// Complex types keep real and imaginary parts in separate LDS planes and use
// four real MFMAs per complex multiply-add.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spd {

typedef double dx4 __attribute__((ext_vector_type(4)));
typedef float fx4 __attribute__((ext_vector_type(4)));

template <typename R> struct AccT;
template <> struct AccT<double> { typedef dx4 type; };
template <> struct AccT<float> { typedef fx4 type; };

__device__ __forceinline__ dx4 mfma16(double a, double b, dx4 c)
{
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ fx4 mfma16(float a, float b, fx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Row of the 16x16 MFMA result held by accumulator register q of a lane in
// lane group g = lane / 16 (the column is lane % 16).  The fp32 instruction
// gives each lane group four consecutive rows; the fp64 one interleaves the
// groups (measured on gfx950 with a known-input probe).
template <typename R> __host__ __device__ inline int acc_row(int g, int q);
template <> __host__ __device__ inline int acc_row<float>(int g, int q) { return 4 * g + q; }
template <> __host__ __device__ inline int acc_row<double>(int g, int q) { return 4 * q + g; }

// k-range restriction for triangular operands whose zero triangle is stored
// explicitly (the inverted diagonal blocks): skip slices that are all zero.
enum KMode : int {
    KM_NONE = 0,
    KM_END_BY_J = 1,  // opB(k, j) = 0 for k > j   (k < (J+1)*BN)
    KM_BEG_BY_J = 2,  // opB(k, j) = 0 for k < j   (k >= J*BN)
    KM_END_BY_I = 3,  // opA(i, k) = 0 for k > i   (k < (I+1)*BM)
    KM_BEG_BY_I = 4,  // opA(i, k) = 0 for k < i   (k >= I*BM)
};

struct GemmArgs {
    const void *A;
    const void *B;
    void *C;
    int64_t lda, ldb, ldc;
    // batch z -> (z / nb_inner, z % nb_inner); offsets in elements
    int64_t sA_out, sA_in, sB_out, sB_in, sC_out, sC_in;
    int nb_inner;
    int m, n, k;
    int tiles_m, tiles_n, ntiles;
    int tri;    // lower-triangular output: tiles I >= J, and i >= j inside
    int kmode;  // KMode
    int neg;    // 1: subtract the product
    int beta;   // 0: C is not read; 1: accumulate into C
    const int *info;  // if non-null and *info != 0 the kernel does nothing
};

template <typename R, bool CPLX> struct Elem;
template <typename R> struct Elem<R, false> {
    typedef R type;
    static __device__ __forceinline__ void load(const R *p, R &re, R & /*im*/) { re = *p; }
    static __device__ __forceinline__ void store(R *p, R re, R /*im*/) { *p = re; }
};
template <typename R> struct Elem<R, true> {
    struct alignas(2 * sizeof(R)) C2 { R re, im; };
    typedef C2 type;
    static __device__ __forceinline__ void load(const C2 *p, R &re, R &im)
    {
        C2 v = *p;
        re = v.re;
        im = v.im;
    }
    static __device__ __forceinline__ void store(C2 *p, R re, R im)
    {
        C2 v;
        v.re = re;
        v.im = im;
        *p = v;
    }
};

// blockIdx.x -> logical tile id so that consecutive logical tiles run on the
// same XCD (workgroups are dealt round-robin over the 8 XCDs).  Bijective for
// any tile count.
__host__ __device__ inline int xcd_remap(int b, int nt)
{
    if (nt < 16)
        return b;
    const int q = nt >> 3, r = nt & 7;
    const int x = b & 7, idx = b >> 3;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + idx;
}

__host__ __device__ inline void tri_index(int t, int &I, int &J)
{
    int i = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while ((int64_t)(i + 1) * (i + 2) / 2 <= t)
        ++i;
    while ((int64_t)i * (i + 1) / 2 > t)
        --i;
    I = i;
    J = t - (int)((int64_t)i * (i + 1) / 2);
}

template <typename R, bool CPLX, int BM, int BN, int KB, int WM, int WN, bool AT, bool BT>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(const GemmArgs p)
{
    typedef typename Elem<R, CPLX>::type E;
    typedef typename AccT<R>::type V4;
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int NP = CPLX ? 2 : 1;
    constexpr int PA = BM + 1, PB = BN + 1;  // odd row length: transposed LDS stores spread over banks
    constexpr int LA = BM * KB / NT, LB = BN * KB / NT;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(KB % 4 == 0, "KB must be a multiple of 4");
    static_assert((BM * KB) % NT == 0 && (BN * KB) % NT == 0, "tile loads must divide evenly");

    __shared__ R As[2][NP][KB][PA];
    __shared__ R Bs[2][NP][KB][PB];

    // ---- tile coordinates
    int I, J;
    const int t = xcd_remap((int)blockIdx.x, p.ntiles);
    if (p.tri) {
        tri_index(t, I, J);
    } else {
        I = t % p.tiles_m;
        J = t / p.tiles_m;
    }
    const int z = blockIdx.z;
    const int zo = z / p.nb_inner, zi = z - zo * p.nb_inner;
    const E *__restrict__ A = (const E *)p.A + zo * p.sA_out + zi * p.sA_in;
    const E *__restrict__ B = (const E *)p.B + zo * p.sB_out + zi * p.sB_in;
    E *__restrict__ C = (E *)p.C + zo * p.sC_out + zi * p.sC_in;

    const int i0 = I * BM, j0 = J * BN;
    const int m = p.m, n = p.n;
    int kbeg = 0, kend = p.k;
    switch (p.kmode) {
    case KM_END_BY_J: kend = min(kend, j0 + BN); break;
    case KM_BEG_BY_J: kbeg = j0; break;
    case KM_END_BY_I: kend = min(kend, i0 + BM); break;
    case KM_BEG_BY_I: kbeg = i0; break;
    default: break;
    }
    kbeg = (kbeg / KB) * KB;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int li = lane & 15, lk = lane >> 4;
    const int ib = wm * TM, jb = wn * TN;  // wave tile origin inside the workgroup tile

    // ---- accumulators: start from C (beta = 1) or zero
    V4 acc[NP][FM][FN];
#pragma unroll
    for (int c = 0; c < NP; ++c)
#pragma unroll
        for (int fi = 0; fi < FM; ++fi)
#pragma unroll
            for (int fj = 0; fj < FN; ++fj)
                acc[c][fi][fj] = V4{0, 0, 0, 0};
    // The product is always accumulated with a plus sign; C - AB is formed as
    // -((-C) + AB), which rounds exactly like C + (-A)B (negation commutes with
    // rounding), so the operands reach the matrix cores as loaded.
    const R sg = p.neg ? R(-1) : R(1);
    if (p.beta) {
#pragma unroll
        for (int fi = 0; fi < FM; ++fi) {
            const int i = i0 + ib + fi * 16 + li;
#pragma unroll
            for (int fj = 0; fj < FN; ++fj) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = j0 + jb + fj * 16 + acc_row<R>(lk, q);
                    if (i < m && j < n) {
                        R re, im = 0;
                        Elem<R, CPLX>::load(C + i + (int64_t)j * p.ldc, re, im);
                        acc[0][fi][fj][q] = sg * re;
                        if constexpr (CPLX)
                            acc[NP - 1][fi][fj][q] = sg * im;
                    }
                }
            }
        }
    }

    // ---- global -> register staging
    R ra[NP][LA], rb[NP][LB];
    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int q = 0; q < LA; ++q) {
            const int e = tid + NT * q;
            int i, kk;
            if constexpr (!AT) { i = e % BM; kk = e / BM; }
            else               { kk = e % KB; i = e / KB; }
            const int gi = i0 + i, gk = k0 + kk;
            R re = 0, im = 0;
            if (gi < m && gk < kend) {
                const E *src = AT ? (A + gk + (int64_t)gi * p.lda) : (A + gi + (int64_t)gk * p.lda);
                Elem<R, CPLX>::load(src, re, im);
                if (AT) im = -im;
            }
            ra[0][q] = re;
            if constexpr (CPLX) ra[NP - 1][q] = im;
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            const int e = tid + NT * q;
            int j, kk;
            if constexpr (BT) { j = e % BN; kk = e / BN; }
            else              { kk = e % KB; j = e / KB; }
            const int gj = j0 + j, gk = k0 + kk;
            R re = 0, im = 0;
            if (gj < n && gk < kend) {
                const E *src = BT ? (B + gj + (int64_t)gk * p.ldb) : (B + gk + (int64_t)gj * p.ldb);
                Elem<R, CPLX>::load(src, re, im);
                if (BT) im = -im;
            }
            rb[0][q] = re;
            if constexpr (CPLX) rb[NP - 1][q] = im;
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int q = 0; q < LA; ++q) {
            const int e = tid + NT * q;
            int i, kk;
            if constexpr (!AT) { i = e % BM; kk = e / BM; }
            else               { kk = e % KB; i = e / KB; }
#pragma unroll
            for (int c = 0; c < NP; ++c)
                As[buf][c][kk][i] = ra[c][q];
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            const int e = tid + NT * q;
            int j, kk;
            if constexpr (BT) { j = e % BN; kk = e / BN; }
            else              { kk = e % KB; j = e / KB; }
#pragma unroll
            for (int c = 0; c < NP; ++c)
                Bs[buf][c][kk][j] = rb[c][q];
        }
    };

    // the status word is read once the first loads are in flight; the operand
    // buffers are valid whatever it holds, and nothing is written before it
    if (kbeg < kend)
        load_tiles(kbeg);
    if (p.info != nullptr && *p.info != 0)
        return;
    if (kbeg < kend) {
        store_tiles(0);
        __syncthreads();
        int cur = 0;
        for (int k0 = kbeg; k0 < kend; k0 += KB) {
            const bool more = (k0 + KB) < kend;
            if (more)
                load_tiles(k0 + KB);
#pragma unroll
            for (int s = 0; s < KB / 4; ++s) {
                const int kr = s * 4 + lk;
                R a[NP][FM], b[NP][FN];
#pragma unroll
                for (int c = 0; c < NP; ++c) {
#pragma unroll
                    for (int fi = 0; fi < FM; ++fi)
                        a[c][fi] = As[cur][c][kr][ib + fi * 16 + li];
#pragma unroll
                    for (int fj = 0; fj < FN; ++fj)
                        b[c][fj] = Bs[cur][c][kr][jb + fj * 16 + li];
                }
#pragma unroll
                for (int fi = 0; fi < FM; ++fi) {
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
            }
            if (more)
                store_tiles(cur ^ 1);
            __syncthreads();
            cur ^= 1;
        }
    }

    // ---- epilogue
#pragma unroll
    for (int fi = 0; fi < FM; ++fi) {
        const int i = i0 + ib + fi * 16 + li;
#pragma unroll
        for (int fj = 0; fj < FN; ++fj) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = j0 + jb + fj * 16 + acc_row<R>(lk, q);
                if (i < m && j < n && (!p.tri || i >= j))
                    Elem<R, CPLX>::store(C + i + (int64_t)j * p.ldc, sg * acc[0][fi][fj][q],
                                         CPLX ? sg * acc[NP - 1][fi][fj][q] : R(0));
            }
        }
    }
}

}  // namespace spd
