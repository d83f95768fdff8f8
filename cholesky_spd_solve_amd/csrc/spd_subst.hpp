// The back substitution L^H X = Y of the solve in one launch (JAXMg paper,
// "Software design": the triangular solves of potrs after the factorization;
// here by tile rows of T_A from the last one up):
//
//   X_i = inv(L_ii)^H (Y_i - sum_{j > i} L_ji^H X_j)
//       = inv(L_ii)^H Z_i + G_i^H X_{i+1},
//   Z_i = Y_i - sum_{j > i+1} L_ji^H X_j,   G_i = -L_{i+1,i} inv(L_ii),
//
// with the inverse of every diagonal tile already built (the factorization
// keeps them) and G_i formed before the launch.  Split this way, the step
// from X_{i+1} to X_i is one product: Z_i and inv(L_ii)^H Z_i only need
// X_{i+2} and are formed while X_{i+1} is still being solved.  Tile row i is
// cut into row pieces of SUB_TR rows and column pieces of TC right-hand
// sides; the workgroup of piece (i, rt, ct) takes two parts in turn:
//
//   R: Z_i(rt, ct) = Y_i(rt, ct) - sum_{j > i+1} L_ji(:, rt)^H X_j(:, ct),
//      a term as soon as X_j(:, ct) is complete, in decreasing j, into a
//      workspace buffer (T rows; tile rows of even and odd index take one
//      buffer each);
//   C: X_i(rt, ct) = sum_{r >= rt} inv(L_ii)^H(rt, r) Z_i(r, ct) once
//      Z_i(:, ct) is complete, then + G_i(:, rt)^H X_{i+1}(:, ct) once that
//      is complete; X goes into B.
//
// Two counters per (i, ct) count the R parts and the C parts done: Z_i(:, ct)
// and X_i(:, ct) are complete when they reach the tile row's number of row
// pieces (one wait each, however many pieces).  Workgroup ids run over the
// tile rows from the last.  A workgroup waits only for workgroups of its own
// tile row (their R parts, which wait for nothing of that row) and of later
// ones; workgroups are dispatched in id order, so by the time one of tile
// row i waits, every workgroup of the later rows and of row i has been
// dispatched or will be as the later rows finish, and no wait can hold back
// the one it waits for.  Every wait is bounded in time as in the
// one-launch diagonal tile (a wait that runs out raises an abort word that
// ends the others and sets info to -1), and the last workgroup to finish
// clears the flags, which are zero between launches (and, if a wait ran out,
// fills X with NaN).
//
// Two Z buffers suffice: the R part of piece (i, rt, ct) writes its piece of
// buffer i % 2 only after X_{i+2}(:, ct) is complete, that is after every C
// part of tile row i + 2 (the previous user of that buffer) has read column
// piece ct of it; the R parts of the last two tile rows have no terms and
// are the first users of their buffers.
#pragma once

#include "spd_kernels.hpp"

namespace spd {

constexpr int SUB_TR = 32;        // rows of a piece
constexpr int SUB_THREADS = 512;  // threads of a workgroup: two halves of 256
// Each counter and word has a 128-byte line of its own: the waiting
// workgroups poll them at agent scope, and polls and updates of different
// counters then go to different lines.
constexpr int SUB_FLAG_STRIDE = 32;
// A waiting workgroup sleeps about 64 SUB_POLL_SLEEP clocks between polls
// and looks at the abort word every fourth poll.
constexpr int SUB_POLL_SLEEP = 4;

struct SubstArgs {
    const void *A;    // L: first element, column-major, lda; lower triangle read
    int64_t lda;
    const void *Inv;  // inv(L_kk) at Inv + k T T, leading dimension T; its 64 x 64
                      // blocks on and below the diagonal are read (those on the
                      // diagonal as whole squares, zero above the diagonal)
    void *B;          // Y on entry, X on exit; ldb
    int64_t ldb;
    const void *G;    // G_i = -L_{i+1,i} inv(L_ii) at G + (i + 1) T T, leading
                      // dimension T, the rows of tile i + 1 (i < nt - 1)
    void *Z;          // two T x nrhs buffers, leading dimension ldz >= T, the
    int64_t ldz;      // second ldz * nrhs elements after the first
    int n, nrhs, T, nt;
    int nr;           // row pieces of a whole tile row: ceil(T / SUB_TR)
    int nc;           // column pieces: ceil(nrhs / TC)
    int *flags;       // subst_flag_ints(nt, nc) ints, zero between launches
    const int *info;  // nothing is done when non-zero on entry (may be null)
    int *status;      // set to -1 if a wait ran out (may be null); X is then NaN
    int64_t limit;    // longest wait, in wall-clock ticks (100 MHz)
};

// counters of Z(:, ct) and of X_i(:, ct) per (i, ct), the abort word and the
// count of workgroups done
__host__ __device__ inline int subst_flag_ints(int nt, int nc) { return (2 * nt * nc + 2) * SUB_FLAG_STRIDE; }

// row pieces of tile row i
__host__ __device__ inline int subst_rows(const SubstArgs &p, int i)
{
    const int tk = (p.n - i * p.T) < p.T ? p.n - i * p.T : p.T;
    return (tk + SUB_TR - 1) / SUB_TR;
}

__host__ __device__ inline int subst_groups(const SubstArgs &p)
{
    return p.nc * (p.nr * (p.nt - 1) + subst_rows(p, p.nt - 1));
}

// Piece of workgroup g: tile row i, row piece rt, column piece ct.
__host__ __device__ inline void subst_piece(const SubstArgs &p, int g, int &i, int &rt, int &ct)
{
    const int first = subst_rows(p, p.nt - 1) * p.nc;
    int idx;
    if (g < first) {
        i = p.nt - 1;
        idx = g;
    } else {
        const int q = g - first, blk = p.nr * p.nc;
        i = p.nt - 2 - q / blk;
        idx = q % blk;
    }
    rt = idx / p.nc;
    ct = idx % p.nc;
}

// Thread 0 polls *f until it reaches target (or the abort word is raised, or
// the time limit passes: then it raises the abort word and sets info = -1
// unless info is set); then the workgroup proceeds.
__device__ inline void subst_wait(const int *f, int target, int *abort_word, int64_t limit, int *info)
{
    if (threadIdx.x == 0) {
        const int64_t t0 = (int64_t)wall_clock64(), max_polls = limit / 16 + 64;
        for (int64_t polls = 0;; ++polls) {
            if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target)
                break;
            if ((polls & 3) == 3 && __hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
                break;
            if ((int64_t)wall_clock64() - t0 > limit || polls > max_polls) {
                __hip_atomic_store(abort_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (info != nullptr)
                    atomicCAS(info, 0, -1);
                break;
            }
            __builtin_amdgcn_s_sleep(SUB_POLL_SLEEP);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

// Every wave's stores are made visible at agent scope, then thread 0 adds 1
// to the counter (or raises the flag).
__device__ inline void subst_signal(int *f)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(f, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The SUB_TR x TC piece a half workgroup (256 threads, h = tid / 256)
// accumulates: wave w of the half holds rows 16 (w % 2) .. + 16 and columns
// (TC / 2) (w / 2) .. + TC / 2 as FN 16 x 16 accumulators (real and
// imaginary planes for complex types); accumulator b element q of lane
// (li, lk) is (16 (w % 2) + li, (TC / 2) (w / 2) + 16 b + acc_row(lk, q)).
template <typename R, bool CPLX, int TC>
struct SubstAcc {
    typedef typename AccT<R>::type V4;
    typedef typename Elem<R, CPLX>::type E;
    static constexpr int FN = TC / 32;
    static constexpr int NP = CPLX ? 2 : 1;
    V4 t[NP][FN];

    __device__ __forceinline__ static int row() { return 16 * ((threadIdx.x >> 6) & 1) + (threadIdx.x & 15); }
    __device__ __forceinline__ static int col(int b, int q)
    {
        return (TC / 2) * ((threadIdx.x >> 7) & 1) + 16 * b + acc_row<R>((threadIdx.x & 63) >> 4, q);
    }
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int c = 0; c < NP; ++c)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                t[c][b] = V4{0, 0, 0, 0};
    }
    // -src(r, c) for r < nr, c < nc (zero elsewhere)
    __device__ __forceinline__ void load_neg(const E *src, int64_t ld, int nr, int nc)
    {
#pragma unroll
        for (int b = 0; b < FN; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = row(), c = col(b, q);
                R x = R(0), y = R(0);
                if (r < nr && c < nc)
                    Elem<R, CPLX>::load(src + r + (int64_t)c * ld, x, y);
                t[0][b][q] = -x;
                if constexpr (CPLX)
                    t[NP - 1][b][q] = -y;
            }
    }
    // dst(r, c) = sg * this for r < nr, c < nc
    __device__ __forceinline__ void store(E *dst, int64_t ld, int nr, int nc, R sg) const
    {
#pragma unroll
        for (int b = 0; b < FN; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = row(), c = col(b, q);
                if (r < nr && c < nc)
                    Elem<R, CPLX>::store(dst + r + (int64_t)c * ld, sg * t[0][b][q], sg * t[NP - 1][b][q]);
            }
    }
    // the second half's accumulators are added to the first's through M
    // (at least NP SUB_TR TC elements of LDS no thread still reads); both
    // halves call it
    __device__ __forceinline__ void fold(R *M)
    {
        const int slot = threadIdx.x & 255;
        if (threadIdx.x >= 256) {
#pragma unroll
            for (int c = 0; c < NP; ++c)
#pragma unroll
                for (int b = 0; b < FN; ++b)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        M[((c * FN + b) * 4 + q) * 256 + slot] = t[c][b][q];
        }
        __syncthreads();
        if (threadIdx.x < 256) {
#pragma unroll
            for (int c = 0; c < NP; ++c)
#pragma unroll
                for (int b = 0; b < FN; ++b)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        t[c][b][q] += M[((c * FN + b) * 4 + q) * 256 + slot];
        }
        __syncthreads();
    }
};

// Each half's LDS: one chunk of both operands.  Within every 16-deep block
// of a row, depth 4 s + g sits at position 4 g + s, so that the four operands
// lane (i, g) gives the four 16x16x4 products of that block (depths 4 s + g,
// s = 0 .. 3) are adjacent and arrive in 16-byte reads; rows are padded by
// 16 bytes (aligned, and spread over the banks).
template <typename R, bool CPLX, int TC, int KC>
struct SubstStage {
    static constexpr int NP = CPLX ? 2 : 1;
    static constexpr int LDR = KC + 16 / (int)sizeof(R);
    R As[NP][SUB_TR][LDR];  // As[.][r][pos(k)] = conj(M(k0 + k, r))
    R Bs[NP][TC][LDR];      // Bs[.][c][pos(k)] = Q(k0 + k, c)
    __device__ __forceinline__ static int pos(int k) { return (k & ~15) + 4 * (k & 3) + ((k >> 2) & 3); }
};

// v[s] = p[s], s < 4, in 16-byte reads (p 16-byte aligned)
__device__ __forceinline__ void lds4(const float *p, float (&v)[4])
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 x = *(const f4 *)p;
    v[0] = x[0];
    v[1] = x[1];
    v[2] = x[2];
    v[3] = x[3];
}
__device__ __forceinline__ void lds4(const double *p, double (&v)[4])
{
    typedef double d2 __attribute__((ext_vector_type(2)));
    const d2 x = *(const d2 *)p, y = *(const d2 *)(p + 2);
    v[0] = x[0];
    v[1] = x[1];
    v[2] = y[0];
    v[3] = y[1];
}

// acc += M^H Q: M(k, r) = m[k + r ldm] for k < K, r < nr and Q(k, c) =
// q[k + c ldq] for k < K, c < nc (zero elsewhere).  The depth goes in steps
// of 2 KC: half h of the workgroup takes [2 KC s + h KC, + KC) into its own
// stage and accumulators, and the loads of its next chunk are in flight
// while its matrix-core waves work on the current one.  Each 16x16x4 product
// takes the operands mma16 (mma16c) would, in the same order.
template <typename R, bool CPLX, int TC, int KC>
__device__ __forceinline__ void subst_mma(SubstAcc<R, CPLX, TC> &acc, const typename Elem<R, CPLX>::type *m,
                                          int64_t ldm, int K, int nr, const typename Elem<R, CPLX>::type *q,
                                          int64_t ldq, int nc, SubstStage<R, CPLX, TC, KC> *st)
{
    typedef SubstStage<R, CPLX, TC, KC> Stage;
    constexpr int NP = CPLX ? 2 : 1;
    constexpr int LA = SUB_TR * KC / 256, LB = TC * KC / 256;
    static_assert((SUB_TR * KC) % 256 == 0 && (TC * KC) % 256 == 0, "chunk loads must divide evenly");
    static_assert(KC % 16 == 0, "chunks are whole 16-deep blocks");
    const int h = threadIdx.x >> 8, tid = threadIdx.x & 255, wave = tid >> 6;
    const int li = tid & 15, lk = (tid >> 4) & 3;
    const int ro = 16 * (wave & 1), co = (TC / 2) * (wave >> 1);
    Stage &S = st[h];
    R ra[NP][LA], rb[NP][LB];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int u = 0; u < LA; ++u) {
            const int e = tid + 256 * u, k = e % KC, r = e / KC;
            R x = R(0), y = R(0);
            if (k0 + k < K && r < nr)
                Elem<R, CPLX>::load(m + (k0 + k) + (int64_t)r * ldm, x, y);
            ra[0][u] = x;
            if constexpr (CPLX)
                ra[NP - 1][u] = -y;
        }
#pragma unroll
        for (int u = 0; u < LB; ++u) {
            const int e = tid + 256 * u, k = e % KC, c = e / KC;
            R x = R(0), y = R(0);
            if (k0 + k < K && c < nc)
                Elem<R, CPLX>::load(q + (k0 + k) + (int64_t)c * ldq, x, y);
            rb[0][u] = x;
            if constexpr (CPLX)
                rb[NP - 1][u] = y;
        }
    };
    const int steps = (K + 2 * KC - 1) / (2 * KC);
    fetch(h * KC);
    for (int s = 0; s < steps; ++s) {
        __syncthreads();  // the previous chunk's products are done with the LDS
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) {
#pragma unroll
            for (int u = 0; u < LA; ++u) {
                const int e = tid + 256 * u;
                S.As[pl][e / KC][Stage::pos(e % KC)] = ra[pl][u];
            }
#pragma unroll
            for (int u = 0; u < LB; ++u) {
                const int e = tid + 256 * u;
                S.Bs[pl][e / KC][Stage::pos(e % KC)] = rb[pl][u];
            }
        }
        __syncthreads();
        if (s + 1 < steps)
            fetch(2 * KC * (s + 1) + h * KC);
#pragma unroll 2
        for (int k = 0; k < KC; k += 16) {
            R a[NP][4], bv[NP][acc.FN][4];
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) {
                lds4(&S.As[pl][ro + li][k + 4 * lk], a[pl]);
#pragma unroll
                for (int b = 0; b < acc.FN; ++b)
                    lds4(&S.Bs[pl][co + 16 * b + li][k + 4 * lk], bv[pl][b]);
            }
#pragma unroll
            for (int b = 0; b < acc.FN; ++b)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if constexpr (!CPLX) {
                        acc.t[0][b] = mfma16(bv[0][b][u], a[0][u], acc.t[0][b]);
                    } else {
                        acc.t[0][b] = mfma16(bv[0][b][u], a[0][u], acc.t[0][b]);
                        acc.t[0][b] = mfma16(-bv[1][b][u], a[1][u], acc.t[0][b]);
                        acc.t[1][b] = mfma16(bv[1][b][u], a[0][u], acc.t[1][b]);
                        acc.t[1][b] = mfma16(bv[0][b][u], a[1][u], acc.t[1][b]);
                    }
                }
        }
    }
}

// SUB_THREADS threads: two halves of 256 share each product (subst_mma).
template <typename R, bool CPLX, int TC>
__global__ void __launch_bounds__(SUB_THREADS) __attribute__((amdgpu_waves_per_eu(4))) subst_kernel(const SubstArgs p)
{
    typedef typename Elem<R, CPLX>::type E;
    constexpr int KC = CPLX ? (TC == 64 ? 16 : 32) : (sizeof(R) == 4 && TC == 64 ? 32 : 64);  // chunk depth: the staging registers of two chunks fit
    typedef SubstStage<R, CPLX, TC, KC> Stage;
    static_assert(2 * sizeof(Stage) >= sizeof(R) * (CPLX ? 2 : 1) * SUB_TR * TC, "the fold needs both stages");
    __shared__ Stage st[2];
    __shared__ int skip, last;

    int i, rt, ct;
    subst_piece(p, (int)blockIdx.x, i, rt, ct);
    const int tid = threadIdx.x;
    const int frows = p.nt * p.nc;
    int *const abort_word = p.flags + 2 * frows * SUB_FLAG_STRIDE;
    int *const ctr = abort_word + SUB_FLAG_STRIDE;
    auto fZ = [&](int ti, int c) { return p.flags + (ti * p.nc + c) * SUB_FLAG_STRIDE; };
    auto fX = [&](int ti, int c) { return p.flags + (frows + ti * p.nc + c) * SUB_FLAG_STRIDE; };
    auto tile_rows = [&](int ti) { return (p.n - ti * p.T) < p.T ? p.n - ti * p.T : p.T; };
    const E *const A = (const E *)p.A;
    E *const B = (E *)p.B;
    E *const Zi = (E *)p.Z + (i & 1) * p.ldz * p.nrhs;  // tile row i's Z buffer
    const int tki = tile_rows(i), r0 = rt * SUB_TR, c0 = ct * TC;
    const int nrow = (tki - r0) < SUB_TR ? tki - r0 : SUB_TR;
    const int ncol = (p.nrhs - c0) < TC ? p.nrhs - c0 : TC;
    const int64_t row0 = (int64_t)i * p.T;  // first row of tile row i
    const bool first = tid < 256;          // the half that holds the result

    if (tid == 0)
        skip = (p.info != nullptr && *(volatile const int *)p.info != 0) ? 1 : 0;
    __syncthreads();
    if (!skip) {
        SubstAcc<R, CPLX, TC> acc;
        {  // R
            if (first)
                acc.load_neg(B + row0 + r0 + (int64_t)c0 * p.ldb, p.ldb, nrow, ncol);
            else
                acc.zero();
            for (int j = p.nt - 1; j > i + 1; --j) {
                subst_wait(fX(j, ct), subst_rows(p, j), abort_word, p.limit, p.status);
                const int64_t rj = (int64_t)j * p.T;
                // -Z += L(rows of j, columns of the piece)^H X_j(:, ct)
                subst_mma<R, CPLX, TC, KC>(acc, A + rj + (row0 + r0) * p.lda, p.lda, tile_rows(j), nrow,
                                           B + rj + (int64_t)c0 * p.ldb, p.ldb, ncol, st);
            }
            __syncthreads();
            acc.fold((R *)st);
            if (first)
                acc.store(Zi + r0 + (int64_t)c0 * p.ldz, p.ldz, nrow, ncol, R(-1));
            subst_signal(fZ(i, ct));
        }
        {  // C
            subst_wait(fZ(i, ct), subst_rows(p, i), abort_word, p.limit, p.status);
            acc.zero();
            // X = inv(L_ii)(rows r0.., columns of the piece)^H Z_i(r0.., ct)
            const E *const Iv = (const E *)p.Inv + (int64_t)i * p.T * p.T;
            subst_mma<R, CPLX, TC, KC>(acc, Iv + r0 + (int64_t)r0 * p.T, p.T, tki - r0, nrow,
                                       Zi + r0 + (int64_t)c0 * p.ldz, p.ldz, ncol, st);
            if (i + 1 < p.nt) {
                // + G_i(:, columns of the piece)^H X_{i+1}(:, ct)
                subst_wait(fX(i + 1, ct), subst_rows(p, i + 1), abort_word, p.limit, p.status);
                const E *const Gi = (const E *)p.G + (int64_t)(i + 1) * p.T * p.T;
                subst_mma<R, CPLX, TC, KC>(acc, Gi + (int64_t)r0 * p.T, p.T, tile_rows(i + 1), nrow,
                                           B + row0 + p.T + (int64_t)c0 * p.ldb, p.ldb, ncol, st);
            }
            __syncthreads();
            acc.fold((R *)st);
            if (first)
                acc.store(B + row0 + r0 + (int64_t)c0 * p.ldb, p.ldb, nrow, ncol, R(1));
            subst_signal(fX(i, ct));
        }
    }

    // count out (the stores above visible first, for the NaN fill below)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0)
        last = atomicAdd(ctr, 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const bool aborted = *(volatile int *)abort_word != 0;
        const int nf = (2 * frows + 1) * SUB_FLAG_STRIDE;  // all lines but the count of workgroups done
        for (int e = tid; e < nf; e += blockDim.x)
            p.flags[e] = 0;
        if (tid == 0)
            *ctr = 0;
        if (aborted) {
            const R nan = __builtin_nan("");
            for (int64_t e = tid; e < (int64_t)p.n * p.nrhs; e += blockDim.x)
                Elem<R, CPLX>::store(B + e % p.n + (e / p.n) * p.ldb, nan, nan);
        }
    }
}

}  // namespace spd
