// The diagonal tile of the blocked Cholesky factorization in one launch, real
// types: A_kk = L_kk L_kk^T and inv(L_kk) (JAXMg paper, "Software design":
// step 1 of each tile of potrf, and the tile inverses that the panel solve and
// the substitutions apply).
//
// The tile (order tk <= T) is cut into nb = ceil(tk / 64) block rows and
// columns.  Every 64 x 64 block of the lower triangle of L, and every block
// below the diagonal of inv(L_kk), is computed by a workgroup of its own
// (left-looking, so each block is written once):
//
//   D_j  (diagonal role, block row j):
//        S    = A_j,j-1 - sum_{l < j-1} L_jl L_j-1,l^T
//        L_j,j-1 = S inv(L_j-1,j-1)^T          (published before the leaf)
//        A'   = A_jj - sum_{l < j} L_jl L_jl^T
//        L_jj, inv(L_jj) from A' inside LDS (the 64 x 64 leaf of the
//        multi-kernel path, the same arithmetic); inv(L_jj) is published
//        before L_jj is stored (no role of the launch reads L_jj)
//   O_ij (i >= j + 2):
//        L_ij = (A_ij - sum_{l < j} L_il L_jl^T) inv(L_jj)^T
//   X_ib (i > b):
//        inv(L)_ib = -inv(L_ii) sum_{b <= k < i} L_ik inv(L)_kb
//
// With wk > 0 the tile first takes the last update of the trailing matrix
// itself: every L block role starts from A_ij - W_i W_j^T, with W (ldw) the
// previous panel's rows of this tile (wk columns), so that the launch need
// not wait for a separate update of the tile.
//
// Each block has a ready flag in the workspace.  A workgroup waits for the
// flags of the blocks it reads (its thread 0 polls with agent-scope loads,
// then an acquire fence) and raises its own after its stores (release fence,
// then an agent-scope store).  Workgroup ids are assigned in the order
// D_0, O_2..nb-1,0, D_1, O_3..,1, ..., D_nb-1, then X_ib by (i, b): every
// block a workgroup waits for belongs to a smaller id.  Workgroups are
// dispatched in id order, so a waiting workgroup never holds back the one it
// waits for; every wait is also bounded in time (a wait that runs out raises
// an abort word that ends every other wait, and sets info to -1), so each
// wave of the launch exits.  Each workgroup counts itself out at the end and
// the last one clears the flags, so they are zero between launches.
#pragma once

#include "spd_kernels.hpp"

namespace spd {

struct TileArgs {
    void *D;        // the diagonal tile: its first element, column-major, lda
    int64_t lda;
    void *Inv;      // inv(L_kk): first element, leading dimension ldi; blocks
    int64_t ldi;    // below and on the diagonal written, the rest left as is
    int tk;         // order of the tile
    int nb;         // block rows = ceil(tk / 64)
    int *flags;     // tile_flag_ints(nb) ints, zero between launches
    int *info;      // first failing global column + 1 (kept if already set);
                    // -1 if a wait ran out of time
    int col0;       // global column of the tile's first column
    int64_t limit;  // longest wait, in ticks of the 100 MHz wall clock
    int hold;       // real types: 1 to launch 512 threads per workgroup (see tile_kernel)
    const void *W;  // wk > 0: A_ij -= W_i W_j^H first, W (ldw) the previous
    int64_t ldw;    // panel's rows of this tile, wk columns (a multiple of 64
    int wk;         // or the panel's zero-padded width)
};

enum { TILE_D = 0, TILE_O = 1, TILE_X = 2 };

__host__ __device__ inline int tile_groups(int nb) { return nb * nb - nb + 1; }
// flags: L blocks (nb x nb), inverse blocks (nb x nb), the abort word and the
// workgroup counter, each on a 128-byte line of its own (TILE_FLAG_STRIDE
// ints), so that polls and raises of different flags go to different lines
constexpr int TILE_FLAG_STRIDE = 32;
__host__ __device__ inline int tile_flag_ints(int nb) { return (2 * nb * nb + 2) * TILE_FLAG_STRIDE; }

// Role of workgroup g: kind and block (i, j); -1 past the last role.
__host__ __device__ inline int tile_role(int nb, int g, int &i, int &j)
{
    for (int c = 0; c < nb; ++c) {
        if (g == 0) {
            i = c;
            j = c;
            return TILE_D;
        }
        --g;
        const int no = nb - c - 2 > 0 ? nb - c - 2 : 0;
        if (g < no) {
            i = c + 2 + g;
            j = c;
            return TILE_O;
        }
        g -= no;
    }
    for (int r = 1; r < nb; ++r) {
        if (g < r) {
            i = r;
            j = g;
            return TILE_X;
        }
        g -= r;
    }
    i = j = -1;
    return -1;
}

// Thread 0 polls the flags (f2 may be null) until both are raised, the abort
// word (looked at every fourth poll) is raised, or the time limit passes (then
// it raises the abort word and records info = -1 unless info is set); then the
// workgroup proceeds.
__device__ inline void tile_wait(const int *f1, const int *f2, int *abort_word, int64_t limit, int *info)
{
    if (threadIdx.x == 0) {
        // the poll count bounds the wait as well, should the clock not run
        // (one poll takes well over 16 ticks: two or three agent-scope loads)
        const int64_t t0 = (int64_t)wall_clock64(), max_polls = limit / 16 + 64;
        for (int64_t polls = 0;; ++polls) {
            if (__hip_atomic_load(f1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 &&
                (f2 == nullptr || __hip_atomic_load(f2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0))
                break;
            if ((polls & 3) == 3 && __hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
                break;
            if ((int64_t)wall_clock64() - t0 > limit || polls > max_polls) {
                __hip_atomic_store(abort_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (info != nullptr)
                    atomicCAS(info, 0, -1);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

// Every wave's stores are made visible at agent scope, then thread 0 raises
// the flag.
__device__ inline void tile_signal(int *flag)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A 64 x 64 block in flight between global memory and LDS: thread (r, g) =
// (tid % 64, tid / 64) holds elements (r, g + 4k), k < 16.
template <typename R>
struct TileBlk {
    R v[LEAF / 4];

    // src(r, c) for r < nr, c < nc, zero elsewhere; lower: zero above the
    // diagonal as well
    __device__ __forceinline__ void load(const R *src, int64_t ld, int nr, int nc, bool lower)
    {
        const int r = threadIdx.x & 63, g = threadIdx.x >> 6;
#pragma unroll
        for (int k = 0; k < LEAF / 4; ++k) {
            const int c = g + 4 * k;
            v[k] = R(0);
            if (r < nr && c < nc && (!lower || r >= c))
                v[k] = src[r + (int64_t)c * ld];
        }
    }
    __device__ __forceinline__ void put(R (*M)[LDL]) const
    {
        const int r = threadIdx.x & 63, g = threadIdx.x >> 6;
#pragma unroll
        for (int k = 0; k < LEAF / 4; ++k)
            M[g + 4 * k][r] = v[k];
    }
};

// This wave's four 16 x 16 tiles of a 64 x 64 block: tile t covers columns
// 16 t .. and rows 16 ((w - t) mod 4) .. (w = wave), one tile in every block
// row and block column, so that the products whose depth depends on the
// tile's row or column (triangular operands, the lower triangle only) share
// out evenly over the four waves.  Element q of lane (li, lk) in tile t is
// (16 ((w - t) mod 4) + li, 16 t + acc_row(lk, q)).
template <typename R>
struct TileQuad {
    typedef typename AccT<R>::type V4;
    V4 t[4];

    __device__ __forceinline__ static int rblk(int u) { return ((int)(threadIdx.x >> 6) - u) & 3; }
    __device__ __forceinline__ static int row(int u) { return 16 * rblk(u) + (threadIdx.x & 15); }
    __device__ __forceinline__ static int col(int u, int q) { return 16 * u + acc_row<R>((threadIdx.x & 63) >> 4, q); }
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            t[u] = V4{0, 0, 0, 0};
    }
    // -src(r, c) for r < nr, c < nc; diag: zero above the diagonal and -1 on
    // the diagonal beyond nr (the identity padding of a short last block)
    __device__ __forceinline__ void load_neg(const R *src, int64_t ld, int nr, int nc, bool diag)
    {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = row(u), c = col(u, q);
                R x = (diag && r == c) ? R(-1) : R(0);
                if (r < nr && c < nc && (!diag || r >= c))
                    x = -src[r + (int64_t)c * ld];
                t[u][q] = x;
            }
    }
    __device__ __forceinline__ void to_lds(R (*M)[LDL], R sg) const
    {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                M[col(u, q)][row(u)] = sg * t[u][q];
    }
    __device__ __forceinline__ void store(R *dst, int64_t ld, int nr, R sg) const
    {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = row(u), c = col(u, q);
                if (r < nr)
                    dst[r + (int64_t)c * ld] = sg * t[u][q];
            }
    }
};

// Depth ranges of a 16 x 16 product tile at (ro, co) (multiples of 16)
enum {
    TK_FULL = 0,     // [0, 64)
    TK_TO_COL = 1,   // [0, co + 16): right operand X^T with X lower triangular
    TK_FROM_COL = 2, // [co, 64): right operand lower triangular
    TK_TO_ROW = 3,   // [0, ro + 16): left operand lower triangular
};

// Q += P B on this wave's tiles, P(r, k) = pa[k ak + r ar], B(k, c) =
// pb[k bk + c bc] (both 64 x 64 in LDS); lower: only the tiles on or below
// the diagonal.
template <typename R>
__device__ __forceinline__ void tile_mma(TileQuad<R> &Q, const R *pa, int ak, int ar, const R *pb, int bk, int bc,
                                         int kmode, bool lower)
{
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int ro = 16 * TileQuad<R>::rblk(u), co = 16 * u;
        if (lower && co > ro)
            continue;
        int k0 = 0, k1 = LEAF;
        if (kmode == TK_TO_COL)
            k1 = co + 16;
        else if (kmode == TK_FROM_COL)
            k0 = co;
        else if (kmode == TK_TO_ROW)
            k1 = ro + 16;
        for (int k = k0; k < k1; k += 16)
            Q.t[u] = mma16<R>(pa + k * ak + ro * ar, ak, ar, pb + k * bk + co * bc, bk, bc, Q.t[u]);
    }
}

// Launched with 256 threads, or with 512 (TileArgs::hold): then waves 4-7 do
// no work and only meet every barrier of waves 0-3 until those are done.  They
// hold registers, so that no wave of another kernel (the trailing update)
// shares a SIMD with this workgroup's working waves: the leaf's sweeps, one
// wave's long chain of vector instructions, then run at their own pace
// instead of sharing the multiply pipeline with matrix-core waves.
template <typename R>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) tile_kernel(const TileArgs p)
{
    __shared__ R S[LEAF][LDL];
    __shared__ R X[LEAF][LDL];
    __shared__ R Tm[4][LB16][LB16 + 1];
    __shared__ int failed, last, done;

    if (threadIdx.x == 0)
        done = 0;
    if (threadIdx.x >= 256) {
        do
            __syncthreads();
        while (!done);
        return;
    }
    const int tid = threadIdx.x, nb = p.nb;
    int bi, bj;
    const int kind = tile_role(nb, (int)blockIdx.x, bi, bj);
    R *const A = (R *)p.D;
    R *const Iv = (R *)p.Inv;
    int *const abort_word = p.flags + 2 * nb * nb * TILE_FLAG_STRIDE;
    int *const ctr = abort_word + TILE_FLAG_STRIDE;
    auto nrows = [&](int b) { return (p.tk - b * LEAF) < LEAF ? p.tk - b * LEAF : LEAF; };
    auto Ab = [&](int i, int j) { return A + (int64_t)i * LEAF + (int64_t)j * LEAF * p.lda; };
    auto Xb = [&](int i, int j) { return Iv + (int64_t)i * LEAF + (int64_t)j * LEAF * p.ldi; };
    auto fL = [&](int i, int j) { return p.flags + (i * nb + j) * TILE_FLAG_STRIDE; };
    auto fX = [&](int i, int j) { return p.flags + (nb * nb + i * nb + j) * TILE_FLAG_STRIDE; };
    auto wait = [&](const int *f1, const int *f2) { tile_wait(f1, f2, abort_word, p.limit, p.info); };
    TileBlk<R> u, w;

    // W_i (rows of block i of the previous panel), columns [c, c + 64)
    const R *const Wp = (const R *)p.W;
    auto Wb = [&](int i, int c) { return Wp + (int64_t)i * LEAF + (int64_t)c * p.ldw; };

    if (kind == TILE_D) {
        const int j = bi, nr = nrows(j);
        TileQuad<R> Fd, Fs;
        Fd.load_neg(Ab(j, j), p.lda, nr, nr, true);
        if (j > 0)
            Fs.load_neg(Ab(j, j - 1), p.lda, nr, LEAF, false);
        for (int c = 0; c < p.wk; c += LEAF) {  // the tile's last trailing update
            u.load(Wb(j, c), p.ldw, nr, p.wk - c, false);
            if (j > 0)
                w.load(Wb(j - 1, c), p.ldw, LEAF, p.wk - c, false);
            u.put(S);
            if (j > 0)
                w.put(X);
            __syncthreads();
            if (j > 0)
                tile_mma<R>(Fs, &S[0][0], LDL, 1, &X[0][0], LDL, 1, TK_FULL, false);
            tile_mma<R>(Fd, &S[0][0], LDL, 1, &S[0][0], LDL, 1, TK_FULL, true);
            __syncthreads();
        }
        for (int l = 0; l + 1 < j; ++l) {
            wait(fL(j, l), fL(j - 1, l));
            u.load(Ab(j, l), p.lda, nr, LEAF, false);
            w.load(Ab(j - 1, l), p.lda, LEAF, LEAF, false);
            u.put(S);
            w.put(X);
            __syncthreads();
            tile_mma<R>(Fs, &S[0][0], LDL, 1, &X[0][0], LDL, 1, TK_FULL, false);
            tile_mma<R>(Fd, &S[0][0], LDL, 1, &S[0][0], LDL, 1, TK_FULL, true);
            __syncthreads();
        }
        if (j > 0) {
            // L_j,j-1 = (A_j,j-1 - ...) inv(L_j-1,j-1)^T
            wait(fL(j - 1, j - 1), nullptr);
            w.load(Xb(j - 1, j - 1), p.ldi, LEAF, LEAF, true);
            Fs.to_lds(S, R(-1));
            w.put(X);
            __syncthreads();
            TileQuad<R> G;
            G.zero();
            tile_mma<R>(G, &S[0][0], LDL, 1, &X[0][0], LDL, 1, TK_TO_COL, false);
            __syncthreads();
            G.store(Ab(j, j - 1), p.lda, nr, R(1));
            G.to_lds(S, R(1));
            __syncthreads();
            tile_mma<R>(Fd, &S[0][0], LDL, 1, &S[0][0], LDL, 1, TK_FULL, true);
            __syncthreads();
        }
        Fd.to_lds(S, R(-1));
#pragma unroll
        for (int k = 0; k < LEAF / 4; ++k)
            X[(tid >> 6) + 4 * k][tid & 63] = R(0);
        if (tid == 0)
            failed = 0;
        // L_j,j-1 is published only now, when its stores have long completed
        // (nothing needs it before the next diagonal block); the barrier of
        // the signal also serves the leaf
        if (j > 0)
            tile_signal(fL(j, j - 1));
        else
            __syncthreads();
        leaf_lds<R>(S, X, Tm, true, nr, p.col0 + j * LEAF, p.info, &failed);
        // inv(L_jj) first: the other roles wait for it, and none reads L_jj
        const int r = tid & 63, g = tid >> 6;
        {
            R *const Xd = Xb(j, j);
#pragma unroll
            for (int k = 0; k < LEAF / 4; ++k) {
                const int c = g + 4 * k;
                if (r < nr && c < nr)
                    Xd[r + (int64_t)c * p.ldi] = (r >= c) ? X[c][r] : R(0);
            }
        }
        tile_signal(fL(j, j));
        {
            R *const Ad = Ab(j, j);
#pragma unroll
            for (int k = 0; k < LEAF / 4; ++k) {
                const int c = g + 4 * k;
                if (r < nr && c < nr && r >= c)
                    Ad[r + (int64_t)c * p.lda] = S[c][r];
            }
        }
    } else if (kind == TILE_O) {
        const int i = bi, j = bj, nr = nrows(i);
        TileQuad<R> F;
        F.load_neg(Ab(i, j), p.lda, nr, LEAF, false);
        for (int c = 0; c < p.wk; c += LEAF) {  // the tile's last trailing update
            u.load(Wb(i, c), p.ldw, nr, p.wk - c, false);
            w.load(Wb(j, c), p.ldw, LEAF, p.wk - c, false);
            u.put(S);
            w.put(X);
            __syncthreads();
            tile_mma<R>(F, &S[0][0], LDL, 1, &X[0][0], LDL, 1, TK_FULL, false);
            __syncthreads();
        }
        for (int l = 0; l < j; ++l) {
            wait(fL(i, l), fL(j, l));
            u.load(Ab(i, l), p.lda, nr, LEAF, false);
            w.load(Ab(j, l), p.lda, LEAF, LEAF, false);
            u.put(S);
            w.put(X);
            __syncthreads();
            tile_mma<R>(F, &S[0][0], LDL, 1, &X[0][0], LDL, 1, TK_FULL, false);
            __syncthreads();
        }
        wait(fL(j, j), nullptr);
        w.load(Xb(j, j), p.ldi, LEAF, LEAF, true);
        F.to_lds(S, R(-1));
        w.put(X);
        __syncthreads();
        TileQuad<R> G;
        G.zero();
        tile_mma<R>(G, &S[0][0], LDL, 1, &X[0][0], LDL, 1, TK_TO_COL, false);
        G.store(Ab(i, j), p.lda, nr, R(1));
        tile_signal(fL(i, j));
    } else if (kind == TILE_X) {
        const int i = bi, b = bj, nr = nrows(i);
        TileQuad<R> G;
        G.zero();
        for (int k = b; k < i; ++k) {
            wait(fL(i, k), k == b ? fL(b, b) : fX(k, b));
            u.load(Ab(i, k), p.lda, nr, LEAF, false);
            w.load(Xb(k, b), p.ldi, LEAF, LEAF, k == b);
            u.put(S);
            w.put(X);
            __syncthreads();
            // G += L_ik inv(L)_kb: B(k, c) = X[c][k]
            tile_mma<R>(G, &S[0][0], LDL, 1, &X[0][0], 1, LDL, k == b ? TK_FROM_COL : TK_FULL, false);
            __syncthreads();
        }
        wait(fL(i, i), nullptr);
        w.load(Xb(i, i), p.ldi, nr, nr, true);
        G.to_lds(S, R(1));
        w.put(X);
        __syncthreads();
        // H = inv(L_ii) G: P(r, k) = X[k][r], B(k, c) = S[c][k]
        TileQuad<R> H;
        H.zero();
        tile_mma<R>(H, &X[0][0], LDL, 1, &S[0][0], 1, LDL, TK_TO_ROW, false);
        H.store(Xb(i, b), p.ldi, nr, R(-1));
        tile_signal(fX(i, b));
    }

    // count out; the last workgroup clears the flags for the next launch
    __syncthreads();
    if (tid == 0)
        last = atomicAdd(ctr, 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (last) {
        for (int e = tid; e < (2 * nb * nb + 1) * TILE_FLAG_STRIDE; e += 256)
            p.flags[e] = 0;
        if (tid == 0)
            *ctr = 0;
    }
    if (tid == 0)
        done = 1;  // the idle waves leave after this barrier
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Complex types: the same roles, flags and order, with conjugate transposes
// (L_ij = (A_ij - sum_l L_il L_jl^H) inv(L_jj)^H, the leaf as the complex
// multi-kernel leaf).  The blocks other workgroups publish are read straight
// from global memory into the matrix-core operand registers; LDS holds only
// what a workgroup hands between its own waves (its updated block before the
// solve product, L_j,j-1 before the diagonal update) and the leaf.

// This wave's four 16 x 16 tiles of a complex 64 x 64 block: tile t covers
// columns 16 t .. and rows 16 ((w - t) mod 4) .. (w = wave), one tile in every
// block row and block column, so that the products whose depth depends on
// the tile's row or column (triangular operands, the lower triangle only)
// share out evenly over the four waves.  Element q of lane (li, lk) in tile
// t is (16 ((w - t) mod 4) + li, 16 t + acc_row(lk, q)).
template <typename R>
struct TileQuadC {
    typedef typename AccT<R>::type V4;
    typedef typename Elem<R, true>::type E;
    V4 re[4], im[4];

    __device__ __forceinline__ static int rblk(int t) { return ((int)(threadIdx.x >> 6) - t) & 3; }
    __device__ __forceinline__ static int row(int t) { return 16 * rblk(t) + (threadIdx.x & 15); }
    __device__ __forceinline__ static int col(int t, int q) { return 16 * t + acc_row<R>((threadIdx.x & 63) >> 4, q); }

    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            re[t] = V4{0, 0, 0, 0};
            im[t] = V4{0, 0, 0, 0};
        }
    }
    // -src(r, c) for r < nr, c < nc; diag: zero above the diagonal, a real
    // diagonal, and -1 on the diagonal beyond nr
    __device__ __forceinline__ void load_neg(const E *src, int64_t ld, int nr, int nc, bool diag)
    {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = row(t), c = col(t, q);
                R x = (diag && r == c) ? R(-1) : R(0), y = R(0);
                if (r < nr && c < nc && (!diag || r >= c)) {
                    Elem<R, true>::load(src + r + (int64_t)c * ld, x, y);
                    x = -x;
                    y = (diag && r == c) ? R(0) : -y;
                }
                re[t][q] = x;
                im[t][q] = y;
            }
    }
    // planes S[0] + i S[1] (S*[c][r] = element (r, c)) = sg * this; realdiag:
    // the diagonal's imaginary part is stored as 0
    __device__ __forceinline__ void to_lds(R (*S)[LEAF][LDL], R sg, bool realdiag) const
    {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = row(t), c = col(t, q);
                S[0][c][r] = sg * re[t][q];
                S[1][c][r] = (realdiag && r == c) ? R(0) : sg * im[t][q];
            }
    }
    __device__ __forceinline__ void store(E *dst, int64_t ld, int nr, R sg) const
    {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = row(t), c = col(t, q);
                if (r < nr)
                    Elem<R, true>::store(dst + r + (int64_t)c * ld, sg * re[t][q], sg * im[t][q]);
            }
    }
};

// Q += P B on this wave's tiles for complex 64 x 64 operands given by fa(r,
// k, re, im) = P(r, k) and fb(k, c, re, im) = B(k, c); kmode and lower as
// tile_mma.  Each 16-deep step first fetches the operands of all the wave's
// tiles that take it (in the lane layout of mma16: lane (li, lk) takes
// P(row + li, k + 4 s + lk) and B(k + 4 s + lk, col + li)), then issues their
// products.
template <typename R, typename FA, typename FB>
__device__ __forceinline__ void tile_mma_c(TileQuadC<R> &Q, FA fa, FB fb, int kmode, bool lower)
{
    const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
    int k0[4], k1[4], kmin = LEAF, kmax = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int ro = 16 * TileQuadC<R>::rblk(t), co = 16 * t;
        int x0 = 0, x1 = LEAF;
        if (kmode == TK_TO_COL)
            x1 = co + 16;
        else if (kmode == TK_FROM_COL)
            x0 = co;
        else if (kmode == TK_TO_ROW)
            x1 = ro + 16;
        if (lower && co > ro)
            x1 = x0;  // no product for tiles above the diagonal
        k0[t] = x0;
        k1[t] = x1;
        if (x0 < x1) {
            kmin = x0 < kmin ? x0 : kmin;
            kmax = x1 > kmax ? x1 : kmax;
        }
    }
    for (int k = kmin; k < kmax; k += 16) {
        R ar[4][4], ai[4][4], br[4][4], bi[4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (k < k0[t] || k >= k1[t])
                continue;
            const int ro = 16 * TileQuadC<R>::rblk(t), co = 16 * t;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                fa(ro + li, k + 4 * s + lk, ar[t][s], ai[t][s]);
                fb(k + 4 * s + lk, co + li, br[t][s], bi[t][s]);
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (k < k0[t] || k >= k1[t])
                continue;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                Q.re[t] = mfma16(br[t][s], ar[t][s], Q.re[t]);
                Q.re[t] = mfma16(-bi[t][s], ai[t][s], Q.re[t]);
                Q.im[t] = mfma16(bi[t][s], ar[t][s], Q.im[t]);
                Q.im[t] = mfma16(br[t][s], ai[t][s], Q.im[t]);
            }
        }
    }
}

template <typename R>
__global__ void __launch_bounds__(256) tile_kernel_c(const TileArgs p)
{
    typedef typename Elem<R, true>::type E;
    __shared__ R S[2][LEAF][LDL];           // planes of the exchanged block, then of the leaf
    __shared__ R Xd[2][LEAF];               // diagonal of the leaf's inverse
    __shared__ R Tm[4][2][LB16][LB16 + 1];  // the leaf's per-wave scratch
    __shared__ int failed, last;

    const int tid = threadIdx.x, nb = p.nb;
    int bi, bj;
    const int kind = tile_role(nb, (int)blockIdx.x, bi, bj);
    E *const A = (E *)p.D;
    E *const Iv = (E *)p.Inv;
    int *const abort_word = p.flags + 2 * nb * nb * TILE_FLAG_STRIDE;
    int *const ctr = abort_word + TILE_FLAG_STRIDE;
    auto nrows = [&](int b) { return (p.tk - b * LEAF) < LEAF ? p.tk - b * LEAF : LEAF; };
    auto Ab = [&](int i, int j) { return A + (int64_t)i * LEAF + (int64_t)j * LEAF * p.lda; };
    auto Xb = [&](int i, int j) { return Iv + (int64_t)i * LEAF + (int64_t)j * LEAF * p.ldi; };
    auto fL = [&](int i, int j) { return p.flags + (i * nb + j) * TILE_FLAG_STRIDE; };
    auto fX = [&](int i, int j) { return p.flags + (nb * nb + i * nb + j) * TILE_FLAG_STRIDE; };
    auto wait = [&](const int *f1, const int *f2) { tile_wait(f1, f2, abort_word, p.limit, p.info); };
    // operand fetchers: M(r, k) of a global block with nr rows, its conjugate
    // transpose conj(M(c, k)) at (k, c), and the LDS planes
    auto gget = [&](const E *M, int64_t ld, int nr, int r, int k, R &x, R &y) {
        x = R(0);
        y = R(0);
        if (r < nr)
            Elem<R, true>::load(M + r + (int64_t)k * ld, x, y);
    };
    auto sget = [&](int r, int k, R &x, R &y) {
        x = S[0][k][r];
        y = S[1][k][r];
    };

    // W_i (rows of block i of the previous panel), columns [c, c + 64)
    const E *const Wp = (const E *)p.W;
    auto Wb = [&](int i, int c) { return Wp + (int64_t)i * LEAF + (int64_t)c * p.ldw; };
    // the tile's last trailing update: F += W_i W_j^H over the panel's columns
    auto pre = [&](TileQuadC<R> &F, int i, int j, int nr, int nc, bool lower) {
        for (int c = 0; c < p.wk; c += LEAF) {
            const E *U = Wb(i, c), *V = Wb(j, c);
            const int kw = p.wk - c;
            tile_mma_c<R>(
                F, [&](int r, int k, R &x, R &y) { gget(U, p.ldw, k < kw ? nr : 0, r, k, x, y); },
                [&](int k, int cc, R &x, R &y) {
                    gget(V, p.ldw, k < kw ? nc : 0, cc, k, x, y);
                    y = -y;
                },
                TK_FULL, lower);
        }
    };

    if (kind == TILE_D) {
        const int j = bi, nr = nrows(j);
        TileQuadC<R> Fd, Fs;
        Fd.load_neg(Ab(j, j), p.lda, nr, nr, true);
        if (j > 0)
            Fs.load_neg(Ab(j, j - 1), p.lda, nr, LEAF, false);
        if (j > 0)
            pre(Fs, j, j - 1, nr, LEAF, false);
        pre(Fd, j, j, nr, nr, true);
        for (int l = 0; l + 1 < j; ++l) {
            wait(fL(j, l), fL(j - 1, l));
            const E *U = Ab(j, l), *V = Ab(j - 1, l);
            tile_mma_c<R>(
                Fs, [&](int r, int k, R &x, R &y) { gget(U, p.lda, nr, r, k, x, y); },
                [&](int k, int c, R &x, R &y) {
                    gget(V, p.lda, LEAF, c, k, x, y);
                    y = -y;
                },
                TK_FULL, false);
            tile_mma_c<R>(
                Fd, [&](int r, int k, R &x, R &y) { gget(U, p.lda, nr, r, k, x, y); },
                [&](int k, int c, R &x, R &y) {
                    gget(U, p.lda, nr, c, k, x, y);
                    y = -y;
                },
                TK_FULL, true);
        }
        if (j > 0) {
            // L_j,j-1 = (A_j,j-1 - ...) inv(L_j-1,j-1)^H
            wait(fL(j - 1, j - 1), nullptr);
            Fs.to_lds(S, R(-1), false);
            __syncthreads();
            const E *Xp = Xb(j - 1, j - 1);
            TileQuadC<R> G;
            G.zero();
            tile_mma_c<R>(G, sget,
                          [&](int k, int c, R &x, R &y) {
                              gget(Xp, p.ldi, LEAF, c, k, x, y);
                              y = -y;
                          },
                          TK_TO_COL, false);
            __syncthreads();
            G.store(Ab(j, j - 1), p.lda, nr, R(1));
            G.to_lds(S, R(1), false);
            __syncthreads();
            tile_mma_c<R>(Fd, sget,
                          [&](int k, int c, R &x, R &y) {
                              sget(c, k, x, y);
                              y = -y;
                          },
                          TK_FULL, true);
            __syncthreads();
        }
        Fd.to_lds(S, R(-1), true);
        if (tid == 0)
            failed = 0;
        // L_j,j-1 published now (see tile_kernel); the barrier serves the leaf
        if (j > 0)
            tile_signal(fL(j, j - 1));
        else
            __syncthreads();
        leafc_lds<R>(S, Xd, Tm, true, nr, p.col0 + j * LEAF, p.info, &failed);
        // inv(L_jj) first: the other roles wait for it, and none reads L_jj
        const int r = tid & 63, g = tid >> 6;
        {
            E *const Xdst = Xb(j, j);
#pragma unroll
            for (int k = 0; k < LEAF / 4; ++k) {
                const int c = g + 4 * k;
                if (r < nr && c < nr) {
                    R x, y;
                    leafc_xget<R>(S, Xd, r, c, x, y);
                    Elem<R, true>::store(Xdst + r + (int64_t)c * p.ldi, x, y);
                }
            }
        }
        tile_signal(fL(j, j));
        {
            E *const Ad = Ab(j, j);
#pragma unroll
            for (int k = 0; k < LEAF / 4; ++k) {
                const int c = g + 4 * k;
                if (r < nr && c < nr && r >= c)
                    Elem<R, true>::store(Ad + r + (int64_t)c * p.lda, S[0][c][r], r == c ? R(0) : S[1][c][r]);
            }
        }
    } else if (kind == TILE_O) {
        const int i = bi, j = bj, nr = nrows(i);
        TileQuadC<R> F;
        F.load_neg(Ab(i, j), p.lda, nr, LEAF, false);
        pre(F, i, j, nr, LEAF, false);
        for (int l = 0; l < j; ++l) {
            wait(fL(i, l), fL(j, l));
            const E *U = Ab(i, l), *V = Ab(j, l);
            tile_mma_c<R>(
                F, [&](int r, int k, R &x, R &y) { gget(U, p.lda, nr, r, k, x, y); },
                [&](int k, int c, R &x, R &y) {
                    gget(V, p.lda, LEAF, c, k, x, y);
                    y = -y;
                },
                TK_FULL, false);
        }
        wait(fL(j, j), nullptr);
        F.to_lds(S, R(-1), false);
        __syncthreads();
        const E *Xj = Xb(j, j);
        TileQuadC<R> G;
        G.zero();
        tile_mma_c<R>(G, sget,
                      [&](int k, int c, R &x, R &y) {
                          gget(Xj, p.ldi, LEAF, c, k, x, y);
                          y = -y;
                      },
                      TK_TO_COL, false);
        G.store(Ab(i, j), p.lda, nr, R(1));
        tile_signal(fL(i, j));
    } else if (kind == TILE_X) {
        const int i = bi, b = bj, nr = nrows(i);
        TileQuadC<R> G;
        G.zero();
        for (int k = b; k < i; ++k) {
            wait(fL(i, k), k == b ? fL(b, b) : fX(k, b));
            const E *U = Ab(i, k), *V = Xb(k, b);
            // G += L_ik inv(L)_kb
            tile_mma_c<R>(
                G, [&](int r, int kk, R &x, R &y) { gget(U, p.lda, nr, r, kk, x, y); },
                [&](int kk, int c, R &x, R &y) { gget(V + (int64_t)c * p.ldi, p.ldi, LEAF, kk, 0, x, y); },
                k == b ? TK_FROM_COL : TK_FULL, false);
        }
        wait(fL(i, i), nullptr);
        G.to_lds(S, R(1), false);
        __syncthreads();
        // H = inv(L_ii) G
        const E *Xi = Xb(i, i);
        TileQuadC<R> H;
        H.zero();
        tile_mma_c<R>(H,
                      [&](int r, int kk, R &x, R &y) {
                          // rows and columns past a short last block are zero
                          gget(Xi, p.ldi, kk < nr ? nr : 0, r, kk, x, y);
                      },
                      [&](int kk, int c, R &x, R &y) { sget(kk, c, x, y); }, TK_TO_ROW, false);
        H.store(Xb(i, b), p.ldi, nr, R(-1));
        tile_signal(fX(i, b));
    }

    __syncthreads();
    if (tid == 0)
        last = atomicAdd(ctr, 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (last) {
        for (int e = tid; e < (2 * nb * nb + 1) * TILE_FLAG_STRIDE; e += blockDim.x)
            p.flags[e] = 0;
        if (tid == 0)
            *ctr = 0;
    }
}

}  // namespace spd
