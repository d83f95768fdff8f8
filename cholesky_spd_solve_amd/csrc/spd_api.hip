// Host side of the gfx950 dense SPD/HPD solver: argument checking, workspace
// layout and the launch sequences of the blocked Cholesky factorization,
// blocked substitution and log-determinant (declared in include/spd.h).
//
// Right-looking blocked Cholesky with tile size T (JAXMg paper, "Software
// design": potrs = potrf + potrs with a user tile size T_A), for k = 0, 1, ...:
//   1. factor the diagonal tile  A_kk = L_kk L_kk^H  and form inv(L_kk)
//   2. panel solve               L_ik = A_ik L_kk^-H  (i > k), as A_ik inv(L_kk)^H
//   3. trailing update           A_ij -= L_ik L_jk^H  (k < j <= i, lower part)
// Step 1 is itself blocked by LEAF = 64 columns: each leaf is factored and
// inverted inside LDS by one workgroup, the rows below it inside the tile are
// solved against the leaf inverse and the rest of the tile is updated; the
// leaf inverses are then merged pairwise (inv([A 0; B C]) has lower-left
// block -inv(C) B inv(A)) until inv(L_kk) is complete.
//
// The solve L L^H X = B walks the same tiles: Y_k = inv(L_kk) (B_k - ...)
// forwards, then X_k = inv(L_kk)^H (Y_k - ...) backwards, with every
// inv(L_kk) built up front by the same leaf + merge kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>
#include <functional>

#include "spd.h"
#include "spd_gemm.hpp"
#include "spd_kernels.hpp"
#include "spd_rect.hpp"
#include "spd_syrk.hpp"
#include "spd_tile.hpp"
#include "spd_subst.hpp"
#include "spd_check.hpp"

namespace spd {

static thread_local std::string g_last_error;

static int hip_fail(hipError_t e, const char *where)
{
    g_last_error = std::string(where) + ": " + hipGetErrorString(e);
    return SPD_ERR_HIP;
}

// Launch validation (spd_debug_validate): 0 off, 1 replay each launch on the
// host before enqueueing it, 2 replay only (no GPU work, no HIP calls).
static int g_validate = 0;
static thread_local Checker g_chk;

static int check_fail()
{
    g_last_error = "launch validation: " + g_chk.err;
    return SPD_ERR_CHECK;
}

// Replays a launch on the host when validation is on; returns 0 to go on,
// -1 to skip the launch (dry run), or an error code.
#define SPD_VALIDATE(check_expr)             \
    do {                                     \
        if (g_validate) {                    \
            if (!(check_expr))               \
                return check_fail();         \
            if (g_validate == 2)             \
                return 0;                    \
        }                                    \
    } while (0)

#define SPD_CHECK_LAUNCH(where)                          \
    do {                                                 \
        hipError_t e_ = hipGetLastError();               \
        if (e_ != hipSuccess)                            \
            return hip_fail(e_, where);                  \
    } while (0)

// ------------------------------------------------------------ profiling ---

struct ProfRec {
    int cls;
    hipEvent_t a, b;
    double flops;
};
static std::mutex g_prof_mu;
static int g_prof_mask = 0;
static std::vector<ProfRec> g_prof;

struct ProfScope {
    bool on = false;
    ProfRec r{};
    hipStream_t s{};
    ProfScope(int cls, double flops, hipStream_t stream)
    {
        std::lock_guard<std::mutex> g(g_prof_mu);
        if (cls < 0 || !(g_prof_mask & (1 << cls)) || g_validate == 2)
            return;
        on = true;
        s = stream;
        r.cls = cls;
        r.flops = flops;
        (void)hipEventCreate(&r.a);
        (void)hipEventCreate(&r.b);
        (void)hipEventRecord(r.a, s);
    }
    ~ProfScope()
    {
        if (!on)
            return;
        (void)hipEventRecord(r.b, s);
        std::lock_guard<std::mutex> g(g_prof_mu);
        g_prof.push_back(r);
    }
};

enum { PROF_SYRK = 0, PROF_PANEL = 1, PROF_DIAG = 2, PROF_SOLVE = 3, PROF_UPDATE = 4, PROF_SYRK_AUX = 5 };

// ------------------------------------------------------------- helpers ----

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline int64_t align_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

enum Lay { NT, NN, TN };

struct Gemm {
    const void *A = nullptr, *B = nullptr;
    void *C = nullptr;
    int64_t lda = 1, ldb = 1, ldc = 1;
    int64_t sA_out = 0, sA_in = 0, sB_out = 0, sB_in = 0, sC_out = 0, sC_in = 0;
    int nb_inner = 1, batch = 1;
    int64_t m = 0, n = 0, k = 0;
    bool tri = false;
    int kmode = KM_NONE;
    bool neg = false;
    bool beta = false;
    const int *info = nullptr;
    bool small = false;    // prefer the small tile shape
};

template <typename R, bool CPLX, int BM, int BN, int KB, int WM, int WN, bool AT, bool BT>
static int launch_gemm_kernel(dim3 grid, dim3 block, const GemmArgs &a, hipStream_t s)
{
    SPD_VALIDATE((check_gemm<R, CPLX, BM, BN, KB, WM, WN, AT, BT>(a, grid, g_chk)));
    gemm_kernel<R, CPLX, BM, BN, KB, WM, WN, AT, BT><<<grid, block, 0, s>>>(a);
    SPD_CHECK_LAUNCH("gemm_kernel");
    return 0;
}

template <typename R, bool CPLX, int BM, int BN, int KB, int WM, int WN>
static int launch_gemm_cfg(Lay lay, const Gemm &g, hipStream_t s)
{
    GemmArgs a;
    a.A = g.A;
    a.B = g.B;
    a.C = g.C;
    a.lda = g.lda;
    a.ldb = g.ldb;
    a.ldc = g.ldc;
    a.sA_out = g.sA_out;
    a.sA_in = g.sA_in;
    a.sB_out = g.sB_out;
    a.sB_in = g.sB_in;
    a.sC_out = g.sC_out;
    a.sC_in = g.sC_in;
    a.nb_inner = g.nb_inner;
    a.m = (int)g.m;
    a.n = (int)g.n;
    a.k = (int)g.k;
    a.tiles_m = (int)cdiv(g.m, BM);
    a.tiles_n = (int)cdiv(g.n, BN);
    a.ntiles = g.tri ? a.tiles_m * (a.tiles_m + 1) / 2 : a.tiles_m * a.tiles_n;
    a.tri = g.tri ? 1 : 0;
    a.kmode = g.kmode;
    a.neg = g.neg ? 1 : 0;
    a.beta = g.beta ? 1 : 0;
    a.info = g.info;
    dim3 grid(a.ntiles, 1, g.batch), block(64 * WM * WN);
    switch (lay) {
    case NT: return launch_gemm_kernel<R, CPLX, BM, BN, KB, WM, WN, false, true>(grid, block, a, s);
    case NN: return launch_gemm_kernel<R, CPLX, BM, BN, KB, WM, WN, false, false>(grid, block, a, s);
    case TN: return launch_gemm_kernel<R, CPLX, BM, BN, KB, WM, WN, true, false>(grid, block, a, s);
    }
    return SPD_ERR_HIP;
}

template <typename R, bool CPLX>
static int gemm(Lay lay, const Gemm &g, hipStream_t s)
{
    if (g.m <= 0 || g.n <= 0 || g.batch <= 0)
        return 0;
    if (g.k <= 0 && g.beta)
        return 0;
    if constexpr (!CPLX) {
        // large products: 128x128 tiles; small ones: 64x64, or 32x32 when even
        // 64x64 tiles would leave most CUs idle (latency-bound chains)
        const int64_t tiles128 = g.tri ? cdiv(g.m, 128) * (cdiv(g.m, 128) + 1) / 2
                                       : cdiv(g.m, 128) * cdiv(g.n, 128);
        const int64_t tiles64 = g.tri ? cdiv(g.m, 64) * (cdiv(g.m, 64) + 1) / 2 : cdiv(g.m, 64) * cdiv(g.n, 64);
        if (!g.small && tiles128 * g.batch >= 512)
            return launch_gemm_cfg<R, CPLX, 128, 128, 16, 2, 2>(lay, g, s);
        if (tiles64 * g.batch >= 128)
            return launch_gemm_cfg<R, CPLX, 64, 64, 16, 2, 2>(lay, g, s);
        return launch_gemm_cfg<R, CPLX, 32, 32, 16, 2, 2>(lay, g, s);
    } else {
        const int64_t tiles64 = g.tri ? cdiv(g.m, 64) * (cdiv(g.m, 64) + 1) / 2 : cdiv(g.m, 64) * cdiv(g.n, 64);
        if (!g.small && tiles64 * g.batch >= 512)
            return launch_gemm_cfg<R, CPLX, 64, 64, 16, 2, 2>(lay, g, s);
        return launch_gemm_cfg<R, CPLX, 32, 32, 16, 2, 2>(lay, g, s);
    }
}

template <typename E>
static int copy2d(E *dst, int64_t ldd, const E *src, int64_t lds, int64_t m, int64_t n, const int *info,
                  hipStream_t s)
{
    if (m <= 0 || n <= 0)
        return 0;
    SPD_VALIDATE(check_2d<E>("copy2d_kernel", dst, ldd, src, lds, m, n, info, g_chk));
    const int64_t blocks = std::min<int64_t>(cdiv(m * n, 256), 4096);
    copy2d_kernel<E><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(dst, ldd, src, lds, m, n, info);
    SPD_CHECK_LAUNCH("copy2d_kernel");
    return 0;
}

template <typename E>
static int zero2d(E *dst, int64_t ldd, int64_t m, int64_t n, hipStream_t s)
{
    if (m <= 0 || n <= 0)
        return 0;
    SPD_VALIDATE(check_2d<E>("zero2d_kernel", dst, ldd, (const E *)nullptr, 0, m, n, nullptr, g_chk));
    const int64_t blocks = std::min<int64_t>(cdiv(m * n, 256), 8192);
    zero2d_kernel<E><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(dst, ldd, m, n);
    SPD_CHECK_LAUNCH("zero2d_kernel");
    return 0;
}

static int set_info(int *info, hipStream_t s)
{
    SPD_VALIDATE(g_chk.access(info, 4, true, "set_int_kernel", 0, 0));
    set_int_kernel<<<1, 1, 0, s>>>(info, 0);
    SPD_CHECK_LAUNCH("set_int_kernel");
    return 0;
}

#define SPD_TRY_HIP(x, where)            \
    do {                                  \
        hipError_t e_ = (x);              \
        if (e_ != hipSuccess)             \
            return hip_fail(e_, where);   \
    } while (0)

#define SPD_TRY(x)              \
    do {                        \
        int r_ = (x);           \
        if (r_ != 0)            \
            return r_;          \
    } while (0)

// Workspace layout, in elements of the working type (each region 256-byte
// aligned):  INV  nt * T * T   inverted diagonal tiles (tile t at t*T*T, ld T)
//            W    npanels (4, or 6 from TRIPLE_MIN_TILES tiles on) x (n rounded
//                 up to 128) x (T rounded up to 32): the panels L21 of as many
//                 consecutive steps (potrf) / merge temporaries (both)
//            TMP  max(T*T, T*n_rhs)   one block row of the right-hand side
struct Layout {
    int64_t T, nt, inv, w, wsz, npanels, tmp, ctr, flags, q, ldq, kq, qsz, gf, gb, part, z, ldz, sflags,
        total;  // offsets / sizes in elements
};

// Right-hand-side columns of a piece of the one-launch back substitution
static int64_t subst_tc(int64_t n_rhs) { return n_rhs <= 32 ? 32 : 64; }

// The trailing-update panel W is stored with its leading dimension rounded up
// to SYRK_LDW rows and its width to SYRK_KP columns, the padding zeroed, so the
// trailing-update kernel reads whole tiles and slices only.
constexpr int64_t SYRK_LDW = 128;  // multiple of every trailing-update tile size
constexpr int64_t SYRK_KP = 32;    // multiple of every trailing-update slice depth
// The substitutions' block update reads the solved block transposed from a
// buffer with RECT_LDQ-aligned rows and RECT_KB-aligned columns, zero padded.
constexpr int64_t RECT_LDQ = 128;  // multiple of every block-update tile width
constexpr int64_t RECT_KB = 32;    // multiple of every block-update slice depth
// The chain product of the substitutions is split into this many partial
// products (two operand pairs, each split along its depth).
constexpr int64_t CHAIN_SPLITS = 8;

// Orders of at least this many tiles keep six trailing-update panel buffers
// (three steps in use, three being built) instead of four.
constexpr int64_t TRIPLE_MIN_TILES = 40;

// The one-launch diagonal tile's flags start 256 bytes after the leaf + panel
// counter (Layout::flags)
static int *tile_flags(int *ctr) { return ctr + 256 / sizeof(int); }

static Layout make_layout(int64_t n, int64_t n_rhs, int64_t T_A, int64_t esize)
{
    Layout L;
    L.T = std::max<int64_t>(1, std::min(T_A, n));
    L.nt = cdiv(n, L.T);
    const int64_t al = 256 / esize;
    L.inv = 0;
    L.w = align_up(L.nt * L.T * L.T, al);
    L.wsz = align_up(align_up(n, SYRK_LDW) * align_up(L.T, SYRK_KP), al);
    // panel buffers: the steps in use and those being built (two and two, or
    // three and three for large orders)
    L.npanels = L.nt >= TRIPLE_MIN_TILES ? 6 : 4;
    L.tmp = L.w + L.npanels * L.wsz;
    // ctr: the fused leaf + panel launch's workgroup counter (one int);
    // flags: the one-launch diagonal tile's block flags and counter
    L.ctr = L.tmp + align_up(std::max(L.T * L.T, L.T * std::max<int64_t>(n_rhs, 1)), al);
    L.flags = L.ctr + al;
    L.q = L.flags + align_up(cdiv(4 * (int64_t)tile_flag_ints((int)cdiv(L.T, LEAF)), esize), al);
    L.ldq = align_up(n_rhs, RECT_LDQ);
    L.kq = align_up(L.T, RECT_KB);
    L.qsz = L.ldq * L.kq;  // two buffers, adjacent
    if (n_rhs > 0) {
        // the substitutions' chain products: -inv(L_k+1,k+1) L_k+1,k and
        // -L_k,k-1 inv(L_k-1,k-1) per block, and the partial sums of the
        // split products
        L.gf = L.q + align_up(2 * L.qsz, al);
        L.gb = L.gf + align_up(L.nt * L.T * L.T, al);
        L.part = L.gb + align_up(L.nt * L.T * L.T, al);
        // the one-launch back substitution's two buffers of one tile row (T x
        // n_rhs each, leading dimension T, adjacent) and its flags
        const int64_t tc = subst_tc(n_rhs);
        L.ldz = L.T;
        L.z = L.part + align_up(CHAIN_SPLITS * L.T * n_rhs, al);
        L.sflags = L.z + align_up(2 * L.T * n_rhs, al);
        const int64_t nfl = subst_flag_ints((int)L.nt, (int)cdiv(n_rhs, tc));
        L.total = L.sflags + align_up(cdiv(4 * nfl, esize), al);
    } else {
        L.gf = L.gb = L.part = L.z = L.sflags = L.q;
        L.ldz = 0;
        L.total = L.q;
    }
    return L;
}

// Workspace of the generalized-eigenproblem reduction, in elements (each
// region 256-byte aligned).  M (n x n, ld n) holds the full Hermitian A and
// then the result.
//   itype 1: the substitution workspace for n right-hand sides (its INV and W
//            regions also serve the blocked sweep), two sets of the rank-2k
//            operand panels P and Q (n rounded up to 128 rows, 2 x (T rounded
//            up to 32) columns; one step ahead), Y and V (n x T, ld n), and two
//            T x T tiles;
//   itypes 2, 3: two square matrices of order n rounded up to 128 (L^H, and
//            the stacked row panels w_k), two operand panels P and Q as for
//            itype 1, the lower triangles of L's diagonal blocks and their
//            products (nt T x T tiles each), and two T x n blocks.
struct GstLayout {
    int64_t T, nt, m, solve, p, q, p2, q2, y, v, d, t1, lh, wf, ld, ldg, total;
};

static GstLayout make_gst_layout(int itype, int64_t n, int64_t T_A, int64_t esize)
{
    GstLayout G{};
    const int64_t al = 256 / esize;
    G.T = std::max<int64_t>(1, std::min(T_A, n));
    G.nt = cdiv(n, G.T);
    G.m = 0;
    int64_t o = align_up(n * n, al);
    if (itype == 1) {
        const int64_t pw = align_up(n, SYRK_LDW) * 2 * align_up(G.T, SYRK_KP);
        G.solve = o;
        o += align_up(make_layout(n, n, T_A, esize).total, al);
        G.p = o;
        o += align_up(pw, al);
        G.q = o;
        o += align_up(pw, al);
        G.p2 = o;
        o += align_up(pw, al);
        G.q2 = o;
        o += align_up(pw, al);
        G.y = o;
        o += align_up(n * G.T, al);
        G.v = o;
        o += align_up(n * G.T, al);
        G.d = o;
        o += align_up(G.T * G.T, al);
        G.t1 = o;
        o += align_up(G.T * G.T, al);
    } else {
        G.ldg = align_up(n, SYRK_LDW);
        const int64_t sq = align_up(G.ldg * G.ldg, al);
        const int64_t pw = G.ldg * 2 * align_up(G.T, SYRK_KP);
        G.p = o;
        o += align_up(pw, al);
        G.q = o;
        o += align_up(pw, al);
        G.lh = o;
        o += sq;
        G.wf = o;
        o += sq;
        G.ld = o;
        o += align_up(G.nt * G.T * G.T, al);
        G.t1 = o;
        o += align_up(G.nt * G.T * G.T, al);
        G.v = o;
        o += align_up(G.T * n, al);
        G.y = o;  // X blocks
        o += align_up(G.T * n, al);
    }
    G.total = o;
    return G;
}

// Schedule and tile-shape options (spd_set_option).  They are process-wide
// atomics; every entry point copies them into g_opt when it is called, so one
// call sees one consistent set whatever other threads change meanwhile.  They
// select among schedules and tile shapes that compute the same factorization
// and solve; results agree with each other within rounding.
enum {
    OPT_LOOKAHEAD,
    OPT_TWO_STEP,
    OPT_PAIR_ROWS,
    OPT_SYRK_DEEP_ROWS,
    OPT_RECT_TALL_ROWS,
    OPT_TILE_LAUNCH,
    OPT_TILE_WAIT_US,
    OPT_COLUMN_FIRST_ROWS,
    OPT_TILE_HOLD_ROWS,
    OPT_SUBST_LAUNCH,
    OPT_TILE_UPDATE_ROWS,
    OPT_TRIPLE_ROWS,
    OPT_COUNT
};
static const int64_t k_opt_default[OPT_COUNT] = {1, 1, -1, -1, 16384, 1, 2000000, 8192, 8192, 2097152, -1, -1};
static std::atomic<int64_t> g_opt_store[OPT_COUNT] = {{1},       {1},    {-1},   {-1},      {16384}, {1},
                                                      {2000000}, {8192}, {8192}, {2097152}, {-1},    {-1}};
struct Options {
    int64_t v[OPT_COUNT];
};
static thread_local Options g_opt = {{1, 1, -1, -1, 16384, 1, 2000000, 8192, 8192, 2097152, -1, -1}};

static void snapshot_options()
{
    for (int i = 0; i < OPT_COUNT; ++i)
        g_opt.v[i] = g_opt_store[i].load(std::memory_order_relaxed);
}

// The multi-step schedule of potrf (trailing updates of depth 2T or 3T, see
// potrf_pairs) is used unless SPD_OPT_TWO_STEP is 0; it pairs steps while at
// least two_step_rows(T) rows remain beyond the pair (SPD_OPT_PAIR_ROWS; by
// default 32 T: below that the auxiliary stream's two-tile chain, sharing the
// GPU with the caller's update, outlasts it).
static bool two_step_enabled() { return g_opt.v[OPT_TWO_STEP] != 0; }

static int64_t two_step_rows(int64_t T)
{
    const int64_t v = g_opt.v[OPT_PAIR_ROWS];
    return v >= 0 ? v : 32 * T;
}

// Orders of at least TRIPLE_MIN_TILES tiles keep six panel buffers instead of
// four, and there the schedule takes steps in threes (trailing updates of
// depth 3T) while at least three_step_rows(T) rows remain beyond the three
// (SPD_OPT_TRIPLE_ROWS; 0: never).
static int64_t three_step_rows(int64_t T)
{
    const int64_t v = g_opt.v[OPT_TRIPLE_ROWS];
    return v >= 0 ? v : 32 * T;
}

// The lookahead schedule is on unless SPD_OPT_LOOKAHEAD is 0 (the sequential
// schedule does the same work without overlap; it is there to measure each
// kernel on its own).
static bool lookahead_enabled() { return g_opt.v[OPT_LOOKAHEAD] != 0; }

// Trailing-update orders from which 128-row tiles take the deeper slices
// (fp64: 16 instead of 8, by default never since the early updates are taken
// at depth 3T; fp32: 32 instead of 16).
static int64_t syrk_deep_rows(int64_t esize)
{
    const int64_t v = g_opt.v[OPT_SYRK_DEEP_ROWS];
    return v >= 0 ? v : (esize == 8 ? INT64_MAX : 8192);
}

// Block-update heights from which the substitutions (and the factorization's
// panel product) take 64-row tiles.
static int64_t rect_tall_rows() { return g_opt.v[OPT_RECT_TALL_ROWS]; }

// Each diagonal tile of the factorization is factored and inverted in one
// launch (tile_kernel, tile_kernel_c) unless SPD_OPT_TILE_LAUNCH is 0 (then by the leaf,
// in-tile update and inverse-merge launches); SPD_OPT_TILE_WAIT_US bounds each
// of that kernel's waits for another workgroup's block.
static bool tile_launch_enabled() { return g_opt.v[OPT_TILE_LAUNCH] != 0; }
static int64_t tile_wait_ticks() { return g_opt.v[OPT_TILE_WAIT_US] * 100; }  // 100 MHz wall clock

// Lookahead steps taken one at a time: while fewer than column_first_rows()
// rows remain beyond the next tile (SPD_OPT_COLUMN_FIRST_ROWS), the caller's
// trailing update waits until the auxiliary stream has updated the next tile
// column.  There the diagonal-tile chain outlasts the caller's update; left to
// run beside that update, the column update shares every CU with it and
// delays the tile that waits for it.
static int64_t column_first_rows() { return g_opt.v[OPT_COLUMN_FIRST_ROWS]; }

// A real diagonal tile with fewer than tile_hold_rows() rows below it
// (SPD_OPT_TILE_HOLD_ROWS) is launched so that each workgroup has a CU to
// itself: idle waves hold registers (see tile_kernel) and the launch asks for
// the CU's whole LDS.  There the chain is the longer path, and the tile's
// leaves sharing SIMDs with the trailing update run two to three times slower.
static int64_t tile_hold_rows() { return g_opt.v[OPT_TILE_HOLD_ROWS]; }

// In the steps taken one at a time (two-step schedule), while fewer than
// tile_update_rows() rows remain beyond the next tile
// (SPD_OPT_TILE_UPDATE_ROWS), the next diagonal tile takes its last trailing
// update inside its own launch (one-launch tile only) and the caller's update
// covers the rest of its tile column; the panel product waits for that.  It
// pays only while that update is short next to the tile: by default 2048 rows
// for real types and never for complex ones (measured: fp64 N = 4096 2.79 ->
// 2.73 ms, fp32 N = 16384 within 0.2 %, complex128 N = 8192 1 % slower).
static int64_t tile_update_rows(bool cplx)
{
    const int64_t v = g_opt.v[OPT_TILE_UPDATE_ROWS];
    return v >= 0 ? v : (cplx ? 0 : 2048);
}

// The back substitution runs in one launch (subst_kernel) while n n_rhs
// (four times that for complex types) is at most SPD_OPT_SUBST_LAUNCH, else
// (and always when it is 0) by block steps on the stream and one auxiliary
// stream.  The one launch removes the block steps' launch and event latency,
// which is what bounds small and medium solves; at n = 32768, n_rhs = 128 its
// block products (a 32-row piece at a time, one chunk of loads in flight)
// are slower than the block steps' large updates.  Its waits are bounded by
// SPD_OPT_TILE_WAIT_US.
static bool subst_launch_enabled(int64_t n, int64_t nrhs, bool cplx)
{
    return (double)n * (double)nrhs * (cplx ? 4.0 : 1.0) <= (double)g_opt.v[OPT_SUBST_LAUNCH];
}

// The auxiliary streams and events of the lookahead schedules: one set per
// host thread and device, created on first use and kept until spd_release is
// called on that thread (or the process ends).  Default priority, non-blocking
// with respect to the null stream.  In a dry run (no HIP calls) every schedule
// runs on the caller's stream.
struct AuxStreams {
    hipStream_t look = nullptr, look2 = nullptr;
    hipEvent_t ev_fork = nullptr, ev_panel = nullptr, ev_rest = nullptr, ev_fw = nullptr, ev_col = nullptr;
};
static thread_local std::vector<std::pair<int, AuxStreams>> g_aux;

// Wait for and destroy the calling thread's auxiliary streams and events.
static int release_aux()
{
    int rc = 0;
    for (auto &pd : g_aux) {
        AuxStreams &x = pd.second;
        for (hipStream_t st : {x.look, x.look2}) {
            if (st == nullptr)
                continue;
            hipError_t e = hipStreamSynchronize(st);
            if (e == hipSuccess)
                e = hipStreamDestroy(st);
            if (e != hipSuccess && rc == 0)
                rc = hip_fail(e, "spd_release");
        }
        for (hipEvent_t ev : {x.ev_fork, x.ev_panel, x.ev_rest, x.ev_fw, x.ev_col}) {
            if (ev == nullptr)
                continue;
            hipError_t e = hipEventDestroy(ev);
            if (e != hipSuccess && rc == 0)
                rc = hip_fail(e, "spd_release");
        }
    }
    g_aux.clear();
    return rc;
}

struct Lookahead {
    hipStream_t look = nullptr, look2 = nullptr;  // look2: the fused solve's forward substitution
    hipEvent_t ev_fork = nullptr, ev_panel = nullptr, ev_rest = nullptr, ev_fw = nullptr, ev_col = nullptr;

    int begin(hipStream_t s)
    {
        if (g_validate == 2) {
            look = look2 = s;
            return 0;
        }
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return hip_fail(e, "hipGetDevice");
        AuxStreams *x = nullptr;
        for (auto &pd : g_aux)
            if (pd.first == dev)
                x = &pd.second;
        if (x == nullptr) {
            AuxStreams n;
            auto undo = [&n] {
                for (hipStream_t st : {n.look, n.look2})
                    if (st != nullptr)
                        (void)hipStreamDestroy(st);
                for (hipEvent_t ev : {n.ev_fork, n.ev_panel, n.ev_rest, n.ev_fw, n.ev_col})
                    if (ev != nullptr)
                        (void)hipEventDestroy(ev);
            };
            if ((e = hipStreamCreateWithFlags(&n.look, hipStreamNonBlocking)) != hipSuccess ||
                (e = hipStreamCreateWithFlags(&n.look2, hipStreamNonBlocking)) != hipSuccess) {
                undo();
                return hip_fail(e, "hipStreamCreateWithFlags");
            }
            for (hipEvent_t *ev : {&n.ev_fork, &n.ev_panel, &n.ev_rest, &n.ev_fw, &n.ev_col})
                if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) {
                    undo();
                    return hip_fail(e, "hipEventCreateWithFlags");
                }
            g_aux.emplace_back(dev, n);
            x = &g_aux.back().second;
        }
        look = x->look;
        look2 = x->look2;
        ev_fork = x->ev_fork;
        ev_panel = x->ev_panel;
        ev_rest = x->ev_rest;
        ev_fw = x->ev_fw;
        ev_col = x->ev_col;
        // the auxiliary streams start after everything already queued on s
        SPD_TRY_HIP(hipEventRecord(ev_fork, s), "hipEventRecord");
        SPD_TRY_HIP(hipStreamWaitEvent(look, ev_fork, 0), "hipStreamWaitEvent");
        SPD_TRY_HIP(hipStreamWaitEvent(look2, ev_fork, 0), "hipStreamWaitEvent");
        return 0;
    }
    int record(hipEvent_t ev, hipStream_t st)
    {
        if (g_validate == 2)
            return 0;
        SPD_TRY_HIP(hipEventRecord(ev, st), "hipEventRecord");
        return 0;
    }
    int wait(hipStream_t st, hipEvent_t ev)
    {
        if (g_validate == 2)
            return 0;
        SPD_TRY_HIP(hipStreamWaitEvent(st, ev, 0), "hipStreamWaitEvent");
        return 0;
    }
};

template <typename R, bool CPLX>
struct Solver {
    typedef typename Elem<R, CPLX>::type E;
    static constexpr double FMUL = CPLX ? 4.0 : 1.0;  // real flops per real-type flop

    static int leaves(E *A, int64_t lda, int64_t n, int64_t T, E *Inv, int64_t ldi, int64_t sInv,
                      int64_t ntiles, bool factor, int *info, int64_t col0, hipStream_t s)
    {
        LeafArgs p;
        p.A = A;
        p.lda = lda;
        p.Inv = Inv;
        p.ldi = ldi;
        p.sInv = sInv;
        p.n = (int)n;
        p.T = (int)T;
        p.lpt = (int)cdiv(T, LEAF);
        p.factor = factor ? 1 : 0;
        p.info = info;
        p.col0 = (int)col0;
        const int64_t grid = ntiles * p.lpt;
        if (grid <= 0)
            return 0;
        p.prows = 0;
        p.ctr = nullptr;
        SPD_VALIDATE((check_leaf<R, CPLX>(p, (unsigned)grid, g_chk)));
        if constexpr (CPLX)
            leaf16c_kernel<R><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
        else
            leaf16_kernel<R><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
        SPD_CHECK_LAUNCH("leaf16_kernel");
        return 0;
    }

    // Factor and invert the lb x lb leaf at D and solve the prows rows below
    // it, P <- P inv(L_leaf)^H in place, in one launch (ctr: the workgroup
    // counter, 0 between launches).
    static int leaf_panel(E *D, int64_t lda, int64_t lb, int64_t prows, E *Inv, int64_t ldi, int *info, int *ctr,
                          int64_t col0, hipStream_t s)
    {
        LeafArgs p;
        p.A = D;
        p.lda = lda;
        p.Inv = Inv;
        p.ldi = ldi;
        p.sInv = 0;
        p.n = (int)lb;
        p.T = (int)lb;
        p.lpt = 1;
        p.factor = 1;
        p.info = info;
        p.col0 = (int)col0;
        p.prows = (int)prows;
        p.ctr = ctr;
        const int64_t grid = 1 + cdiv(prows, LEAF);
        SPD_VALIDATE((check_leaf<R, CPLX>(p, (unsigned)grid, g_chk, true)));
        if constexpr (CPLX)
            leaf16c_kernel<R, true><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
        else
            leaf16_kernel<R, true><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
        SPD_CHECK_LAUNCH("leaf16_kernel (leaf + panel)");
        return 0;
    }

    // Complete inv(L_tt) from its inverted leaves for `ntiles` tiles of size tk
    // whose diagonal blocks start at D (stride sD between tiles, leading
    // dimension lda) and whose inverses start at Inv (stride sInv, ld ldi).
    // Level h merges blocks [2ph, (2p+1)h) and [(2p+1)h, (2p+2)h):
    //   X21 = -inv(C) (L21 inv(A)).   Tmp holds the L21 inv(A) products.
    static int merge_inverses(const E *D, int64_t lda, int64_t sD, E *Inv, int64_t ldi, int64_t sInv,
                              int64_t ntiles, int64_t tk, E *Tmp, const int *info, hipStream_t s)
    {
        for (int64_t h = LEAF; h < tk; h *= 2) {
            const int64_t nblk = cdiv(tk, h), pairs = nblk / 2;
            if (pairs == 0)
                break;
            const bool ragged = (2 * pairs * h) > tk;
            const int64_t pf = pairs - (ragged ? 1 : 0);
            if (pf > 0) {
                Gemm g1;  // T1 = L21 inv(A)      (h x h) * (h x h)
                g1.A = D + h;
                g1.lda = lda;
                g1.sA_out = sD;
                g1.sA_in = 2 * h * (1 + lda);
                g1.B = Inv;
                g1.ldb = ldi;
                g1.sB_out = sInv;
                g1.sB_in = 2 * h * (1 + ldi);
                g1.C = Tmp;
                g1.ldc = h;
                g1.sC_out = pf * h * h;
                g1.sC_in = h * h;
                g1.nb_inner = (int)pf;
                g1.batch = (int)(pf * ntiles);
                g1.m = h;
                g1.n = h;
                g1.k = h;
                g1.kmode = KM_BEG_BY_J;
                g1.info = info;
                SPD_TRY((gemm<R, CPLX>(NN, g1, s)));
                Gemm g2;  // X21 = -inv(C) T1
                g2.A = Inv + h * (1 + ldi);
                g2.lda = ldi;
                g2.sA_out = sInv;
                g2.sA_in = 2 * h * (1 + ldi);
                g2.B = Tmp;
                g2.ldb = h;
                g2.sB_out = pf * h * h;
                g2.sB_in = h * h;
                g2.C = Inv + h;
                g2.ldc = ldi;
                g2.sC_out = sInv;
                g2.sC_in = 2 * h * (1 + ldi);
                g2.nb_inner = (int)pf;
                g2.batch = (int)(pf * ntiles);
                g2.m = h;
                g2.n = h;
                g2.k = h;
                g2.kmode = KM_END_BY_I;
                g2.neg = true;
                g2.info = info;
                SPD_TRY((gemm<R, CPLX>(NN, g2, s)));
            }
            if (ragged) {
                const int64_t p = pairs - 1, a0 = 2 * p * h, c0 = a0 + h, hc = tk - c0;
                Gemm g1;
                g1.A = D + c0 + a0 * lda;
                g1.lda = lda;
                g1.sA_out = sD;
                g1.B = Inv + a0 * (1 + ldi);
                g1.ldb = ldi;
                g1.sB_out = sInv;
                g1.C = Tmp;
                g1.ldc = hc;
                g1.sC_out = hc * h;
                g1.batch = (int)ntiles;
                g1.m = hc;
                g1.n = h;
                g1.k = h;
                g1.kmode = KM_BEG_BY_J;
                g1.info = info;
                SPD_TRY((gemm<R, CPLX>(NN, g1, s)));
                Gemm g2;
                g2.A = Inv + c0 * (1 + ldi);
                g2.lda = ldi;
                g2.sA_out = sInv;
                g2.B = Tmp;
                g2.ldb = hc;
                g2.sB_out = hc * h;
                g2.C = Inv + c0 + a0 * ldi;
                g2.ldc = ldi;
                g2.sC_out = sInv;
                g2.batch = (int)ntiles;
                g2.m = hc;
                g2.n = h;
                g2.k = hc;
                g2.kmode = KM_END_BY_I;
                g2.neg = true;
                g2.info = info;
                SPD_TRY((gemm<R, CPLX>(NN, g2, s)));
            }
        }
        return 0;
    }

    // Factor the tk x tk diagonal tile at D and write inv(L_kk) to Inv (ld
    // ldi) in one launch (tile_kernel, tile_kernel_c)
    static int tile_launch(E *D, int64_t lda, int64_t tk, E *Inv, int64_t ldi, int *info, int *flags, int64_t col0,
                           int64_t rows_below, hipStream_t s, const E *W = nullptr, int64_t ldw = 0, int64_t wk = 0)
    {
        {
            TileArgs p;
            p.W = W;
            p.ldw = ldw;
            p.wk = W != nullptr ? (int)wk : 0;
            p.D = D;
            p.lda = lda;
            p.Inv = Inv;
            p.ldi = ldi;
            p.tk = (int)tk;
            p.nb = (int)cdiv(tk, LEAF);
            p.flags = flags;
            p.info = info;
            p.col0 = (int)col0;
            p.limit = tile_wait_ticks();
            p.hold = (!CPLX && rows_below < tile_hold_rows()) ? 1 : 0;
            const unsigned grid = (unsigned)tile_groups(p.nb);
            SPD_VALIDATE((check_tile<R, CPLX>(p, grid, g_chk)));
            if constexpr (CPLX) {
                tile_kernel_c<R><<<dim3(grid), dim3(256), 0, s>>>(p);
            } else {
                // holding: the idle waves take the registers, and group memory
                // up to the CU's whole LDS (not used) keeps every other
                // workgroup off the CU
                size_t dyn = 0;
                if (p.hold) {
                    int dev = 0, lds = 0;
                    hipFuncAttributes fa;
                    SPD_TRY_HIP(hipGetDevice(&dev), "hipGetDevice");
                    SPD_TRY_HIP(hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev),
                                "hipDeviceGetAttribute");
                    SPD_TRY_HIP(hipFuncGetAttributes(&fa, (const void *)tile_kernel<R>), "hipFuncGetAttributes");
                    if ((size_t)lds > fa.sharedSizeBytes) {
                        dyn = (size_t)lds - fa.sharedSizeBytes;
                        SPD_TRY_HIP(hipFuncSetAttribute((const void *)tile_kernel<R>,
                                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn),
                                    "hipFuncSetAttribute");
                    }
                }
                tile_kernel<R><<<dim3(grid), dim3(p.hold ? 512 : 256), dyn, s>>>(p);
            }
            SPD_CHECK_LAUNCH("tile_kernel");
            return 0;
        }
    }

    static constexpr int64_t syrk_bm() { return CPLX ? 64 : 128; }

    // Lower triangle of C (m x m, ldc) -= W W^H with W as laid out above; with
    // jt_end > 0 only the first jt_end tile columns (jt_end * BM columns of C).
    // Extra operands of the rank-2k form: the column operand V (nullptr: W) and
    // the depth range and sign (see SyrkArgs).
    struct Syr2 {
        const E *V = nullptr;
        int krange = SYRK_K_ALL;
        bool add = false;
        int64_t ncols = 0;  // > 0: the whole m x ncols rectangle (rect_update)
        const E *W2 = nullptr;  // second operand for depth [kp1, kp) (a group of panels that
                                // wraps from the last panel buffer to the first)
        int64_t kp1 = 0;
        bool aux = false;  // potrf's auxiliary stream (timed as its own class)
        int64_t skip = 0;  // the lower triangle without its leading skip x skip block
                           // (a multiple of the tile order)
    };

    template <int BM, int KB, int WM, int WN, bool BIGLD = false, bool PK = false>
    static int syrk_cfg(int64_t m, const E *W, int64_t ldw, int64_t kp, E *C, int64_t ldc, int jt_end,
                        const int *info, hipStream_t s, const Syr2 &x = Syr2())
    {
        static_assert(SYRK_LDW % BM == 0 && SYRK_KP % KB == 0, "panel padding too small for the tile");
        SyrkArgs a;
        a.W = W;
        a.V = x.V != nullptr ? x.V : W;
        a.W2 = x.W2;
        a.V2 = x.W2;  // the symmetric form only
        a.kp1 = (int)x.kp1;
        a.krange = x.krange;
        a.add = x.add ? 1 : 0;
        a.ldw = ldw;
        a.C = C;
        a.ldc = ldc;
        a.m = (int)m;
        a.kp = (int)kp;
        a.tiles = (int)cdiv(m, BM);
        a.jt_end = (jt_end > 0 && jt_end < a.tiles) ? jt_end : 0;
        a.ncols = (int)x.ncols;
        if (a.ncols > 0) {
            a.ntiles = a.tiles * (int)cdiv(x.ncols, BM);
        } else if (a.jt_end > 0) {
            a.ntiles = 0;
            for (int J = 0; J < a.jt_end; ++J)
                a.ntiles += a.tiles - J;
        } else {
            a.ntiles = a.tiles * (a.tiles + 1) / 2;
        }
        a.tskip = 0;
        if (x.skip >= m)
            return 0;  // all of C is the block left to the next tile
        if (x.skip > 0) {
            const int sk = (int)(x.skip / BM);
            if (a.ncols > 0 || a.jt_end > 0 || (int64_t)sk * BM != x.skip) {
                g_last_error = "trailing update: the skipped block must be whole lower-triangle tiles";
                return SPD_ERR_HIP;
            }
            a.tskip = sk * (sk + 1) / 2;
            a.ntiles -= a.tskip;
            if (a.ntiles <= 0)
                return 0;
        }
        a.info = info;
        a.vecc = ((uintptr_t)C % 16 == 0 && (ldc * (int64_t)sizeof(E)) % 16 == 0) ? 1 : 0;
        const dim3 grid((unsigned)a.ntiles), block(64 * WM * WN);
        SPD_VALIDATE((check_syrk<R, CPLX, BM, KB, WM, WN, BIGLD, PK>(a, grid, g_chk)));
        syrk_kernel<R, CPLX, BM, KB, WM, WN, BIGLD, PK><<<grid, block, 0, s>>>(a);
        SPD_CHECK_LAUNCH("syrk_kernel");
        return 0;
    }

    // kw: the panel's true width (kp is it rounded up), for the flop count;
    // cols > 0: only the first cols columns of C (a multiple of 128)
    static Syr2 aux_update()
    {
        Syr2 x;
        x.aux = true;
        return x;
    }

    // x: the rank-2k form (timed by its caller, not as the trailing update)
    static int syrk(int64_t m, const E *W, int64_t ldw, int64_t kp, int64_t kw, E *C, int64_t ldc, int64_t cols,
                    const int *info, hipStream_t s, const Syr2 &x = Syr2())
    {
        if (m <= 0 || x.skip >= m)
            return 0;  // nothing to update (no launch, nothing timed)
        const int64_t w = cols > 0 ? std::min<int64_t>(m, cols) : m;  // columns of C updated
        if (x.W2 != nullptr && x.V != nullptr) {
            g_last_error = "two-panel update is for the symmetric form";
            return SPD_ERR_HIP;
        }
        const double sk = (double)std::min(x.skip, m);  // the leading block left to the next tile
        ProfScope ps(x.V != nullptr ? -1 : x.aux ? PROF_SYRK_AUX : PROF_SYRK,
                     FMUL * ((double)w * (2.0 * m - w + 1.0) - sk * (sk + 1.0)) * (double)kw, s);
        auto jt = [&](int64_t bm) { return cols > 0 ? (int)(cols / bm) : 0; };
        if (ldc >= SYRK_LD32)  // 64-bit offsets into C; one 64-row tile shape for every such case
            return syrk_cfg<64, 16, 2, 2, true>(m, W, ldw, kp, C, ldc, jt(64), info, s, x);
        if constexpr (CPLX) {
            // 8 waves on 64 x 64 complex tiles: 3-6 % above 4 waves (c128, T = 256)
            return syrk_cfg<64, 16, 2, 4>(m, W, ldw, kp, C, ldc, jt(64), info, s, x);
        } else {
            // Launches with fewer 128-row tiles than two per CU take 64-row
            // tiles: one 128 x 128 x T tile is a fixed ~55 us of a CU's
            // matrix-core time, so a small update finishes sooner on four times
            // as many workgroups with a quarter of the work each.
            // Packed rows (two or four adjacent rows per lane, 16-byte LDS
            // operand reads and C vectors; the same bits) where they measured
            // faster alone: fp64 64-row tiles 3-4.5 % (m = 2048-4096, depth
            // 512), fp32 32-deep 128-row tiles 1-2 % at depth 512; fp64
            // 128-row tiles within 1 %, fp32 16-deep and 64-row tiles 3-5 %
            // slower, so those keep the plain layout.
            const int64_t t128 = cdiv(m, 128);
            const int64_t n128 = cols > 0 ? std::min<int64_t>(cols / 128, t128) * t128 : t128 * (t128 + 1) / 2;
            if (n128 < 512)
                return syrk_cfg<64, 16, 2, 2, false, sizeof(R) == 8>(m, W, ldw, kp, C, ldc, jt(64), info, s, x);
            if constexpr (sizeof(R) == 4) {
                // fp32: 32-deep slices for large orders (72 % of the fp32 peak
                // against 61 % at m = 15872), 16-deep below
                if (m >= syrk_deep_rows(4))
                    return syrk_cfg<128, 32, 2, 4, false, true>(m, W, ldw, kp, C, ldc, jt(128), info, s, x);
                return syrk_cfg<128, 16, 2, 4>(m, W, ldw, kp, C, ldc, jt(128), info, s, x);
            } else {
                // slice depth 8 (more workgroups in flight per byte of LDS);
                // 16 from syrk_deep_rows(8) on, which the option can set
                if (m >= syrk_deep_rows(8))
                    return syrk_cfg<128, 16, 2, 4>(m, W, ldw, kp, C, ldc, jt(128), info, s, x);
                return syrk_cfg<128, 8, 2, 4>(m, W, ldw, kp, C, ldc, jt(128), info, s, x);
            }
        }
    }

    // C (m x ncols, ldc) -/+= W V^H over every tile, W and V in the padded
    // panel layout (same ldw, rows up to the larger of m and ncols rounded to
    // the tile); on the trailing-update kernel.
    static int rect_update(int64_t m, int64_t ncols, const E *W, const E *Vc, int64_t ldw, int64_t kp, E *C,
                           int64_t ldc, bool add, const int *info, hipStream_t s)
    {
        if (m <= 0 || ncols <= 0)
            return 0;
        Syr2 x;
        x.V = Vc;
        x.add = add;
        x.ncols = ncols;
        if (ldc >= SYRK_LD32)  // 64-bit offsets into C
            return syrk_cfg<64, 16, 2, 2, true>(m, W, ldw, kp, C, ldc, 0, info, s, x);
        if constexpr (CPLX) {
            return syrk_cfg<64, 16, 2, 2>(m, W, ldw, kp, C, ldc, 0, info, s, x);
        } else {
            if (cdiv(m, 128) * cdiv(ncols, 128) < 512)
                return syrk_cfg<64, 16, 2, 2>(m, W, ldw, kp, C, ldc, 0, info, s, x);
            if constexpr (sizeof(R) == 4)
                return syrk_cfg<128, 16, 2, 4>(m, W, ldw, kp, C, ldc, 0, info, s, x);
            else
                return syrk_cfg<128, 16, 2, 4>(m, W, ldw, kp, C, ldc, 0, info, s, x);
        }
    }

    template <int BM, int BN, int KB, int WM, int WN, bool PT, bool VEC, bool STORE = false>
    static int rect_cfg(const E *P, int64_t ldp, const E *Q, int64_t ldq, E *C, int64_t ldc, int64_t m,
                        int64_t n, int64_t kp, int64_t kvalid, const int *info, hipStream_t s)
    {
        static_assert(RECT_LDQ % BN == 0 && RECT_KB % KB == 0, "operand buffer padding too small for the tile");
        RectArgs a;
        a.P = P;
        a.ldp = ldp;
        a.Q = Q;
        a.ldq = ldq;
        a.C = C;
        a.ldc = ldc;
        a.m = (int)m;
        a.n = (int)n;
        a.kp = (int)kp;
        a.kvalid = (int)kvalid;
        a.tiles_m = (int)cdiv(m, BM);
        a.ntiles = a.tiles_m * (int)cdiv(n, BN);
        a.info = info;
        const dim3 grid((unsigned)a.ntiles), block(64 * WM * WN);
        SPD_VALIDATE((check_rect<R, BM, BN, KB, WM, WN, PT, VEC, STORE>(a, grid, g_chk)));
        ProfScope ps(STORE ? -1 : PROF_UPDATE, 2.0 * (double)m * n * kvalid, s);  // STORE: potrf's panel
        rect_kernel<R, BM, BN, KB, WM, WN, PT, VEC, 1, STORE><<<grid, block, 0, s>>>(a);
        SPD_CHECK_LAUNCH("rect_kernel");
        return 0;
    }

    // C(m x n) -= P Q^T for the substitutions (see spd_rect.hpp); Q is the
    // solved block transposed into the ldq x kp operand buffer.
    template <bool PT>
    static int rect(const E *P, int64_t ldp, const E *Q, int64_t ldq, E *C, int64_t ldc, int64_t m, int64_t n,
                    int64_t kp, int64_t kvalid, bool vec, const int *info, hipStream_t s)
    {
        if (m <= 0 || n <= 0)
            return 0;
        if constexpr (CPLX) {
            g_last_error = "block update kernel is for real types";
            return SPD_ERR_HIP;
        } else {
            // tile rows by update height: 64 x 64 tiles from 16384 rows (two to
            // four workgroups per CU at 128 columns; measured 5 % faster over a
            // solve than 64 x 128 tiles, which leave CUs idle where the tile
            // count is not a multiple of the CU count), else 32-row tiles (one
            // workgroup's 512-deep product is a fixed latency, so more, smaller
            // tiles finish sooner)
            constexpr int KBL = sizeof(R) == 8 ? 16 : 32;  // slice depth of the 64-row tiles
            if (m >= rect_tall_rows())
                return vec ? rect_cfg<64, 64, KBL, 2, 2, PT, true>(P, ldp, Q, ldq, C, ldc, m, n, kp, kvalid, info, s)
                           : rect_cfg<64, 64, KBL, 2, 2, PT, false>(P, ldp, Q, ldq, C, ldc, m, n, kp, kvalid, info, s);
            if (n > 64)
                return vec ? rect_cfg<32, 128, 32, 1, 4, PT, true>(P, ldp, Q, ldq, C, ldc, m, n, kp, kvalid, info, s)
                           : rect_cfg<32, 128, 32, 1, 4, PT, false>(P, ldp, Q, ldq, C, ldc, m, n, kp, kvalid, info, s);
            return vec ? rect_cfg<32, 64, 32, 1, 2, PT, true>(P, ldp, Q, ldq, C, ldc, m, n, kp, kvalid, info, s)
                       : rect_cfg<32, 64, 32, 1, 2, PT, false>(P, ldp, Q, ldq, C, ldc, m, n, kp, kvalid, info, s);
        }
    }

    // The block update kernel addresses P with 32-bit offsets inside a tile
    // (64 columns of A must span fewer than 2^31 elements).  It reads P with
    // 16-byte vectors when A is 16-byte aligned and the leading dimension and
    // the block offsets (multiples of T) keep every vector aligned; otherwise
    // element by element, with the same arithmetic.
    static bool rect_usable(int64_t lda) { return !CPLX && lda < (INT64_C(1) << 24); }
    static bool rect_vec(const E *A, int64_t lda, int64_t T)
    {
        const int64_t V = 16 / (int64_t)sizeof(E);
        return ((uintptr_t)A % 16 == 0) && (lda % V == 0) && (T % V == 0);
    }

    static int copy_t(E *dst, int64_t ldd, E *qt, int64_t ldq, const E *src, int64_t lds, int64_t m, int64_t n,
                      int64_t kp, const int *info, hipStream_t s)
    {
        if (kp <= 0 || n <= 0)
            return 0;
        SPD_VALIDATE((check_copy_t<E>(dst, ldd, qt, ldq, src, lds, m, n, kp, info, g_chk)));
        const int64_t blocks = std::min<int64_t>(cdiv(kp * n, 256), 4096);
        copy_t_kernel<E><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(dst, ldd, qt, ldq, src, lds, m, n, kp, info);
        SPD_CHECK_LAUNCH("copy_t_kernel");
        return 0;
    }

    // Diagonal tile at (c0, c0) of order tk = min(T, n - c0): factor it in
    // place and build inv(L_kk) in Inv (ld T); then, if rows remain below it,
    // solve the panel into Wk with the zero-padded layout the trailing update
    // reads (leading dimension m rounded up to SYRK_LDW, width tk rounded up to
    // SYRK_KP) and copy it back into A.  All on stream s.
    // ldw_fixed > 0: Wk's leading dimension (the two-step schedule keeps all
    // panels at one leading dimension); rows [m, m rounded up to SYRK_LDW) are
    // zeroed either way.
    // Wprev (ld ldw_fixed), wk > 0: the tile first takes the last trailing
    // update A_kk -= Wprev_k Wprev_k^H itself (one-launch tile only), Wprev_k
    // the previous panel's rows of this tile; then before_panel (if given)
    // runs between the tile and the panel product (the caller makes s wait
    // for the update of the rest of the tile column there).
    static int diag_panel(int64_t n, E *A, int64_t lda, int64_t T, int64_t c0, E *Inv, E *Wk, int *info,
                          int *ctr, hipStream_t s, int64_t ldw_fixed = 0, const E *Wprev = nullptr,
                          int64_t wk = 0, const std::function<int()> *before_panel = nullptr)
    {
        const int64_t tk = std::min(T, n - c0);
        E *D = A + c0 + c0 * lda;
        if (Wprev != nullptr && (!tile_launch_enabled() || ldw_fixed <= 0)) {
            g_last_error = "the tile's own trailing update needs the one-launch tile";
            return SPD_ERR_HIP;
        }
        if (tile_launch_enabled()) {
            ProfScope ps(PROF_DIAG, FMUL * 2.0 * (double)tk * tk * tk / 3.0, s);
            SPD_TRY(tile_launch(D, lda, tk, Inv, T, info, tile_flags(ctr), c0, n - c0 - tk, s, Wprev, ldw_fixed,
                                wk));
        } else {
            ProfScope ps(PROF_DIAG, FMUL * 2.0 * (double)tk * tk * tk / 3.0, s);
            for (int64_t b0 = 0; b0 < tk; b0 += LEAF) {
                const int64_t lb = std::min<int64_t>(LEAF, tk - b0);
                E *Db = D + b0 + b0 * lda;
                const int64_t r = tk - b0 - lb;
                E *P = Db + lb;  // r x lb below the leaf
                // the leaf and P <- P inv(Lb)^H in one launch
                SPD_TRY(leaf_panel(Db, lda, lb, std::max<int64_t>(r, 0), Inv + b0 * (1 + T), T, info, ctr, c0 + b0, s));
                if (r <= 0)
                    continue;
                Gemm u;  // rest of the tile: lower part of D22 -= P P^H
                u.A = P;
                u.lda = lda;
                u.B = P;
                u.ldb = lda;
                u.C = P + lb * lda;
                u.ldc = lda;
                u.m = r;
                u.n = r;
                u.k = lb;
                u.tri = true;
                u.neg = true;
                u.beta = true;
                u.info = info;
                SPD_TRY((gemm<R, CPLX>(NT, u, s)));
            }
            SPD_TRY(merge_inverses(D, lda, 0, Inv, T, 0, 1, tk, Wk, info, s));
        }
        if (before_panel != nullptr)
            SPD_TRY((*before_panel)());
        const int64_t m = n - c0 - tk;
        if (m <= 0)
            return 0;
        E *P = D + tk;  // m x tk panel
        const int64_t ldw = ldw_fixed > 0 ? ldw_fixed : align_up(m, SYRK_LDW), kp = align_up(tk, SYRK_KP);
        ProfScope ps(PROF_PANEL, FMUL * (double)m * tk * tk, s);
        bool done = false;
        if constexpr (!CPLX) {
            if (T % RECT_LDQ == 0 && tk == T && rect_usable(lda)) {
                // Wk = P inv(L_kk)^T on the block-update kernel (C = P Q^T with
                // Q = inv(L_kk), ld T): more, shorter workgroups than the general
                // product, which matters in the late steps where this product is
                // on the critical path
                const bool vec = rect_vec(A, lda, T);
                if (m >= rect_tall_rows())
                    SPD_TRY((vec ? rect_cfg<64, 128, (sizeof(R) == 8 ? 16 : 32), 2, 4, false, true, true>(
                                       P, lda, Inv, T, Wk, ldw, m, tk, tk, tk, info, s)
                                 : rect_cfg<64, 128, (sizeof(R) == 8 ? 16 : 32), 2, 4, false, false, true>(
                                       P, lda, Inv, T, Wk, ldw, m, tk, tk, tk, info, s)));
                else
                    SPD_TRY((vec ? rect_cfg<32, 128, 32, 1, 4, false, true, true>(P, lda, Inv, T, Wk, ldw, m, tk, tk, tk,
                                                                                 info, s)
                                 : rect_cfg<32, 128, 32, 1, 4, false, false, true>(P, lda, Inv, T, Wk, ldw, m, tk, tk,
                                                                                  tk, info, s)));
                done = true;
            }
        }
        if (!done) {
            Gemm g;  // Wk = P inv(L_kk)^H
            g.A = P;
            g.lda = lda;
            g.B = Inv;
            g.ldb = T;
            g.C = Wk;
            g.ldc = ldw;
            g.m = m;
            g.n = tk;
            g.k = tk;
            g.kmode = KM_END_BY_J;
            g.info = info;
            g.small = true;  // lean tiles: this product shares the GPU with the trailing update
            SPD_TRY((gemm<R, CPLX>(NT, g, s)));
        }
        SPD_TRY(zero2d<E>(Wk + m, ldw, align_up(m, SYRK_LDW) - m, kp, s));
        SPD_TRY(zero2d<E>(Wk + tk * ldw, ldw, m, kp - tk, s));
        SPD_TRY(copy2d<E>(P, lda, Wk, ldw, m, tk, info, s));
        return 0;
    }

    // Right-looking blocked Cholesky.  Without lookahead, step k is: diagonal
    // tile and panel k, then the whole trailing update with panel k.  With
    // lookahead (T a multiple of the trailing-update tile, three or more
    // tiles), an auxiliary stream runs ahead by one step: it applies panel k to
    // the next tile column only, factors diagonal tile k+1 and solves panel k+1
    // (into the other panel buffer), while the caller's stream applies panel k
    // to the rest of the trailing matrix.  Events order the two streams:
    // panel k is ready before stream s uses it, and the update of step k-1 has
    // finished before the auxiliary stream touches tile column k+1.
    // Called as tiles of L become final (tiles [k0, k1)), on the host, right
    // after the auxiliary stream's event for them is recorded; the fused
    // solve enqueues its forward substitution steps from it.
    typedef std::function<int(int64_t, int64_t)> PanelHook;

    static bool two_step_schedule(int64_t T, int64_t nt)
    {
        return lookahead_enabled() && (T % syrk_bm() == 0) && nt >= 3 && two_step_enabled();
    }

    // hook (the two-step schedule only): every tile's inverse is kept (tile k
    // at Inv + k T^2) and hook is called as tiles become final
    static int potrf(int64_t n, E *A, int64_t lda, int64_t T_A, int *info, void *work, hipStream_t s,
                     const PanelHook *hook = nullptr)
    {
        SPD_TRY(set_info(info, s));
        if (n == 0)
            return 0;
        const Layout L = make_layout(n, 0, T_A, sizeof(E));
        const int64_t T = L.T, nt = L.nt;
        E *Inv = (E *)work + L.inv;  // inverse of the current diagonal tile, ld T
        int *ctr = (int *)((E *)work + L.ctr);
        SPD_TRY(set_info(ctr, s));
        SPD_TRY(zero2d<int>(tile_flags(ctr), 1, tile_flag_ints((int)cdiv(T, LEAF)), 1, s));
        E *Wb[2] = {(E *)work + L.w, (E *)work + L.w + L.wsz};
        SPD_TRY(zero2d<E>(Inv, T, T, hook != nullptr ? nt * T : T, s));
        if (hook != nullptr && !two_step_schedule(T, nt)) {
            g_last_error = "panel hook needs the two-step schedule";
            return SPD_ERR_HIP;
        }
        const bool lookahead = lookahead_enabled() && (T % syrk_bm() == 0) && nt >= 3;
        if (!lookahead) {
            for (int64_t c0 = 0; c0 < n; c0 += T) {
                const int64_t tk = std::min(T, n - c0), m = n - c0 - tk;
                SPD_TRY(diag_panel(n, A, lda, T, c0, Inv, Wb[0], info, ctr, s));
                if (m > 0)
                    SPD_TRY(syrk(m, Wb[0], align_up(m, SYRK_LDW), align_up(tk, SYRK_KP), tk,
                                 A + (c0 + tk) * (1 + lda), lda, 0, info, s));
            }
            return 0;
        }
        if (two_step_enabled())
            return potrf_pairs(n, A, lda, L, Inv, info, ctr, work, s, hook);
        Lookahead la;
        SPD_TRY(la.begin(s));
        hipStream_t sl = la.look;
        SPD_TRY(diag_panel(n, A, lda, T, 0, Inv, Wb[0], info, ctr, sl));
        SPD_TRY(la.record(la.ev_panel, sl));
        const int kp = (int)align_up(T, SYRK_KP);
        for (int64_t k = 0; k + 1 < nt; ++k) {
            const int64_t c0 = k * T, m = n - c0 - T, ldw = align_up(m, SYRK_LDW);
            E *Wk = Wb[k % 2];
            SPD_TRY(la.wait(s, la.ev_panel));  // panel k
            if (k > 0)
                SPD_TRY(la.wait(sl, la.ev_rest));  // update of step k-1 done
            // tile column k+1 of the trailing matrix, then diagonal tile and panel k+1
            SPD_TRY(syrk(m, Wk, ldw, kp, T, A + (c0 + T) * (1 + lda), lda, T, info, sl, aux_update()));
            if (m - T < column_first_rows()) {
                SPD_TRY(la.record(la.ev_col, sl));
                SPD_TRY(la.wait(s, la.ev_col));
            }
            SPD_TRY(diag_panel(n, A, lda, T, c0 + T, Inv, Wb[(k + 1) % 2], info, ctr, sl));
            SPD_TRY(la.record(la.ev_panel, sl));
            // the rest of the trailing matrix, beyond tile column k+1
            if (m > T)
                SPD_TRY(syrk(m - T, Wk + T, ldw, kp, T, A + (c0 + 2 * T) * (1 + lda), lda, 0, info, s));
            SPD_TRY(la.record(la.ev_rest, s));
        }
        SPD_TRY(la.wait(s, la.ev_panel));  // join: last diagonal tile
        return 0;
    }

    // Multi-step lookahead: while the trailing matrix is large, the update
    // beyond the next tiles is applied once per group of steps with all of the
    // group's panels at once (depth gT, g = 2 or 3), which the trailing-update
    // kernel runs at a higher rate than depth T.  In state S(a, g) the panels
    // W_a .. W_{a+g-1} are solved, tile columns a+1 .. a+g-1 have every update
    // and the tiles from a+g on have the updates by the panels before a.  One
    // group step S(a, g) -> S(a+g, h): the auxiliary stream applies
    // [W_a | .. | W_{a+g-1}] to tile columns a+g .. a+g+h-1 and then factors
    // those h tiles one after the other (each tile's panel applied to the
    // group's later tile columns before the next tile), while the caller's
    // stream applies [W_a | .. | W_{a+g-1}] to the trailing matrix from tile
    // a+g+h on.  Groups of three while three_step_rows() rows remain beyond
    // the new group (orders with six panel buffers), of two while
    // two_step_rows() do; below that the auxiliary stream's chain (two or three
    // tiles) would outlast the caller's update, and the schedule continues one
    // step at a time as in potrf.  The first step, from tile 0 alone, already
    // solves two or three tiles, so that the caller's first update starts after
    // tile 0.  Panel k lives in buffer k mod npanels; every buffer's row r
    // holds row r + T of A (panel k's first row, row (k+1)T, is its row kT),
    // and the buffers are adjacent, so the panels of a group read from one
    // row of A on are one operand of depth gT (two, where the group wraps
    // from the last buffer to the first).
    static int potrf_pairs(int64_t n, E *A, int64_t lda, const Layout &L, E *Inv0, int *info, int *ctr, void *work,
                           hipStream_t s, const PanelHook *hook = nullptr)
    {
        const int64_t T = L.T, nt = L.nt, ldw = align_up(n, SYRK_LDW), kp = align_up(T, SYRK_KP);
        const int64_t NB = L.npanels;
        E *const W0 = (E *)work + L.w;
        auto Wp = [&](int64_t k) { return W0 + (k % NB) * L.wsz + k * T; };
        // [W_a | .. | W_{a+g-1}] from row r of A on; x gets the second operand
        // if the group wraps past the last buffer
        auto group = [&](int64_t a, int64_t g, int64_t r, Syr2 &x) -> const E * {
            const int64_t b = a % NB;
            x.W2 = nullptr;
            x.kp1 = 0;
            if (b + g > NB) {
                x.W2 = W0 + (r - T);
                x.kp1 = (NB - b) * kp;
            }
            return W0 + b * L.wsz + (r - T);
        };
        auto C = [&](int64_t k) { return A + k * T * (1 + lda); };  // trailing matrix from tile k
        auto Iv = [&](int64_t k) { return hook != nullptr ? Inv0 + k * T * T : Inv0; };
        auto diag_panel = [&](int64_t c0, E *Wk, hipStream_t st, const E *Wprev = nullptr,
                              const std::function<int()> *before_panel = nullptr) {
            return Solver::diag_panel(n, A, lda, T, c0, Iv(c0 / T), Wk, info, ctr, st, ldw, Wprev, T, before_panel);
        };
        auto done = [&](int64_t k0, int64_t k1) { return hook != nullptr ? (*hook)(std::min(k0, nt), std::min(k1, nt)) : 0; };
        Lookahead la;
        SPD_TRY(la.begin(s));
        hipStream_t sl = la.look;
        // S(a, g) -> S(a+g, h)
        auto group_step = [&](int64_t a, int64_t g, int64_t h) -> int {
            const int64_t c = a + g, e = c + h;
            SPD_TRY(la.wait(s, la.ev_panel));  // panels a .. c-1
            if (a > 0)
                SPD_TRY(la.wait(sl, la.ev_rest));  // the caller's update before has reached tile column c
            Syr2 x;
            x.aux = true;
            const E *Wc = group(a, g, c * T, x);
            SPD_TRY(syrk(n - c * T, Wc, ldw, g * kp, g * T, C(c), lda, h * T, info, sl, x));
            for (int64_t t = c; t < e; ++t) {
                SPD_TRY(diag_panel(t * T, Wp(t), sl));
                if (t + 1 < e)
                    SPD_TRY(syrk(n - (t + 1) * T, Wp(t), ldw, kp, T, C(t + 1), lda, (e - 1 - t) * T, info, sl,
                                 aux_update()));
            }
            SPD_TRY(la.record(la.ev_panel, sl));
            SPD_TRY(done(c, e));
            if (e * T < n) {
                Syr2 y;
                const E *We = group(a, g, e * T, y);
                SPD_TRY(syrk(n - e * T, We, ldw, g * kp, g * T, C(e), lda, 0, info, s, y));
            }
            SPD_TRY(la.record(la.ev_rest, s));
            return 0;
        };
        // the size of the next group from S(a, g)
        const int64_t triple_rows = NB >= 6 ? three_step_rows(T) : 0, pair_rows = two_step_rows(T);
        auto next_group = [&](int64_t a, int64_t g) -> int64_t {
            const int64_t c = a + g;
            if (triple_rows > 0 && c + 3 <= nt && n - (c + 3) * T >= triple_rows)
                return 3;
            if (c + 2 <= nt && (a == 0 || n - (c + 2) * T >= pair_rows))
                return 2;
            return 1;
        };
        SPD_TRY(diag_panel(0, Wp(0), sl));
        SPD_TRY(la.record(la.ev_panel, sl));
        SPD_TRY(done(0, 1));
        int64_t a = 0, g = 1;
        for (;;) {
            if (a + g >= nt)
                break;
            const int64_t h = next_group(a, g);
            if (g == 1 && h == 1 && a > 0)
                break;  // single steps from k = a on
            SPD_TRY(group_step(a, g, h));
            a += g;
            g = h;
        }
        if (a + g >= nt) {
            SPD_TRY(la.wait(s, la.ev_panel));  // join: the last tile
            return 0;
        }
        // single steps from k = a (S(a, 1): panel a solved, the tiles from a+1
        // on updated by the panels before a)
        for (int64_t k = a; k + 1 < nt; ++k) {
            if (tile_launch_enabled() && n - (k + 2) * T < tile_update_rows(CPLX)) {
                // Tile k+1 takes its update by W_k inside its own launch, beside
                // the caller's update of everything else from tile column k+1
                // on; panel k+1 waits for that update (the rest of its column).
                SPD_TRY(la.wait(sl, la.ev_rest));  // the update of step k-1 reached tile k+1
                const std::function<int()> rest = [&]() -> int {
                    SPD_TRY(la.wait(s, la.ev_panel));  // panel k
                    Syr2 x;
                    x.skip = T;
                    SPD_TRY(syrk(n - (k + 1) * T, Wp(k), ldw, kp, T, C(k + 1), lda, 0, info, s, x));
                    SPD_TRY(la.record(la.ev_rest, s));
                    return la.wait(sl, la.ev_rest);
                };
                SPD_TRY(diag_panel((k + 1) * T, Wp(k + 1), sl, Wp(k), &rest));
                SPD_TRY(la.record(la.ev_panel, sl));
                SPD_TRY(done(k + 1, k + 2));
                continue;
            }
            SPD_TRY(la.wait(s, la.ev_panel));  // panel k
            SPD_TRY(la.wait(sl, la.ev_rest));  // the update of step k-1 reached tile column k+1
            SPD_TRY(syrk(n - (k + 1) * T, Wp(k), ldw, kp, T, C(k + 1), lda, T, info, sl, aux_update()));
            if (n - (k + 2) * T < column_first_rows()) {
                SPD_TRY(la.record(la.ev_col, sl));
                SPD_TRY(la.wait(s, la.ev_col));
            }
            SPD_TRY(diag_panel((k + 1) * T, Wp(k + 1), sl));
            SPD_TRY(la.record(la.ev_panel, sl));
            SPD_TRY(done(k + 1, k + 2));
            if ((k + 2) * T < n)
                SPD_TRY(syrk(n - (k + 2) * T, Wp(k) + T, ldw, kp, T, C(k + 2), lda, 0, info, s));
            SPD_TRY(la.record(la.ev_rest, s));
        }
        SPD_TRY(la.wait(s, la.ev_panel));  // join: the last tile
        return 0;
    }

    // Y_k (or X_k) = inv(L_kk) B_k (TRANS: inv(L_kk)^H B_k) into Tmp (ld T)
    static int apply_inv(const E *Inv, int64_t k, int64_t T, E *B, int64_t ldb, int64_t c0, int64_t tk, int64_t nrhs,
                         E *Tmp, bool trans, const int *info, hipStream_t s)
    {
        Gemm g;
        g.A = Inv + k * T * T;
        g.lda = T;
        g.B = B + c0;
        g.ldb = ldb;
        g.C = Tmp;
        g.ldc = T;
        g.m = tk;
        g.n = nrhs;
        g.k = tk;
        g.kmode = trans ? KM_BEG_BY_I : KM_END_BY_I;
        g.info = info;
        return trans ? gemm<R, CPLX>(TN, g, s) : gemm<R, CPLX>(NN, g, s);
    }

    // inverses of every diagonal tile, for the block substitutions
    static int all_inverses(int64_t n, const E *A, int64_t lda, int64_t T, int64_t nt, E *Inv, E *W, const int *info,
                            hipStream_t s)
    {
        SPD_TRY(zero2d<E>(Inv, T, T, nt * T, s));
        SPD_TRY(leaves(const_cast<E *>(A), lda, n, T, Inv, T, T * T, nt, false, const_cast<int *>(info), 0, s));
        const int64_t nfull = (n % T == 0) ? nt : nt - 1;
        if (nfull > 0)
            SPD_TRY(merge_inverses(A, lda, T * (1 + lda), Inv, T, T * T, nfull, T, W, info, s));
        if (nfull < nt) {
            const int64_t c0 = nfull * T;
            SPD_TRY(merge_inverses(A + c0 + c0 * lda, lda, 0, Inv + nfull * T * T, T, 0, 1, n - c0, W, info, s));
        }
        return 0;
    }

    // GB_k = -L_k,k-1 inv(L_k-1,k-1) into GB + k T T (leading dimension T) for
    // the batch tiles k, k + 1, ..., each of m rows (m = min(T, n - k T) for
    // one tile alone).
    static int back_chain_product(int64_t k, int64_t m, int batch, const E *A, int64_t lda, int64_t T,
                                  const E *Inv, E *GB, const int *info, hipStream_t s)
    {
        Gemm h;
        h.A = A + k * T + (k - 1) * T * lda;
        h.lda = lda;
        h.sA_out = T * (1 + lda);
        h.B = Inv + (k - 1) * T * T;
        h.ldb = T;
        h.sB_out = T * T;
        h.C = GB + k * T * T;
        h.ldc = T;
        h.sC_out = T * T;
        h.batch = batch;
        h.m = m;
        h.n = h.k = T;
        h.kmode = KM_BEG_BY_J;
        h.neg = true;
        h.info = info;
        return gemm<R, CPLX>(NN, h, s);
    }

    // GB_k for the whole tiles k = 1 .. n / T - 1 in one batched product and,
    // with ragged, for a short last tile in a second one.
    static int back_chain_products(int64_t n, const E *A, int64_t lda, int64_t T, const E *Inv, E *GB,
                                   bool ragged, const int *info, hipStream_t s)
    {
        const int64_t nfull = n / T, tail = n - nfull * T;
        auto product = [&](int64_t k, int64_t m, int batch) {
            return back_chain_product(k, m, batch, A, lda, T, Inv, GB, info, s);
        };
        if (nfull >= 2)
            SPD_TRY(product(1, T, (int)(nfull - 1)));
        if (ragged && tail > 0 && nfull >= 1)
            SPD_TRY(product(nfull, tail, 1));
        return 0;
    }

    // The back substitution L^H X = Y in one launch (subst_kernel), with the
    // inverse of every diagonal tile in the workspace's INV region and the
    // products G_i = GB_{i+1} formed first (back_chain_products); Z and the
    // flags in the workspace (the flags zeroed first).  status (may be null)
    // becomes -1 if a wait of the launch runs out; X is then NaN.
    template <int TC>
    static int back_subst_tc(int64_t n, int64_t nrhs, const E *A, int64_t lda, E *B, int64_t ldb, const Layout &L,
                             const int *info, int *status, void *work, hipStream_t s, bool have_g)
    {
        SubstArgs p;
        E *const GB = (E *)work + L.gb;
        if (!have_g)
            SPD_TRY(back_chain_products(n, A, lda, L.T, (const E *)work + L.inv, GB, true, info, s));
        p.A = A;
        p.lda = lda;
        p.Inv = (const E *)work + L.inv;
        p.G = GB;
        p.B = B;
        p.ldb = ldb;
        p.Z = (E *)work + L.z;
        p.ldz = L.ldz;
        p.n = (int)n;
        p.nrhs = (int)nrhs;
        p.T = (int)L.T;
        p.nt = (int)L.nt;
        p.nr = (int)cdiv(L.T, SUB_TR);
        p.nc = (int)cdiv(nrhs, TC);
        p.flags = (int *)((E *)work + L.sflags);
        p.info = info;
        p.status = status;
        p.limit = tile_wait_ticks();
        SPD_TRY(zero2d<int>(p.flags, 1, subst_flag_ints(p.nt, p.nc), 1, s));
        const unsigned grid = (unsigned)subst_groups(p);
        SPD_VALIDATE((check_subst<R, CPLX, TC>(p, grid, g_chk)));
        subst_kernel<R, CPLX, TC><<<dim3(grid), dim3(SUB_THREADS), 0, s>>>(p);
        SPD_CHECK_LAUNCH("subst_kernel");
        return 0;
    }
    // have_g: the products G_i are already in the workspace's GB region
    static int back_subst(int64_t n, int64_t nrhs, const E *A, int64_t lda, E *B, int64_t ldb, const Layout &L,
                          const int *info, int *status, void *work, hipStream_t s, bool have_g = false)
    {
        if (subst_tc(nrhs) == 32)
            return back_subst_tc<32>(n, nrhs, A, lda, B, ldb, L, info, status, work, s, have_g);
        return back_subst_tc<64>(n, nrhs, A, lda, B, ldb, L, info, status, work, s, have_g);
    }

    // backward = false: the forward substitution L Y = B only
    static int potrs(int64_t n, int64_t nrhs, const E *A, int64_t lda, E *B, int64_t ldb, int64_t T_A,
                     const int *info, void *work, hipStream_t s, bool backward = true)
    {
        if (n == 0 || nrhs == 0)
            return 0;
        const Layout L = make_layout(n, nrhs, T_A, sizeof(E));
        {
            ProfScope ps(PROF_SOLVE, FMUL * (backward ? 2.0 : 1.0) * (double)n * n * nrhs, s);
            // the back substitution in one launch: the sweeps below only solve
            // L Y = B (and build the tile inverses)
            const bool one = backward && subst_launch_enabled(n, nrhs, CPLX);
            if (rect_usable(lda))
                SPD_TRY(potrs_blocks(n, nrhs, A, lda, B, ldb, L, info, work, s, backward && !one));
            else
                SPD_TRY(potrs_general(n, nrhs, A, lda, B, ldb, L, info, work, s, backward && !one));
            if (one)  // d_info is read-only here: a wait that runs out shows as NaN in X
                SPD_TRY(back_subst(n, nrhs, A, lda, B, ldb, L, info, nullptr, work, s));
        }
        return nan_fill(n, nrhs, B, ldb, info, s);
    }

    // Gaussian-process marginal log-likelihood of the residual columns of R
    // (real types): R <- L^-1 R, then the per-column reduction.
    static int gp_loglik(int64_t n, int64_t nrhs, const E *A, int64_t lda, E *Rm, int64_t ldr, int64_t T_A,
                         const int *info, double *out, void *work, hipStream_t s)
    {
        if (nrhs == 0)
            return 0;
        SPD_TRY(potrs(n, nrhs, A, lda, Rm, ldr, T_A, info, work, s, false));
        if constexpr (CPLX) {
            g_last_error = "the likelihood is defined for real types";
            return SPD_ERR_HIP;
        } else {
            SPD_VALIDATE((check_gp_loglik<R>(Rm, ldr, A, lda, n, nrhs, info, out, g_chk)));
            gp_loglik_kernel<R><<<dim3((unsigned)nrhs), dim3(256), 0, s>>>(Rm, ldr, A, lda, n, info, out);
            SPD_CHECK_LAUNCH("gp_loglik_kernel");
            return 0;
        }
    }

    // Fused solve: potrf, log det (optional) and potrs in one call.  With the
    // multi-step factorization schedule (any type) the forward substitution
    // runs on a second auxiliary stream, one block as
    // soon as its tile of L is final (the factorization keeps every tile's
    // inverse), so that it fills the factorization's chain-bound tail; the
    // back substitution follows.  Otherwise the three calls in sequence.
    static int posv(int64_t n, int64_t nrhs, E *A, int64_t lda, E *B, int64_t ldb, int64_t T_A, int *info,
                    double *logdet_out, void *work, hipStream_t s)
    {
        const Layout L = make_layout(std::max<int64_t>(n, 1), nrhs, T_A, sizeof(E));
        // real types take the block-update kernel for the substitutions, complex
        // types (and very large leading dimensions) the general product
        const bool blocks = !CPLX && rect_usable(lda);
        bool fused = n > 0 && nrhs > 0 && two_step_schedule(L.T, L.nt);
        if (!fused) {
            SPD_TRY(potrf(n, A, lda, T_A, info, work, s));
            if (logdet_out != nullptr)
                SPD_TRY(logdet(n, A, lda, info, logdet_out, s));
            return potrs(n, nrhs, A, lda, B, ldb, T_A, info, work, s);
        }
        const int64_t T = L.T;
        // The forward steps run beside the factorization, which uses INV, W and
        // its counter (placed for n_rhs = 0, possibly inside this layout's
        // TMP): they take their block row from PART and their transposed
        // block from the first operand buffer, both beyond the factorization's
        // regions.
        E *Inv = (E *)work + L.inv;
        E *Tmp = (E *)work + L.part;
        E *Qf = (E *)work + L.q;
        const bool vec = rect_vec(A, lda, T);
        Lookahead la;  // the factorization's streams and events (shared per thread and device)
        SPD_TRY(la.begin(s));
        hipStream_t fs = la.look2;
        // the back substitution's chain products G_k = GB_{k+1} (in GB, beyond
        // the factorization's regions too), one per tile as its tile column of
        // L becomes final (for the one launch and for the block steps)
        const bool one = subst_launch_enabled(n, nrhs, CPLX);
        auto step = [&](int64_t k) -> int {  // Y_k = inv(L_kk) B_k, then B below -= L_panel Y_k
            const int64_t c0 = k * T, tk = std::min(T, n - c0), r0 = c0 + tk, kp = align_up(tk, RECT_KB);
            if ((one || blocks) && r0 < n)
                SPD_TRY(back_chain_product(k + 1, std::min(T, n - r0), 1, A, lda, T, Inv, (E *)work + L.gb, info,
                                           fs));
            SPD_TRY(apply_inv(Inv, k, T, B, ldb, c0, tk, nrhs, Tmp, false, info, fs));
            if (!blocks) {
                SPD_TRY(copy2d<E>(B + c0, ldb, Tmp, T, tk, nrhs, info, fs));
                if (r0 < n) {
                    Gemm u;  // B_below -= L_panel Y_k
                    u.A = A + r0 + c0 * lda;
                    u.lda = lda;
                    u.B = B + c0;
                    u.ldb = ldb;
                    u.C = B + r0;
                    u.ldc = ldb;
                    u.m = n - r0;
                    u.n = nrhs;
                    u.k = tk;
                    u.neg = true;
                    u.beta = true;
                    u.info = info;
                    SPD_TRY((gemm<R, CPLX>(NN, u, fs)));
                }
                return 0;
            }
            SPD_TRY(copy_t(B + c0, ldb, Qf, L.ldq, Tmp, T, tk, nrhs, kp, info, fs));
            if (r0 < n)
                SPD_TRY(rect<false>(A + r0 + c0 * lda, lda, Qf, L.ldq, B + r0, ldb, n - r0, nrhs, kp, tk, vec, info,
                                    fs));
            return 0;
        };
        const PanelHook hook = [&](int64_t k0, int64_t k1) -> int {
            if (k0 >= k1)
                return 0;
            SPD_TRY(la.wait(fs, la.ev_panel));  // tiles [k0, k1) of L are final
            for (int64_t k = k0; k < k1; ++k)
                SPD_TRY(step(k));
            return 0;
        };
        {
            ProfScope ps(PROF_SOLVE, FMUL * (double)n * n * nrhs, s);  // the factorization with the forward sweep
            SPD_TRY(potrf(n, A, lda, T_A, info, work, s, &hook));
            SPD_TRY(la.record(la.ev_fw, fs));
            SPD_TRY(la.wait(s, la.ev_fw));
        }
        if (logdet_out != nullptr)
            SPD_TRY(logdet(n, A, lda, info, logdet_out, s));
        {
            ProfScope ps(PROF_SOLVE, FMUL * (double)n * n * nrhs, s);
            if (one)
                SPD_TRY(back_subst(n, nrhs, A, lda, B, ldb, L, info, info, work, s, true));
            else if (blocks)
                SPD_TRY(potrs_blocks(n, nrhs, A, lda, B, ldb, L, info, work, s, true, false, nullptr, false));
            else
                SPD_TRY(potrs_general(n, nrhs, A, lda, B, ldb, L, info, work, s, true, false, false));
        }
        return nan_fill(n, nrhs, B, ldb, info, s);
    }

    // Reduction of the Hermitian-definite generalized eigenproblem to standard
    // form from B = L L^H (L from potrf, lower triangle read only):
    //   itype 1 (A v = w B v):             C = inv(L) A inv(L)^H
    //   itype 2, 3 (A B v = w v, B A v = w v): C = L^H A L
    // A's lower triangle is read and overwritten by C's.  Both run by T-blocks
    // with their bulk in rank-2k products on the trailing-update kernel; the
    // flop count is that of the unblocked definition's symmetric form, n^3.
    static int gst(int itype, int64_t n, E *A, int64_t lda, const E *Lb, int64_t ldl, int64_t T_A, const int *info,
                   void *work, hipStream_t s)
    {
        if (n == 0)
            return 0;
        const GstLayout G = make_gst_layout(itype, n, T_A, sizeof(E));
        E *M = (E *)work + G.m;
        SPD_TRY(herm_full(A, lda, M, n, n, s));
        if (itype == 1)
            SPD_TRY(gst1(n, M, Lb, ldl, T_A, G, info, work, s));
        else
            SPD_TRY(gst23(n, M, Lb, ldl, G, info, work, s));
        const int64_t blocks = std::min<int64_t>(cdiv(n * n, 256), 8192);
        SPD_VALIDATE(check_copy_lower<E>(A, lda, M, n, n, info, g_chk));
        copy_lower_kernel<R, CPLX><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(A, lda, M, n, n, info);
        SPD_CHECK_LAUNCH("copy_lower_kernel");
        return 0;
    }

    // D (n x n, ldd) = the full Hermitian matrix whose lower triangle is in S
    static int herm_full(const E *S, int64_t lds, E *D, int64_t ldd, int64_t n, hipStream_t s)
    {
        const int64_t tt = cdiv(n, 32), pairs = tt * (tt + 1) / 2;  // 32 x 32 tile pairs
        SPD_VALIDATE(check_expand<E>("herm_full_kernel", S, lds, D, ldd, n, true, g_chk));
        herm_full_kernel<R, CPLX><<<dim3((unsigned)pairs), dim3(256), 0, s>>>(S, lds, D, ldd, n);
        SPD_CHECK_LAUNCH("herm_full_kernel");
        return 0;
    }

    // Type 1, right-looking by T-blocks.  With the leading block split off and
    // W11 = inv(L11):
    //   C11 = W11 A11 W11^H,  Y = A21 W11^H,  Z = Y - L21 C11 / 2,
    //   A22 <- A22 - Z L21^H - L21 Z^H       (then reduced the same way),
    //   C21 = inv(L22) (Y - L21 C11).
    // Y - L21 C11 is kept in place of A21; the solves by the trailing factors
    // L22 of every step are one forward substitution at the end, of the block
    // strictly-lower part (block row r non-zero in columns [0, rT) only).
    static int gst1(int64_t n, E *M, const E *Lb, int64_t ldl, int64_t T_A, const GstLayout &G, const int *info,
                    void *work, hipStream_t s)
    {
        const Layout SL = make_layout(n, n, T_A, sizeof(E));
        const int64_t T = SL.T, nt = SL.nt, kh = align_up(T, SYRK_KP);
        E *sw = (E *)work + G.solve;
        E *Inv = sw + SL.inv;
        E *P[2] = {(E *)work + G.p, (E *)work + G.p2}, *Q[2] = {(E *)work + G.q, (E *)work + G.q2};
        E *Y = (E *)work + G.y, *V = (E *)work + G.v;
        E *D = (E *)work + G.d, *T1 = (E *)work + G.t1;
        SPD_TRY(all_inverses(n, Lb, ldl, T, nt, Inv, sw + SL.w, info, s));
        // block k's diagonal C_kk (from its current lower triangle) and, below
        // it, Y - L21 C_kk back into M and the rank-2k operands into P[q], Q[q]
        auto prep = [&](int64_t k, int q, hipStream_t st) -> int {
            const int64_t c0 = k * T, tk = std::min(T, n - c0), r0 = c0 + tk, m = n - r0;
            E *Mkk = M + c0 + c0 * n;
            const E *Wk = Inv + k * T * T;
            SPD_TRY(herm_full(Mkk, n, D, T, tk, st));
            Gemm g1;  // T1 = W11 A11
            g1.A = Wk;
            g1.lda = T;
            g1.B = D;
            g1.ldb = T;
            g1.C = T1;
            g1.ldc = T;
            g1.m = g1.n = g1.k = tk;
            g1.kmode = KM_END_BY_I;
            g1.info = info;
            g1.small = true;
            SPD_TRY((gemm<R, CPLX>(NN, g1, st)));
            Gemm g2;  // C11 = T1 W11^H, the whole tile
            g2.A = T1;
            g2.lda = T;
            g2.B = Wk;
            g2.ldb = T;
            g2.C = Mkk;
            g2.ldc = n;
            g2.m = g2.n = g2.k = tk;
            g2.kmode = KM_END_BY_J;
            g2.info = info;
            g2.small = true;
            SPD_TRY((gemm<R, CPLX>(NT, g2, st)));
            if (m <= 0)
                return 0;
            Gemm g3;  // Y = A21 W11^H
            g3.A = M + r0 + c0 * n;
            g3.lda = n;
            g3.B = Wk;
            g3.ldb = T;
            g3.C = Y;
            g3.ldc = n;
            g3.m = m;
            g3.n = g3.k = tk;
            g3.kmode = KM_END_BY_J;
            g3.info = info;
            SPD_TRY((gemm<R, CPLX>(NT, g3, st)));
            Gemm g4;  // V = L21 C11
            g4.A = Lb + r0 + c0 * ldl;
            g4.lda = ldl;
            g4.B = Mkk;
            g4.ldb = n;
            g4.C = V;
            g4.ldc = n;
            g4.m = m;
            g4.n = g4.k = tk;
            g4.info = info;
            SPD_TRY((gemm<R, CPLX>(NN, g4, st)));
            const int64_t ldw = align_up(m, SYRK_LDW);
            SPD_VALIDATE(check_gst_pack<E>(Y, n, V, n, Lb + r0 + c0 * ldl, ldl, P[q], Q[q], ldw, M + r0 + c0 * n, n,
                                           m, tk, kh, g_chk));
            const int64_t pb = std::min<int64_t>(cdiv(ldw * kh, 256), 8192);
            gst_pack_kernel<R, CPLX><<<dim3((unsigned)pb), dim3(256), 0, st>>>(
                Y, n, V, n, Lb + r0 + c0 * ldl, ldl, P[q], Q[q], ldw, M + r0 + c0 * n, n, m, tk, kh);
            SPD_CHECK_LAUNCH("gst_pack_kernel");
            return 0;
        };
        // A22 -= P Q^H = Z L21^H + L21 Z^H over rows and columns from r (a
        // multiple of T past the block's end; cols > 0: that many columns only)
        auto update = [&](int64_t k, int q, int64_t r, int64_t cols, int cls, hipStream_t st) -> int {
            const int64_t c0 = k * T, tk = std::min(T, n - c0), r0 = c0 + tk, m = n - r;
            if (m <= 0)
                return 0;
            const int64_t w = cols > 0 ? std::min(cols, m) : m;
            ProfScope ps(cls, FMUL * (double)w * (2.0 * m - w + 1.0) * 2.0 * tk, st);
            Syr2 x;
            x.V = Q[q] + (r - r0);
            return syrk(m, P[q] + (r - r0), align_up(n - r0, SYRK_LDW), 2 * kh, 2 * tk, M + r + r * n, n, cols, info,
                        st, x);
        };
        const bool ahead = lookahead_enabled() && T % syrk_bm() == 0 && nt >= 3;
        if (!ahead) {
            for (int64_t k = 0; k < nt; ++k) {
                SPD_TRY(prep(k, 0, s));
                SPD_TRY(update(k, 0, std::min(n, (k + 1) * T), 0, PROF_SYRK, s));
            }
        } else {
            // one step ahead on the auxiliary stream, as in potrf: tile column
            // k+1 by block k's operands, then block k+1's preparation into the
            // other operand buffers; the caller's stream updates the rest
            Lookahead la;
            SPD_TRY(la.begin(s));
            hipStream_t sl = la.look;
            SPD_TRY(prep(0, 0, sl));
            SPD_TRY(la.record(la.ev_panel, sl));
            int q = 0;
            for (int64_t k = 0; k + 1 < nt; ++k) {
                const int64_t r0 = (k + 1) * T;
                SPD_TRY(la.wait(s, la.ev_panel));  // operands of block k
                if (k > 0)
                    SPD_TRY(la.wait(sl, la.ev_rest));  // the update of step k-1 reached tile column k+1
                SPD_TRY(update(k, q, r0, T, PROF_SYRK_AUX, sl));
                SPD_TRY(prep(k + 1, q ^ 1, sl));
                SPD_TRY(la.record(la.ev_panel, sl));
                SPD_TRY(update(k, q, r0 + T, 0, PROF_SYRK, s));
                SPD_TRY(la.record(la.ev_rest, s));
                q ^= 1;
            }
            SPD_TRY(la.wait(s, la.ev_panel));  // join: the last block's C_kk
        }
        // C21 blocks: the forward substitution of the block strictly-lower part
        if (rect_usable(ldl)) {
            E *lp[2] = {P[0], Q[0]};  // the rank-2k panels are free now; each holds ldq x kq
            return potrs_blocks(n, n, Lb, ldl, M, n, SL, info, sw, s, false, true, lp);
        }
        return potrs_general(n, n, Lb, ldl, M, n, SL, info, sw, s, false, true);
    }

    // D (ldw x halves*kh) <- zero-padded column panels [S0 | S1] (rows [0, m),
    // tk columns each)
    static int panel_pack(const E *S0, int64_t ld0, const E *S1, int64_t ld1, E *D, int64_t ldw, int64_t m,
                          int64_t tk, int64_t kh, int halves, hipStream_t s)
    {
        SPD_VALIDATE(check_panel_pack<E>(S0, ld0, S1, ld1, D, ldw, m, tk, kh, halves, g_chk));
        const int64_t blocks = std::min<int64_t>(cdiv(ldw * kh * halves, 256), 8192);
        panel_pack_kernel<R, CPLX><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(S0, ld0, S1, ld1, D, ldw, m, tk, kh,
                                                                               halves);
        SPD_CHECK_LAUNCH("panel_pack_kernel");
        return 0;
    }

    // Types 2 and 3 (C = L^H A L) by T-blocks.  For block row k (p = kT columns
    // before it) let a21 = A(k, 0:p), l21 = L(k, 0:p), a22 = A_kk, l22 = L_kk
    // and
    //   w_k = a21 L(0:p, 0:p) + a22 l21 / 2.
    // Then C(k, 0:p) receives l22^H (w_k + a22 l21 / 2), C_kk receives
    // l22^H a22 l22, and the leading p x p block receives w_k^H l21 + l21^H w_k.
    // The first terms of all w_k together are Gsb L (Gsb the block
    // strictly-lower part of A), accumulated right-looking one depth block at
    // a time; the leading-block terms are one rank-2k update per block row.
    static int gst23(int64_t n, E *M, const E *Lb, int64_t ldl, const GstLayout &G, const int *info, void *work,
                     hipStream_t s)
    {
        const int64_t T = G.T, nt = G.nt, ldg = G.ldg, nfull = n / T, kh = align_up(T, SYRK_KP);
        E *P = (E *)work + G.p, *Q = (E *)work + G.q, *LH = (E *)work + G.lh, *Wf = (E *)work + G.wf;
        E *Ld = (E *)work + G.ld, *T1 = (E *)work + G.t1, *Vb = (E *)work + G.v, *Xb = (E *)work + G.y;
        SPD_VALIDATE(check_gst_diag_tril<E>(Lb, ldl, Ld, n, T, nt, g_chk));
        gst_diag_tril_kernel<R, CPLX><<<dim3((unsigned)std::min<int64_t>(cdiv(nt * T * T, 256), 8192)), dim3(256), 0,
                                        s>>>(Lb, ldl, Ld, n, T, nt);
        SPD_CHECK_LAUNCH("gst_diag_tril_kernel");
        SPD_VALIDATE(check_gst_lh<E>(Lb, ldl, LH, ldg, n, g_chk));
        const int64_t tg = ldg / 32;  // 32 x 32 tile pairs of the padded square
        gst_lh_kernel<R, CPLX><<<dim3((unsigned)(tg * (tg + 1) / 2)), dim3(256), 0, s>>>(Lb, ldl, LH, ldg, n, T, 0);
        SPD_CHECK_LAUNCH("gst_lh_kernel");
        SPD_TRY(zero2d<E>(Wf, ldg, ldg, ldg, s));
        // Wf(r0:n, 0:r0) += A(r0:n, block kk) L(block kk, 0:r0), r0 = (kk+1)T
        for (int64_t kk = 0; kk + 1 < nt; ++kk) {
            const int64_t r0 = (kk + 1) * T, m = n - r0, ldw = align_up(std::max(m, r0), SYRK_LDW);
            SPD_TRY(panel_pack(M + r0 + kk * T * n, n, nullptr, 0, P, ldw, m, T, kh, 1, s));
            SPD_TRY(panel_pack(LH + kk * T * ldg, ldg, nullptr, 0, Q, ldw, r0, T, kh, 1, s));
            ProfScope ps(PROF_SYRK, FMUL * 2.0 * (double)m * r0 * T, s);
            SPD_TRY(rect_update(m, r0, P, Q, ldw, kh, Wf + r0, ldg, true, info, s));
        }
        // block rows k >= 1: V = a22 l21, w_k += V/2, X = w_k + V/2, C(k, 0:p) = l22^H X
        for (int64_t k = 1; k < nt; ++k) {
            const int64_t c0 = k * T, tk = std::min(T, n - c0);
            Gemm g;
            g.A = M + c0 + c0 * n;
            g.lda = n;
            g.B = Lb + c0;
            g.ldb = ldl;
            g.C = Vb;
            g.ldc = T;
            g.m = tk;
            g.n = c0;
            g.k = tk;
            g.info = info;
            SPD_TRY((gemm<R, CPLX>(NN, g, s)));
            SPD_VALIDATE(check_gst_half<E>(Wf + c0, ldg, Vb, Xb, T, tk, c0, g_chk));
            gst_half_kernel<R, CPLX><<<dim3((unsigned)std::min<int64_t>(cdiv(tk * c0, 256), 8192)), dim3(256), 0, s>>>(
                Wf + c0, ldg, Vb, Xb, T, tk, c0);
            SPD_CHECK_LAUNCH("gst_half_kernel");
            Gemm h;
            h.A = Ld + k * T * T;
            h.lda = T;
            h.B = Xb;
            h.ldb = T;
            h.C = M + c0;
            h.ldc = n;
            h.m = tk;
            h.n = c0;
            h.k = tk;
            h.kmode = KM_BEG_BY_I;
            h.info = info;
            SPD_TRY((gemm<R, CPLX>(TN, h, s)));
        }
        // diagonal blocks: C_kk = l22^H (a22 l22), whole blocks batched, then the ragged one
        auto diag = [&](int64_t k0, int64_t cnt, int64_t tk) -> int {
            const int64_t c0 = k0 * T;
            Gemm g;
            g.A = M + c0 + c0 * n;
            g.lda = n;
            g.sA_out = T * (1 + n);
            g.B = Ld + k0 * T * T;
            g.ldb = T;
            g.sB_out = T * T;
            g.C = T1;
            g.ldc = T;
            g.sC_out = T * T;
            g.batch = (int)cnt;
            g.m = g.n = g.k = tk;
            g.kmode = KM_BEG_BY_J;
            g.info = info;
            SPD_TRY((gemm<R, CPLX>(NN, g, s)));
            Gemm h;
            h.A = Ld + k0 * T * T;
            h.lda = T;
            h.sA_out = T * T;
            h.B = T1;
            h.ldb = T;
            h.sB_out = T * T;
            h.C = M + c0 + c0 * n;
            h.ldc = n;
            h.sC_out = T * (1 + n);
            h.batch = (int)cnt;
            h.m = h.n = h.k = tk;
            h.kmode = KM_BEG_BY_I;
            h.info = info;
            return gemm<R, CPLX>(TN, h, s);
        };
        if (nfull > 0)
            SPD_TRY(diag(0, nfull, T));
        if (nfull < nt)
            SPD_TRY(diag(nfull, 1, n - nfull * T));
        // Wf^H in place: block column k of it is w_k^H (rows [0, kT))
        const int64_t tt = cdiv(n, 32), pairs = tt * (tt + 1) / 2;
        SPD_VALIDATE(check_conj_transpose<E>(Wf, ldg, n, (unsigned)pairs, info, g_chk));
        conj_transpose_kernel<R, CPLX><<<dim3((unsigned)pairs), dim3(256), 0, s>>>(Wf, ldg, n, info);
        SPD_CHECK_LAUNCH("conj_transpose_kernel");
        // C(0:p, 0:p) += w_k^H l21 + l21^H w_k = P Q^H with P = [w_k^H | l21^H],
        // Q = [l21^H | w_k^H] (l21^H is block column k of L^H, rows [0, p))
        for (int64_t k = 1; k < nt; ++k) {
            const int64_t p = k * T, tk = std::min(T, n - p), ldw = align_up(p, SYRK_LDW);
            SPD_TRY(panel_pack(Wf + p * ldg, ldg, LH + p * ldg, ldg, P, ldw, p, tk, kh, 2, s));
            SPD_TRY(panel_pack(LH + p * ldg, ldg, Wf + p * ldg, ldg, Q, ldw, p, tk, kh, 2, s));
            ProfScope ps(PROF_SYRK, FMUL * 2.0 * (double)p * (p + 1) * tk, s);
            Syr2 x;
            x.V = Q;
            x.add = true;
            SPD_TRY(syrk(p, P, ldw, 2 * kh, 2 * tk, M, n, 0, info, s, x));
        }
        return 0;
    }

    // prefix (forward only): block row r of B has non-zero columns [0, r T)
    // only and the rest of it is left alone (see potrs_blocks).
    // forward = false (the fused solve): only L^H X = B, with the tile
    // inverses already in the workspace.
    static int potrs_general(int64_t n, int64_t nrhs, const E *A, int64_t lda, E *B, int64_t ldb, const Layout &L,
                             const int *info, void *work, hipStream_t s, bool backward, bool prefix = false,
                             bool forward = true)
    {
        const int64_t T = L.T, nt = L.nt;
        E *Inv = (E *)work + L.inv;
        E *Tmp = (E *)work + L.tmp;  // T x nrhs, ld T
        if (forward)
            SPD_TRY(all_inverses(n, A, lda, T, nt, Inv, (E *)work + L.w, info, s));
        // forward: L Y = B
        for (int64_t k = 0; forward && k < nt; ++k) {
            const int64_t c0 = k * T, tk = std::min(T, n - c0), m = n - c0 - tk;
            const int64_t nc = prefix ? std::min(nrhs, c0) : nrhs;  // columns of block row k
            if (nc <= 0)
                continue;
            SPD_TRY(apply_inv(Inv, k, T, B, ldb, c0, tk, nc, Tmp, false, info, s));
            SPD_TRY(copy2d<E>(B + c0, ldb, Tmp, T, tk, nc, info, s));
            if (m > 0) {
                Gemm u;  // B_below -= L_panel Y_k
                u.A = A + (c0 + tk) + c0 * lda;
                u.lda = lda;
                u.B = Tmp;
                u.ldb = T;
                u.C = B + c0 + tk;
                u.ldc = ldb;
                u.m = m;
                u.n = nc;
                u.k = tk;
                u.neg = true;
                u.beta = true;
                u.info = info;
                SPD_TRY((gemm<R, CPLX>(NN, u, s)));
            }
        }
        if (!backward)
            return 0;
        // backward: L^H X = Y
        for (int64_t k = nt - 1; k >= 0; --k) {
            const int64_t c0 = k * T, tk = std::min(T, n - c0);
            SPD_TRY(apply_inv(Inv, k, T, B, ldb, c0, tk, nrhs, Tmp, true, info, s));
            SPD_TRY(copy2d<E>(B + c0, ldb, Tmp, T, tk, nrhs, info, s));
            if (c0 > 0) {
                Gemm u;  // Y_top -= L_k,0:k^H X_k
                u.A = A + c0;
                u.lda = lda;
                u.B = Tmp;
                u.ldb = T;
                u.C = B;
                u.ldc = ldb;
                u.m = c0;
                u.n = nrhs;
                u.k = tk;
                u.neg = true;
                u.beta = true;
                u.info = info;
                SPD_TRY((gemm<R, CPLX>(TN, u, s)));
            }
        }
        return 0;
    }

    // Block substitutions on the block-update kernel (real types), one block
    // ahead on the auxiliary stream when there are at least three blocks:
    //
    //   chain (auxiliary stream): update the next block's rows with the block
    //     just solved, solve the next block (inverse product), write it back
    //     into B and, transposed, into one of two operand buffers;
    //   caller's stream: update every row beyond the next block with the block
    //     just solved.
    //
    // Events: the caller's stream waits for the operand buffer of block k
    // before its update; the chain waits for the caller's update of step k-1
    // before it touches the next block's rows (which that update wrote) and
    // before it overwrites the operand buffer that update read.  The back
    // substitution runs the same way from the last block up.
    //
    // prefix (forward only; the second substitution of the type-1 reduction):
    // block row r of B is non-zero in columns [0, r T) only and its other
    // columns (the diagonal block and the rest) are left alone; step k then
    // updates and solves only the columns block k's solution can reach.
    //
    // lp (forward only, nrhs >= n): two buffers of L.ldq x L.kq elements; each
    // step's panel of L is packed into one of them, zero padded, and the block
    // updates run on the trailing-update kernel's rectangular mode (wide
    // right-hand sides).
    //
    // forward = false (the fused solve): only L^H X = B, with the tile
    // inverses and the chain products GB_k already in the workspace.
    static int potrs_blocks(int64_t n, int64_t nrhs, const E *A, int64_t lda, E *B, int64_t ldb, const Layout &L,
                            const int *info, void *work, hipStream_t s, bool backward, bool prefix = false,
                            E *const *lp = nullptr, bool forward = true)
    {
        if (lp != nullptr && (backward || nrhs < n)) {
            g_last_error = "packed-panel block update is for the forward substitution with nrhs >= n";
            return SPD_ERR_HIP;
        }
        if (prefix && backward) {
            g_last_error = "column-prefix substitution is forward only";
            return SPD_ERR_HIP;
        }
        const int64_t T = L.T, nt = L.nt;
        E *Inv = (E *)work + L.inv;
        E *Tmp = (E *)work + L.tmp;
        E *Qb[2] = {(E *)work + L.q, (E *)work + L.q + L.qsz};
        E *GF = (E *)work + L.gf, *GB = (E *)work + L.gb, *Part = (E *)work + L.part;
        const bool vec = rect_vec(A, lda, T);
        if (forward)
            SPD_TRY(all_inverses(n, A, lda, T, nt, Inv, (E *)work + L.w, info, s));
        SPD_TRY(zero2d<E>(Qb[0], L.ldq, L.ldq, 2 * L.kq, s));  // both buffers (adjacent, same ld)
        const int64_t nfull = n / T;  // whole blocks
        // split chain: depth split of each operand pair, sh parts of ks
        const int64_t sh = (T % 4 == 0 && T >= 64) ? 4 : (T % 2 == 0 && T >= 32) ? 2 : 1, ks = T / sh;
        const bool split = nfull >= 2 && !prefix;
        auto cols = [&](int64_t r) { return prefix ? std::min(nrhs, r * T) : nrhs; };  // columns of block row r
        if (split && forward) {
            // GF_k = -inv(L_k+1,k+1) L_k+1,k for whole blocks k+1 (k = 0 .. nfull-2)
            Gemm g;
            g.A = Inv + T * T;
            g.lda = T;
            g.sA_out = T * T;
            g.B = A + T;
            g.ldb = lda;
            g.sB_out = T * (1 + lda);
            g.C = GF;
            g.ldc = T;
            g.sC_out = T * T;
            g.batch = (int)(nfull - 1);
            g.m = g.n = g.k = T;
            g.kmode = KM_END_BY_I;
            g.neg = true;
            g.info = info;
            SPD_TRY((gemm<R, CPLX>(NN, g, s)));
        }
        if (split && backward && forward)  // GB_k for whole blocks k (k = 1 .. nfull-1)
            SPD_TRY(back_chain_products(n, A, lda, T, Inv, GB, false, info, s));
        // Next block (index kn, rows [cn, cn + T)) in one split product:
        //   forward:  Y_kn = GF_k Y_k + inv(L_kn,kn) B_kn          (kn = k + 1)
        //   backward: X_kn = inv(L_kn,kn)^T B_kn + GB_k^T X_k      (kn = k - 1)
        // as 2*sh partial products of depth ks, then their fixed-order sum,
        // written back into B and, transposed, into operand buffer q.
        auto chain = [&](int64_t k, int64_t kn, bool back, int q, hipStream_t st) -> int {
            const int64_t c0 = k * T, cn = kn * T;
            Gemm g;
            const E *A0 = back ? Inv + kn * T * T : GF + k * T * T;  // pairs with B rows c0 (fwd) / cn (bwd)
            const E *A1 = back ? GB + k * T * T : Inv + kn * T * T;
            g.A = A0;
            g.lda = T;
            g.sA_out = (int64_t)(A1 - A0);
            g.sA_in = back ? ks : ks * T;
            g.B = B + std::min(c0, cn);
            g.ldb = ldb;
            g.sB_out = T;
            g.sB_in = ks;
            g.C = Part;
            g.ldc = T;
            g.sC_out = sh * T * nrhs;
            g.sC_in = T * nrhs;
            g.nb_inner = (int)sh;
            g.batch = (int)(2 * sh);
            g.m = T;
            g.n = nrhs;
            g.k = ks;
            g.small = true;
            g.info = info;
            SPD_TRY((back ? gemm<R, CPLX>(TN, g, st) : gemm<R, CPLX>(NN, g, st)));
            if constexpr (CPLX) {
                g_last_error = "split substitution chain is for real types";
                return SPD_ERR_HIP;
            } else {
                const int64_t kp = align_up(T, RECT_KB);
                SPD_VALIDATE((check_reduce_copy_t<E>(B + cn, ldb, Qb[q], L.ldq, Part, T, T * nrhs, (int)(2 * sh), T,
                                                      nrhs, kp, info, g_chk)));
                const int64_t blocks = std::min<int64_t>(cdiv(kp * nrhs, 256), 4096);
                reduce_copy_t_kernel<E><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
                    B + cn, ldb, Qb[q], L.ldq, Part, T, T * nrhs, (int)(2 * sh), T, nrhs, kp, info);
                SPD_CHECK_LAUNCH("reduce_copy_t_kernel");
                return 0;
            }
        };
        // With packed panels (wide right-hand sides) every product fills the GPU
        // by itself, and the next block's inverse product, run beside the
        // update, would only get the CUs the update leaves: one stream.
        const bool ahead = lookahead_enabled() && nt >= 3 && lp == nullptr;
        Lookahead la;
        hipStream_t sl = s;
        if (ahead) {
            SPD_TRY(la.begin(s));
            sl = la.look;
        }
        auto rec = [&](hipEvent_t ev, hipStream_t st) { return ahead ? la.record(ev, st) : 0; };
        auto wait = [&](hipStream_t st, hipEvent_t ev) { return ahead ? la.wait(st, ev) : 0; };
        int qi = 0;  // operand buffer of the block being applied
        // solve block k (inverse product), write it back and transpose it into Qb[q]
        auto solve_block = [&](int64_t k, bool trans, int q, hipStream_t st) -> int {
            const int64_t c0 = k * T, tk = std::min(T, n - c0), nc = cols(k);
            SPD_TRY(apply_inv(Inv, k, T, B, ldb, c0, tk, nc, Tmp, trans, info, st));
            return copy_t(B + c0, ldb, Qb[q], L.ldq, Tmp, T, tk, nc, align_up(tk, RECT_KB), info, st);
        };
        // B(rows r, r + h) -= L(same rows, block k) Y_k, Y_k transposed in Qb[qi]
        auto update = [&](int64_t k, int64_t r, int64_t h, int q, hipStream_t st) -> int {
            const int64_t c0 = k * T, tk = std::min(T, n - c0), kp = align_up(tk, RECT_KB);
            if (lp != nullptr)  // panel packed at rows r0 = c0 + tk onwards
                return rect_update(h, cols(k), lp[q] + (r - c0 - tk), Qb[q], L.ldq, L.kq, B + r, ldb, false, info,
                                   st);
            return rect<false>(A + r + c0 * lda, lda, Qb[q], L.ldq, B + r, ldb, h, cols(k), kp, tk, vec, info, st);
        };
        // the panel of L below block k, packed into lp[q] (on the chain stream,
        // before the event the caller's stream waits on for step k)
        auto pack_panel = [&](int64_t k, int q, hipStream_t st) -> int {
            const int64_t c0 = k * T, r0 = c0 + std::min(T, n - c0);
            if (lp == nullptr || r0 >= n)
                return 0;
            return panel_pack(A + r0 + c0 * lda, lda, nullptr, 0, lp[q], L.ldq, n - r0, std::min(T, n - c0), L.kq, 1,
                              st);
        };
        // ---- forward: L Y = B
        if (forward) {
        SPD_TRY(solve_block(0, false, qi, sl));
        SPD_TRY(pack_panel(0, qi, sl));
        SPD_TRY(rec(la.ev_panel, sl));
        for (int64_t k = 0; k < nt; ++k) {
            const int64_t c0 = k * T, tk = std::min(T, n - c0), r0 = c0 + tk, m = n - r0;
            SPD_TRY(wait(s, la.ev_panel));  // Y_k in Qb[qi]
            if (m <= 0)
                break;
            if (lp != nullptr) {  // one stream: all rows below block k at once, then block k+1
                SPD_TRY(update(k, r0, m, qi, s));
                SPD_TRY(solve_block(k + 1, false, qi ^ 1, s));
                SPD_TRY(pack_panel(k + 1, qi ^ 1, s));
                qi ^= 1;
                continue;
            }
            const int64_t t1 = std::min(T, m);  // rows of block k+1
            if (k > 0)  // step k-1's update wrote block k+1 and read Qb[qi^1] and lp[qi^1]
                SPD_TRY(wait(sl, la.ev_rest));
            if (split && k + 1 < nfull) {
                SPD_TRY(chain(k, k + 1, false, qi ^ 1, sl));
            } else {
                SPD_TRY(update(k, r0, t1, qi, sl));
                SPD_TRY(solve_block(k + 1, false, qi ^ 1, sl));
            }
            SPD_TRY(pack_panel(k + 1, qi ^ 1, sl));
            SPD_TRY(rec(la.ev_panel, sl));
            if (m > t1)
                SPD_TRY(update(k, r0 + t1, m - t1, qi, s));
            SPD_TRY(rec(la.ev_rest, s));
            qi ^= 1;
        }
        }
        if (!backward)
            return 0;
        // ---- backward: L^H X = Y, from the last block up
        if (forward)
            SPD_TRY(wait(sl, la.ev_rest));  // every forward update is done
        qi ^= 1;
        SPD_TRY(solve_block(nt - 1, true, qi, sl));
        SPD_TRY(rec(la.ev_panel, sl));
        for (int64_t k = nt - 1; k >= 0; --k) {
            const int64_t c0 = k * T, tk = std::min(T, n - c0), kp = align_up(tk, RECT_KB);
            SPD_TRY(wait(s, la.ev_panel));  // X_k in Qb[qi]
            if (k == 0)
                break;
            const int64_t cp = c0 - T;  // block k-1 is rows [cp, c0)
            SPD_TRY(wait(sl, la.ev_rest));
            if (split && k < nfull) {
                SPD_TRY(chain(k, k - 1, true, qi ^ 1, sl));
            } else {
                SPD_TRY(rect<true>(A + c0 + cp * lda, lda, Qb[qi], L.ldq, B + cp, ldb, T, nrhs, kp, tk, vec, info,
                                   sl));
                SPD_TRY(solve_block(k - 1, true, qi ^ 1, sl));
            }
            SPD_TRY(rec(la.ev_panel, sl));
            if (cp > 0)
                SPD_TRY(rect<true>(A + c0, lda, Qb[qi], L.ldq, B, ldb, cp, nrhs, kp, tk, vec, info, s));
            SPD_TRY(rec(la.ev_rest, s));
            qi ^= 1;
        }
        return 0;
    }

    static int nan_fill(int64_t n, int64_t nrhs, E *B, int64_t ldb, const int *info, hipStream_t s)
    {
        SPD_VALIDATE(check_2d<E>("nan_fill_kernel", B, ldb, (const E *)nullptr, 0, n, nrhs, info, g_chk));
        const int64_t blocks = std::min<int64_t>(cdiv(n * nrhs, 256), 4096);
        nan_fill_kernel<R, CPLX><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(B, ldb, n, nrhs, info);
        SPD_CHECK_LAUNCH("nan_fill_kernel");
        return 0;
    }

    static int logdet(int64_t n, const E *A, int64_t lda, const int *info, double *out, hipStream_t s)
    {
        SPD_VALIDATE(check_2d<E>("logdet_kernel", (E *)nullptr, 0, A, lda + 1, 1, n, info, g_chk) &&
                     g_chk.access(out, sizeof(double), true, "logdet_kernel", 0, 0));
        logdet_kernel<R, CPLX><<<1, 1024, 0, s>>>(A, lda, n, info, out);
        SPD_CHECK_LAUNCH("logdet_kernel");
        return 0;
    }
};

static int64_t elem_size(int dt)
{
    switch (dt) {
    case SPD_R32: return 4;
    case SPD_R64: return 8;
    case SPD_C64: return 8;
    case SPD_C128: return 16;
    default: return 0;
    }
}

// Bytes spanned by an m x n column-major matrix with leading dimension ld
// (the last column needs only m rows).
static size_t matrix_bytes(int dt, int64_t m, int64_t n, int64_t ld)
{
    if (m <= 0 || n <= 0)
        return 0;
    return (size_t)(((n - 1) * ld + m) * elem_size(dt));
}

// ------------------------------------------------ fixed scratch buffer ---
// spd_posv_noalloc takes its workspace from this array instead of from the
// caller.  Each device the library runs on holds its own copy from the time
// the library's code is loaded there until the process ends.  Host code never
// passes the array's name to a kernel (on the host it only names a stand-in):
// the device address of each device's copy comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// used.
static __device__ __align__(256) unsigned char scratch[SPD_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static std::vector<std::pair<int, void *>> g_scratch_addr;  // (device, address of its copy)

// Address of the current device's copy of `scratch` (a fixed stand-in in a
// dry run, which makes no HIP calls and dereferences nothing).
static int scratch_address(void **out)
{
    if (g_validate == 2) {
        *out = (void *)(uintptr_t)(UINT64_C(0x7e0000000000));
        return 0;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> g(g_scratch_mu);
    for (auto &d : g_scratch_addr)
        if (d.first == dev) {
            *out = d.second;
            return 0;
        }
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || (uintptr_t)p % 256 != 0) {
        g_last_error = "hipGetSymbolAddress(scratch): unexpected address";
        return SPD_ERR_HIP;
    }
    g_scratch_addr.emplace_back(dev, p);
    *out = p;
    return 0;
}

}  // namespace spd

using namespace spd;

extern "C" {

size_t spd_workspace_size(spd_dtype_t dt, int64_t n, int64_t n_rhs, int64_t T_A)
{
    const int64_t es = elem_size(dt);
    if (es == 0 || n < 0 || n_rhs < 0 || T_A < 1 || n == 0)
        return 0;
    return (size_t)(make_layout(n, n_rhs, T_A, es).total * es);
}

int spd_potrf(spd_dtype_t dt, int64_t n, void *dA, int64_t lda, int64_t T_A, int32_t *d_info, void *d_work,
              size_t work_bytes, void *stream)
{
    if (elem_size(dt) == 0) return -1;
    if (n < 0 || n > INT32_MAX) return -2;
    if (dA == nullptr && n > 0) return -3;
    if (lda < std::max<int64_t>(1, n)) return -4;
    if (T_A < 1) return -5;
    if (d_info == nullptr) return -6;
    const size_t need = spd_workspace_size(dt, n, 0, T_A);
    if (d_work == nullptr && need > 0) return -7;
    if (work_bytes < need) return -8;
    if (g_validate) {
        g_chk.begin();
        g_chk.add(dA, matrix_bytes(dt, n, n, lda), true, "A");
        g_chk.add(d_info, 4, true, "info");
        g_chk.add(d_work, work_bytes, true, "workspace");
    }
    snapshot_options();
    hipStream_t s = (hipStream_t)stream;
    switch (dt) {
    case SPD_R32: return Solver<float, false>::potrf(n, (float *)dA, lda, T_A, d_info, d_work, s);
    case SPD_R64: return Solver<double, false>::potrf(n, (double *)dA, lda, T_A, d_info, d_work, s);
    case SPD_C64:
        return Solver<float, true>::potrf(n, (Elem<float, true>::type *)dA, lda, T_A, d_info, d_work, s);
    case SPD_C128:
        return Solver<double, true>::potrf(n, (Elem<double, true>::type *)dA, lda, T_A, d_info, d_work, s);
    }
    return -1;
}

int spd_potrs(spd_dtype_t dt, int64_t n, int64_t n_rhs, const void *dA, int64_t lda, void *dB, int64_t ldb,
              int64_t T_A, const int32_t *d_info, void *d_work, size_t work_bytes, void *stream)
{
    if (elem_size(dt) == 0) return -1;
    if (n < 0 || n > INT32_MAX) return -2;
    if (n_rhs < 0 || n_rhs > INT32_MAX) return -3;
    if (dA == nullptr && n > 0) return -4;
    if (lda < std::max<int64_t>(1, n)) return -5;
    if (dB == nullptr && n > 0 && n_rhs > 0) return -6;
    if (ldb < std::max<int64_t>(1, n)) return -7;
    if (T_A < 1) return -8;
    const size_t need = spd_workspace_size(dt, n, n_rhs, T_A);
    if (d_work == nullptr && need > 0) return -10;
    if (work_bytes < need) return -11;
    if (g_validate) {
        g_chk.begin();
        g_chk.add(dA, matrix_bytes(dt, n, n, lda), false, "L");
        g_chk.add(dB, matrix_bytes(dt, n, n_rhs, ldb), true, "B");
        g_chk.add(d_info, 4, false, "info");
        g_chk.add(d_work, work_bytes, true, "workspace");
    }
    snapshot_options();
    hipStream_t s = (hipStream_t)stream;
    switch (dt) {
    case SPD_R32:
        return Solver<float, false>::potrs(n, n_rhs, (const float *)dA, lda, (float *)dB, ldb, T_A, d_info, d_work, s);
    case SPD_R64:
        return Solver<double, false>::potrs(n, n_rhs, (const double *)dA, lda, (double *)dB, ldb, T_A, d_info,
                                            d_work, s);
    case SPD_C64:
        return Solver<float, true>::potrs(n, n_rhs, (const Elem<float, true>::type *)dA, lda,
                                          (Elem<float, true>::type *)dB, ldb, T_A, d_info, d_work, s);
    case SPD_C128:
        return Solver<double, true>::potrs(n, n_rhs, (const Elem<double, true>::type *)dA, lda,
                                           (Elem<double, true>::type *)dB, ldb, T_A, d_info, d_work, s);
    }
    return -1;
}

int spd_forward_solve(spd_dtype_t dt, int64_t n, int64_t n_rhs, const void *dA, int64_t lda, void *dB, int64_t ldb,
                      int64_t T_A, const int32_t *d_info, void *d_work, size_t work_bytes, void *stream)
{
    if (elem_size(dt) == 0) return -1;
    if (n < 0 || n > INT32_MAX) return -2;
    if (n_rhs < 0 || n_rhs > INT32_MAX) return -3;
    if (dA == nullptr && n > 0) return -4;
    if (lda < std::max<int64_t>(1, n)) return -5;
    if (dB == nullptr && n > 0 && n_rhs > 0) return -6;
    if (ldb < std::max<int64_t>(1, n)) return -7;
    if (T_A < 1) return -8;
    const size_t need = spd_workspace_size(dt, n, n_rhs, T_A);
    if (d_work == nullptr && need > 0) return -10;
    if (work_bytes < need) return -11;
    if (g_validate) {
        g_chk.begin();
        g_chk.add(dA, matrix_bytes(dt, n, n, lda), false, "L");
        g_chk.add(dB, matrix_bytes(dt, n, n_rhs, ldb), true, "B");
        g_chk.add(d_info, 4, false, "info");
        g_chk.add(d_work, work_bytes, true, "workspace");
    }
    snapshot_options();
    hipStream_t s = (hipStream_t)stream;
    switch (dt) {
    case SPD_R32:
        return Solver<float, false>::potrs(n, n_rhs, (const float *)dA, lda, (float *)dB, ldb, T_A, d_info, d_work, s,
                                           false);
    case SPD_R64:
        return Solver<double, false>::potrs(n, n_rhs, (const double *)dA, lda, (double *)dB, ldb, T_A, d_info,
                                            d_work, s, false);
    case SPD_C64:
        return Solver<float, true>::potrs(n, n_rhs, (const Elem<float, true>::type *)dA, lda,
                                          (Elem<float, true>::type *)dB, ldb, T_A, d_info, d_work, s, false);
    case SPD_C128:
        return Solver<double, true>::potrs(n, n_rhs, (const Elem<double, true>::type *)dA, lda,
                                           (Elem<double, true>::type *)dB, ldb, T_A, d_info, d_work, s, false);
    }
    return -1;
}

int spd_gp_loglik(spd_dtype_t dt, int64_t n, int64_t n_rhs, const void *dA, int64_t lda, void *dR, int64_t ldr,
                  int64_t T_A, const int32_t *d_info, double *d_out, void *d_work, size_t work_bytes, void *stream)
{
    if (dt != SPD_R32 && dt != SPD_R64) return -1;
    if (n < 0 || n > INT32_MAX) return -2;
    if (n_rhs < 0 || n_rhs > INT32_MAX) return -3;
    if (dA == nullptr && n > 0) return -4;
    if (lda < std::max<int64_t>(1, n)) return -5;
    if (dR == nullptr && n > 0 && n_rhs > 0) return -6;
    if (ldr < std::max<int64_t>(1, n)) return -7;
    if (T_A < 1) return -8;
    if (d_out == nullptr && n_rhs > 0) return -10;
    const size_t need = spd_workspace_size(dt, n, n_rhs, T_A);
    if (d_work == nullptr && need > 0) return -11;
    if (work_bytes < need) return -12;
    if (g_validate) {
        g_chk.begin();
        g_chk.add(dA, matrix_bytes(dt, n, n, lda), false, "L");
        g_chk.add(dR, matrix_bytes(dt, n, n_rhs, ldr), true, "R");
        g_chk.add(d_info, 4, false, "info");
        g_chk.add(d_out, (size_t)n_rhs * sizeof(double), true, "out");
        g_chk.add(d_work, work_bytes, true, "workspace");
    }
    snapshot_options();
    hipStream_t s = (hipStream_t)stream;
    if (dt == SPD_R32)
        return Solver<float, false>::gp_loglik(n, n_rhs, (const float *)dA, lda, (float *)dR, ldr, T_A, d_info, d_out,
                                               d_work, s);
    return Solver<double, false>::gp_loglik(n, n_rhs, (const double *)dA, lda, (double *)dR, ldr, T_A, d_info, d_out,
                                            d_work, s);
}

size_t spd_sygst_workspace_size(spd_dtype_t dt, int itype, int64_t n, int64_t T_A)
{
    const int64_t es = elem_size(dt);
    if (es == 0 || itype < 1 || itype > 3 || n <= 0 || T_A < 1)
        return 0;
    return (size_t)(make_gst_layout(itype, n, T_A, es).total * es);
}

int spd_sygst(spd_dtype_t dt, int itype, int64_t n, void *dA, int64_t lda, const void *dL, int64_t ldl, int64_t T_A,
              const int32_t *d_info, void *d_work, size_t work_bytes, void *stream)
{
    if (elem_size(dt) == 0) return -1;
    if (itype < 1 || itype > 3) return -2;
    if (n < 0 || n > (1 << 20)) return -3;  // keeps the transpose grid below 2^31 workgroups
    if (dA == nullptr && n > 0) return -4;
    if (lda < std::max<int64_t>(1, n)) return -5;
    if (dL == nullptr && n > 0) return -6;
    if (ldl < std::max<int64_t>(1, n)) return -7;
    if (T_A < 1) return -8;
    const size_t need = spd_sygst_workspace_size(dt, itype, n, T_A);
    if (d_work == nullptr && need > 0) return -10;
    if (work_bytes < need) return -11;
    if (g_validate) {
        g_chk.begin();
        g_chk.add(dA, matrix_bytes(dt, n, n, lda), true, "A");
        g_chk.add(dL, matrix_bytes(dt, n, n, ldl), false, "L");
        g_chk.add(d_info, 4, false, "info");
        g_chk.add(d_work, work_bytes, true, "workspace");
    }
    snapshot_options();
    hipStream_t s = (hipStream_t)stream;
    switch (dt) {
    case SPD_R32:
        return Solver<float, false>::gst(itype, n, (float *)dA, lda, (const float *)dL, ldl, T_A, d_info, d_work, s);
    case SPD_R64:
        return Solver<double, false>::gst(itype, n, (double *)dA, lda, (const double *)dL, ldl, T_A, d_info, d_work,
                                          s);
    case SPD_C64:
        return Solver<float, true>::gst(itype, n, (Elem<float, true>::type *)dA, lda,
                                        (const Elem<float, true>::type *)dL, ldl, T_A, d_info, d_work, s);
    case SPD_C128:
        return Solver<double, true>::gst(itype, n, (Elem<double, true>::type *)dA, lda,
                                         (const Elem<double, true>::type *)dL, ldl, T_A, d_info, d_work, s);
    }
    return -1;
}

int spd_posv(spd_dtype_t dt, int64_t n, int64_t n_rhs, void *dA, int64_t lda, void *dB, int64_t ldb, int64_t T_A,
             int32_t *d_info, double *d_logdet, void *d_work, size_t work_bytes, void *stream)
{
    if (elem_size(dt) == 0) return -1;
    if (n < 0 || n > INT32_MAX) return -2;
    if (n_rhs < 0 || n_rhs > INT32_MAX) return -3;
    if (dA == nullptr && n > 0) return -4;
    if (lda < std::max<int64_t>(1, n)) return -5;
    if (dB == nullptr && n > 0 && n_rhs > 0) return -6;
    if (ldb < std::max<int64_t>(1, n)) return -7;
    if (T_A < 1) return -8;
    if (d_info == nullptr) return -9;
    const size_t need = spd_workspace_size(dt, n, n_rhs, T_A);
    if (d_work == nullptr && need > 0) return -11;
    if (work_bytes < need) return -12;
    if (g_validate) {
        g_chk.begin();
        g_chk.add(dA, matrix_bytes(dt, n, n, lda), true, "A");
        g_chk.add(dB, matrix_bytes(dt, n, n_rhs, ldb), true, "B");
        g_chk.add(d_info, 4, true, "info");
        if (d_logdet != nullptr)
            g_chk.add(d_logdet, sizeof(double), true, "logdet");
        g_chk.add(d_work, work_bytes, true, "workspace");
    }
    snapshot_options();
    hipStream_t s = (hipStream_t)stream;
    switch (dt) {
    case SPD_R32:
        return Solver<float, false>::posv(n, n_rhs, (float *)dA, lda, (float *)dB, ldb, T_A, d_info, d_logdet, d_work,
                                          s);
    case SPD_R64:
        return Solver<double, false>::posv(n, n_rhs, (double *)dA, lda, (double *)dB, ldb, T_A, d_info, d_logdet,
                                           d_work, s);
    case SPD_C64:
        return Solver<float, true>::posv(n, n_rhs, (Elem<float, true>::type *)dA, lda, (Elem<float, true>::type *)dB,
                                         ldb, T_A, d_info, d_logdet, d_work, s);
    case SPD_C128:
        return Solver<double, true>::posv(n, n_rhs, (Elem<double, true>::type *)dA, lda,
                                          (Elem<double, true>::type *)dB, ldb, T_A, d_info, d_logdet, d_work, s);
    }
    return -1;
}

int spd_posv_noalloc(spd_dtype_t dt, int64_t n, int64_t n_rhs, void *dA, int64_t lda, void *dB, int64_t ldb,
                     int64_t T_A, int32_t *d_info, double *d_logdet, void *stream)
{
    if (elem_size(dt) == 0) return -1;
    if (n < 0 || n > INT32_MAX) return -2;
    if (n_rhs < 0 || n_rhs > INT32_MAX) return -3;
    if (dA == nullptr && n > 0) return -4;
    if (lda < std::max<int64_t>(1, n)) return -5;
    if (dB == nullptr && n > 0 && n_rhs > 0) return -6;
    if (ldb < std::max<int64_t>(1, n)) return -7;
    if (T_A < 1) return -8;
    if (d_info == nullptr) return -9;
    const size_t need = spd_workspace_size(dt, n, n_rhs, T_A);
    if (need > (size_t)SPD_NOALLOC_SCRATCH_BYTES) {
        g_last_error = "spd_posv_noalloc: these sizes need " + std::to_string(need) +
                       " bytes of workspace; the fixed scratch buffer holds " +
                       std::to_string((size_t)SPD_NOALLOC_SCRATCH_BYTES);
        return SPD_ERR_SCRATCH;
    }
    void *ws = nullptr;
    SPD_TRY(scratch_address(&ws));
    if (g_validate) {
        g_chk.begin();
        g_chk.add(dA, matrix_bytes(dt, n, n, lda), true, "A");
        g_chk.add(dB, matrix_bytes(dt, n, n_rhs, ldb), true, "B");
        g_chk.add(d_info, 4, true, "info");
        if (d_logdet != nullptr)
            g_chk.add(d_logdet, sizeof(double), true, "logdet");
        g_chk.add(ws, SPD_NOALLOC_SCRATCH_BYTES, true, "scratch");
    }
    snapshot_options();
    g_opt.v[OPT_LOOKAHEAD] = 0;  // every kernel in order on `stream`: no auxiliary streams or events
    hipStream_t s = (hipStream_t)stream;
    switch (dt) {
    case SPD_R32:
        return Solver<float, false>::posv(n, n_rhs, (float *)dA, lda, (float *)dB, ldb, T_A, d_info, d_logdet, ws, s);
    case SPD_R64:
        return Solver<double, false>::posv(n, n_rhs, (double *)dA, lda, (double *)dB, ldb, T_A, d_info, d_logdet, ws,
                                           s);
    case SPD_C64:
        return Solver<float, true>::posv(n, n_rhs, (Elem<float, true>::type *)dA, lda, (Elem<float, true>::type *)dB,
                                         ldb, T_A, d_info, d_logdet, ws, s);
    case SPD_C128:
        return Solver<double, true>::posv(n, n_rhs, (Elem<double, true>::type *)dA, lda,
                                          (Elem<double, true>::type *)dB, ldb, T_A, d_info, d_logdet, ws, s);
    }
    return -1;
}

int spd_logdet(spd_dtype_t dt, int64_t n, const void *dA, int64_t lda, const int32_t *d_info, double *d_logdet,
               void *stream)
{
    if (elem_size(dt) == 0) return -1;
    if (n < 0) return -2;
    if (dA == nullptr && n > 0) return -3;
    if (lda < std::max<int64_t>(1, n)) return -4;
    if (d_logdet == nullptr) return -6;
    if (g_validate) {
        g_chk.begin();
        g_chk.add(dA, matrix_bytes(dt, n, n, lda), false, "L");
        g_chk.add(d_info, 4, false, "info");
        g_chk.add(d_logdet, sizeof(double), true, "logdet");
    }
    snapshot_options();
    hipStream_t s = (hipStream_t)stream;
    switch (dt) {
    case SPD_R32: return Solver<float, false>::logdet(n, (const float *)dA, lda, d_info, d_logdet, s);
    case SPD_R64: return Solver<double, false>::logdet(n, (const double *)dA, lda, d_info, d_logdet, s);
    case SPD_C64:
        return Solver<float, true>::logdet(n, (const Elem<float, true>::type *)dA, lda, d_info, d_logdet, s);
    case SPD_C128:
        return Solver<double, true>::logdet(n, (const Elem<double, true>::type *)dA, lda, d_info, d_logdet, s);
    }
    return -1;
}

const char *spd_last_error(void) { return g_last_error.c_str(); }

int spd_set_option(spd_option_t opt, int64_t value)
{
    const int i = (int)opt - 1;
    if (i < 0 || i >= OPT_COUNT)
        return -1;
    if (value == SPD_OPT_DEFAULT)
        value = k_opt_default[i];
    switch (i) {
    case OPT_LOOKAHEAD:
    case OPT_TWO_STEP:
    case OPT_TILE_LAUNCH:
        if (value != 0 && value != 1)
            return -2;
        break;
    case OPT_PAIR_ROWS:
    case OPT_SYRK_DEEP_ROWS:
    case OPT_TILE_UPDATE_ROWS:
    case OPT_TRIPLE_ROWS:
        if (value < -1)
            return -2;
        break;
    default:
        if (value < 0)
            return -2;
        break;
    }
    g_opt_store[i].store(value, std::memory_order_relaxed);
    return 0;
}

int64_t spd_get_option(spd_option_t opt)
{
    const int i = (int)opt - 1;
    if (i < 0 || i >= OPT_COUNT)
        return INT64_MIN;
    return g_opt_store[i].load(std::memory_order_relaxed);
}

int spd_release(void) { return release_aux(); }

int spd_debug_validate(int mode)
{
    if (mode < 0 || mode > 2)
        return -1;
    g_validate = mode;
    return 0;
}

int spd_profile_enable(int mask)
{
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof_mask = mask;
    return 0;
}

int spd_profile_read(int kernel_class, double *ms, int64_t *launches, double *flops)
{
    if (kernel_class < 0 || kernel_class > 5)
        return -1;
    std::vector<ProfRec> mine;
    {
        std::lock_guard<std::mutex> g(g_prof_mu);
        std::vector<ProfRec> rest;
        for (auto &r : g_prof)
            (r.cls == kernel_class ? mine : rest).push_back(r);
        g_prof.swap(rest);
    }
    double tot = 0.0, fl = 0.0;
    int rc = 0;
    for (auto &r : mine) {
        float t = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&t, r.a, r.b);
        if (e != hipSuccess && rc == 0)
            rc = hip_fail(e, "spd_profile_read");
        tot += t;
        fl += r.flops;
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    if (ms) *ms = tot;
    if (launches) *launches = (int64_t)mine.size();
    if (flops) *flops = fl;
    return rc;
}

}  // extern "C"
