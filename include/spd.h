/*
 * spd.h - C ABI of the MI355X (gfx950) dense symmetric / Hermitian
 * positive-definite solver: blocked Cholesky factorization (potrf), the
 * triangular solves that use it (potrs, and the forward substitution alone),
 * the log-determinant (logdet) and the Gaussian-process marginal
 * log-likelihood built from them.
 *
 * The operation (JAXMg paper, "Software design", the potrs routine): solve
 * A X = B for an N x N symmetric (Hermitian) positive-definite A and an
 * N x N_RHS right-hand side B through the Cholesky factorization A = L L^H,
 * and optionally return log det(A) from the same factor.  The tile size T_A
 * is the caller's throughput / memory knob (same paper, "Software design" and
 * Figure 4); here it is the outer panel width of the right-looking blocked
 * factorization and the block size of the blocked triangular solves.
 * Supported element types: float32, float64, complex64, complex128 (same
 * paper, "Software design": all four dtypes).
 *
 * Conventions shared by every entry point
 *   - Matrices are column-major: element (i, j) of A is at A[i + j*lda].
 *     Complex elements are (real, imaginary) pairs, as C99 / std::complex.
 *   - Only the lower triangle of A (i >= j) is read or written; the strict
 *     upper triangle and the rows [n, lda) of every column are never touched.
 *     For complex A only the real part of the diagonal is read.
 *   - Buffers are transformed in place: potrf overwrites the lower triangle of
 *     A with L (real positive diagonal); potrs overwrites B with X.
 *   - All pointers named d_* or dA/dB are device pointers owned by the caller.
 *     The library allocates no device memory.  Its only state between calls is
 *     the options of spd_set_option, what spd_profile_* keeps while profiling
 *     is on and, for the lookahead schedules, two auxiliary HIP streams
 *     (default priority, non-blocking) and four events per host thread and
 *     device, created on first use and kept until spd_release is called on
 *     that thread (or the process ends).  Calls from one host thread must not
 *     overlap on one device (they share those streams).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the calls return without waiting for it.  spd_potrf may also run part of
 *     the factorization on its auxiliary stream, ordered with `stream` by
 *     events: it starts after the work already on `stream` and everything it
 *     enqueues is complete before any work enqueued on `stream` afterwards.
 *     Numerical status is reported on the device through d_info, so no host
 *     synchronisation happens inside.
 *   - Return value: 0 when the work was enqueued; -i when the i-th argument is
 *     invalid (nothing is enqueued); SPD_ERR_HIP when the HIP runtime reported
 *     an error while enqueueing, SPD_ERR_CHECK when launch validation (see
 *     spd_debug_validate) rejected a launch (spd_last_error() describes it).
 *   - Calls on one stream run in order; calls that share a workspace must not
 *     run concurrently.
 */
#ifndef SPD_H
#define SPD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPD_R32 = 0,  /* float                */
    SPD_R64 = 1,  /* double               */
    SPD_C64 = 2,  /* complex float        */
    SPD_C128 = 3  /* complex double       */
} spd_dtype_t;

#define SPD_ERR_HIP 1
#define SPD_ERR_CHECK 2
#define SPD_ERR_SCRATCH 3

/* Size of the fixed device scratch buffer of spd_posv_noalloc (per device). */
#define SPD_NOALLOC_SCRATCH_BYTES (64 << 20)

/* Bytes of device workspace that spd_potrf and spd_potrs need for these
 * sizes (one workspace serves both).  Returns 0 for invalid arguments
 * (n < 0, n_rhs < 0, T_A < 1, unknown dtype) and for n == 0. */
size_t spd_workspace_size(spd_dtype_t dt, int64_t n, int64_t n_rhs, int64_t T_A);

/* Cholesky factorization A = L L^H (JAXMg paper, "Software design": the
 * factorization step of potrs).
 *   dt        element type
 *   n         order of A, n >= 0
 *   dA        device, n x n column-major, leading dimension lda; on exit the
 *             lower triangle holds L (diagonal real, > 0)
 *   lda       >= max(1, n)
 *   T_A       tile size >= 1 (values > n mean one tile); n need not be a
 *             multiple of T_A
 *   d_info    device int32, written by the call: 0 on success, or j > 0 when
 *             the leading minor of order j is not positive definite (the pivot
 *             of column j-1 is <= 0 or NaN); then the factorization stopped
 *             there and the contents of the lower triangle from column j-1 on
 *             are unspecified; -1 if a wait of the one-launch diagonal tile
 *             ran out of time (SPD_OPT_TILE_WAIT_US; the factor is unusable)
 *   d_work    device workspace of work_bytes >= spd_workspace_size(dt, n, 0, T_A)
 *             bytes (may be NULL when that size is 0)
 *   stream    hipStream_t
 * Argument numbers for the -i return: dt=1 n=2 dA=3 lda=4 T_A=5 d_info=6
 * d_work=7 work_bytes=8. */
int spd_potrf(spd_dtype_t dt, int64_t n, void *dA, int64_t lda, int64_t T_A,
              int32_t *d_info, void *d_work, size_t work_bytes, void *stream);

/* Solve A X = B from the factor of spd_potrf: L Y = B, then L^H X = Y
 * (JAXMg paper, "Software design": potrs; B is N x N_RHS).
 *   dA, lda   the factor L as left by spd_potrf (lower triangle read only)
 *   dB, ldb   device, n x n_rhs column-major, ldb >= max(1, n); overwritten by X
 *   T_A       block size of the blocked substitution (any value >= 1)
 *   d_info    the d_info written by spd_potrf (may be NULL: treated as 0);
 *             if it is non-zero every entry of X is set to NaN
 *   d_work    workspace of >= spd_workspace_size(dt, n, n_rhs, T_A) bytes
 * Argument numbers: dt=1 n=2 n_rhs=3 dA=4 lda=5 dB=6 ldb=7 T_A=8 d_info=9
 * d_work=10 work_bytes=11. */
int spd_potrs(spd_dtype_t dt, int64_t n, int64_t n_rhs, const void *dA, int64_t lda,
              void *dB, int64_t ldb, int64_t T_A, const int32_t *d_info,
              void *d_work, size_t work_bytes, void *stream);

/* Solve A X = B in one call: the factorization of spd_potrf, log det(A) as
 * spd_logdet (when d_logdet is not NULL) and the substitutions of spd_potrs
 * (JAXMg paper, "Software design": potrs factors A and solves, optionally
 * returning log det(A)).  The results are those of the three calls; with the
 * default factorization schedule (any dtype) the forward substitution runs
 * on a second auxiliary stream (default priority, non-blocking, created once
 * per host thread and device like the first), one block as soon as its tile
 * of L is final, so that it overlaps the factorization.
 *   dA, lda   as spd_potrf: overwritten by L
 *   dB, ldb   as spd_potrs: n x n_rhs, overwritten by X (NaN if d_info != 0)
 *   d_info    device int32, written (as spd_potrf)
 *   d_logdet  device double or NULL (NaN if d_info != 0)
 *   d_work    workspace of >= spd_workspace_size(dt, n, n_rhs, T_A) bytes
 * Argument numbers: dt=1 n=2 n_rhs=3 dA=4 lda=5 dB=6 ldb=7 T_A=8 d_info=9
 * d_logdet=10 d_work=11 work_bytes=12. */
int spd_posv(spd_dtype_t dt, int64_t n, int64_t n_rhs, void *dA, int64_t lda, void *dB,
             int64_t ldb, int64_t T_A, int32_t *d_info, double *d_logdet, void *d_work,
             size_t work_bytes, void *stream);

/* spd_posv for callers that cannot allocate device memory or pass a
 * workspace: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and argument
 * numbers as spd_posv without d_work and work_bytes (dt=1 n=2 n_rhs=3 dA=4
 * lda=5 dB=6 ldb=7 T_A=8 d_info=9 d_logdet=10).
 *   - The workspace is a fixed buffer of SPD_NOALLOC_SCRATCH_BYTES bytes
 *     compiled into the library: each device the library runs on holds its
 *     own copy until the process ends.  Sizes whose
 *     spd_workspace_size(dt, n, n_rhs, T_A) exceeds it are rejected with
 *     SPD_ERR_SCRATCH (spd_last_error() gives both sizes) and nothing is
 *     enqueued; 64 MiB covers, e.g., fp64 n = 4096 with T_A = 256 and up to
 *     128 right-hand sides.
 *   - The call allocates nothing (no hipMalloc, no library routine that
 *     allocates) and creates no stream or event (while spd_profile_enable's
 *     kernel timing is off; that timing records events): every kernel runs in
 *     order on `stream` (the sequential schedule), on the current device,
 *     whose copy of the buffer it uses.  The first call on a device looks up
 *     that copy's address once.
 *   - Every call on one device shares that device's buffer, which keeps the
 *     previous call's contents; the call initialises what it needs.  Calls
 *     that overlap on one device (on different streams, or from different
 *     host threads) race on the buffer and must be ordered by the caller.
 * Returns 0, -i for an invalid argument, SPD_ERR_SCRATCH, SPD_ERR_HIP or
 * SPD_ERR_CHECK as the other entry points. */
int spd_posv_noalloc(spd_dtype_t dt, int64_t n, int64_t n_rhs, void *dA, int64_t lda, void *dB,
                     int64_t ldb, int64_t T_A, int32_t *d_info, double *d_logdet, void *stream);

/* Forward substitution only: overwrite B with Y = L^-1 B, from the factor of
 * spd_potrf (JAXMg paper, "Software design": the first of potrs' two
 * triangular solves; "Research Impact Statement", "Cholesky solve (potrs)":
 * the quadratic term of the Gaussian-process likelihood is |L^-1 r|^2).
 * Arguments, layout, workspace and the NaN-on-failure rule are those of
 * spd_potrs (same argument numbers); only L Y = B is solved. */
int spd_forward_solve(spd_dtype_t dt, int64_t n, int64_t n_rhs, const void *dA, int64_t lda,
                      void *dB, int64_t ldb, int64_t T_A, const int32_t *d_info,
                      void *d_work, size_t work_bytes, void *stream);

/* Gaussian-process marginal log-likelihood (JAXMg paper, "Research Impact
 * Statement", "Cholesky solve (potrs)"): for A = K + Sigma factored by
 * spd_potrf and each residual column r_j = y_j - m_j of R,
 *     out[j] = -1/2 r_j^T A^-1 r_j - 1/2 log det A - (n/2) log(2 pi),
 * computed as -1/2 |L^-1 r_j|^2 - sum_i log L_ii - (n/2) log(2 pi).
 * Real types only (dt = SPD_R32 or SPD_R64; the formula is the real Gaussian
 * density).
 *   dA, lda   the factor L (lower triangle read only)
 *   dR, ldr   device, n x n_rhs column-major residuals; overwritten by L^-1 R
 *   d_info    the d_info of spd_potrf (may be NULL); non-zero gives NaN in
 *             every out[j] and in R
 *   d_out     device double[n_rhs], written; each value is summed in double by
 *             a fixed reduction tree, so repeated calls give identical bits
 *   d_work    workspace of >= spd_workspace_size(dt, n, n_rhs, T_A) bytes
 * Argument numbers: dt=1 n=2 n_rhs=3 dA=4 lda=5 dR=6 ldr=7 T_A=8 d_info=9
 * d_out=10 d_work=11 work_bytes=12. */
int spd_gp_loglik(spd_dtype_t dt, int64_t n, int64_t n_rhs, const void *dA, int64_t lda,
                  void *dR, int64_t ldr, int64_t T_A, const int32_t *d_info, double *d_out,
                  void *d_work, size_t work_bytes, void *stream);

/* Bytes of device workspace spd_sygst needs; 0 for invalid arguments
 * (unknown dtype or itype, n <= 0, T_A < 1).  About n^2 + 10 n T_A elements
 * plus the substitution workspace for n right-hand sides (itype 1), or
 * 3 n^2 + 8 n T_A elements (itypes 2 and 3), n rounded up to 128. */
size_t spd_sygst_workspace_size(spd_dtype_t dt, int itype, int64_t n, int64_t T_A);

/* Reduction of a Hermitian-definite generalized eigenproblem to standard form
 * (the Cholesky-based reduction behind the "eigh_gen(a, b, itype)" solver of
 * the page "Differentiable Generalized Eigenvalue Decomposition", section
 * "API Reference", whose types 1-3 are the three problems below; the
 * eigen-solve that follows is not part of this library).  With
 * B = L L^H factored by spd_potrf:
 *     itype 1  (A v = w B v):                   C = L^-1 A L^-H
 *     itype 2, 3 (A B v = w v, B A v = w v):    C = L^H A L
 * C is Hermitian with the same eigenvalues w as the generalized problem (the
 * eigenvectors are v = L^-H u for itype 1 and 2, v = L u for itype 3, u those
 * of C).
 *   itype     1, 2 or 3
 *   dA, lda   device, n x n column-major, lda >= max(1, n); the lower triangle
 *             of the Hermitian A is read (the diagonal's imaginary part taken
 *             as 0) and overwritten by the lower triangle of C (with a real
 *             diagonal); the strict upper triangle is not touched
 *   dL, ldl   the factor of B as left by spd_potrf (lower triangle read only)
 *   T_A       block size of the substitutions (itype 1; any value >= 1)
 *   d_info    the d_info of spd_potrf for B (may be NULL: treated as 0); if it
 *             is non-zero the lower triangle of A is set to NaN
 *   d_work    workspace of >= spd_sygst_workspace_size(dt, itype, n, T_A) bytes
 * n is limited to 2^20.
 * Argument numbers: dt=1 itype=2 n=3 dA=4 lda=5 dL=6 ldl=7 T_A=8 d_info=9
 * d_work=10 work_bytes=11. */
int spd_sygst(spd_dtype_t dt, int itype, int64_t n, void *dA, int64_t lda, const void *dL,
              int64_t ldl, int64_t T_A, const int32_t *d_info, void *d_work, size_t work_bytes,
              void *stream);

/* log det(A) = 2 * sum_i log(Re L_ii) from the factor L of spd_potrf (JAXMg
 * paper, "Software design": the same factorization can return log det(A);
 * "Cholesky solve (potrs)": the log-determinant term of the Gaussian-process
 * marginal likelihood).  Accumulated in double for every dtype by a fixed
 * reduction tree, so repeated calls give identical bits.
 *   dA, lda    the factor L
 *   d_info     the d_info of spd_potrf (may be NULL); non-zero gives NaN
 *   d_logdet   device double, written by the call (0 for n == 0)
 * Argument numbers: dt=1 n=2 dA=3 lda=4 d_info=5 d_logdet=6. */
int spd_logdet(spd_dtype_t dt, int64_t n, const void *dA, int64_t lda,
               const int32_t *d_info, double *d_logdet, void *stream);

/* Text of the last error (HIP or launch validation) seen by this library in
 * the calling thread. */
const char *spd_last_error(void);

/* Schedule and tile-shape options.  None of them changes what is computed:
 * every setting gives the same factorization, log-determinant and solution
 * within rounding (the bits may differ between settings, and are the same
 * from run to run for one setting).  They exist to measure the schedules
 * against each other and to let tests reach every kernel variant at sizes a
 * plain CPU reference can check.  Options are process-wide; each entry point
 * reads all of them once when it is called, so a call sees one consistent set.
 *   SPD_OPT_LOOKAHEAD        1 (default): the factorization and the
 *                            substitutions run one step ahead on an auxiliary
 *                            stream; 0: everything in order on `stream`
 *   SPD_OPT_TWO_STEP         1 (default): under lookahead, groups of steps
 *                            (pairs, threes: TRIPLE_ROWS) share one trailing
 *                            update of depth 2 or 3 T_A while the trailing
 *                            matrix is large; 0: one step at a time
 *                            (spd_posv then runs its three parts in sequence)
 *   SPD_OPT_PAIR_ROWS        steps are paired while at least this many rows
 *                            remain beyond the pair; -1 (default): 32 T_A
 *   SPD_OPT_SYRK_DEEP_ROWS   trailing updates of at least this order on
 *                            128-row tiles take the deeper operand slices;
 *                            -1 (default): never (fp64), 8192 (fp32)
 *   SPD_OPT_RECT_TALL_ROWS   block updates of the substitutions and the
 *                            panel products of at least this many rows take
 *                            64-row tiles, fewer rows 32-row tiles (default
 *                            16384)
 *   SPD_OPT_TILE_LAUNCH      1 (default): each diagonal tile of a real
 *                            factorization is factored and inverted in one
 *                            launch whose workgroups hand 64 x 64 blocks to
 *                            each other through flags in the workspace; 0: by
 *                            a sequence of leaf, in-tile update and
 *                            inverse-merge launches (complex types always)
 *   SPD_OPT_TILE_WAIT_US     longest wait of that launch for another
 *                            workgroup's block, in microseconds (default
 *                            2000000).  A wait that runs out ends the
 *                            launch's other waits as well and sets info to -1
 *                            (the factor is then not usable); it exists so
 *                            that no wave can wait forever.
 *   SPD_OPT_COLUMN_FIRST_ROWS  under lookahead, in the steps taken one at a
 *                            time, the trailing update on `stream` waits for
 *                            the auxiliary stream's update of the next tile
 *                            column while fewer than this many rows remain
 *                            beyond the next tile (default 8192; 0: never)
 *   SPD_OPT_TILE_HOLD_ROWS   a real diagonal tile with fewer than this many
 *                            rows below it is factored by workgroups that keep
 *                            a CU each to themselves (twice the threads, half
 *                            of them idle, and all of the CU's group memory),
 *                            so that no other kernel's waves share the working
 *                            waves' SIMDs (default 8192; 0: never)
 *   SPD_OPT_SUBST_LAUNCH     the back substitution L^H X = Y runs in one
 *                            launch whose workgroups hand solved pieces of X
 *                            to each other through flags in the workspace
 *                            (waits bounded as for TILE_LAUNCH) while
 *                            n * n_rhs (4 n * n_rhs for complex types) is at
 *                            most this value (default 2097152), otherwise by
 *                            block steps on `stream` and an auxiliary stream
 *                            (0: always by block steps)
 *   SPD_OPT_TILE_UPDATE_ROWS in the steps taken one at a time, while fewer
 *                            than this many rows remain beyond the next tile,
 *                            that tile takes its last trailing update inside
 *                            its own launch (TILE_LAUNCH = 1 only) and the
 *                            update on `stream` covers the rest of its tile
 *                            column; -1 (default): 2048 for real types, 0
 *                            (never) for complex ones
 *   SPD_OPT_TRIPLE_ROWS      orders of at least 40 tiles (whose workspace
 *                            holds six trailing-update panels) take the
 *                            factorization's steps in threes, one trailing
 *                            update of depth 3 T_A per three steps, while at
 *                            least this many rows remain beyond the three;
 *                            then in pairs (PAIR_ROWS) and one at a time; -1
 *                            (default): 32 T_A; 0: never
 * spd_set_option returns 0, -1 for an unknown option, -2 for a value out of
 * range (LOOKAHEAD, TWO_STEP and TILE_LAUNCH take 0 or 1, PAIR_ROWS,
 * SYRK_DEEP_ROWS, TILE_UPDATE_ROWS and TRIPLE_ROWS >= -1, RECT_TALL_ROWS, TILE_WAIT_US,
 * COLUMN_FIRST_ROWS, TILE_HOLD_ROWS and SUBST_LAUNCH >= 0);
 * SPD_OPT_DEFAULT restores an option's default.
 * spd_get_option returns the current value (INT64_MIN for an unknown
 * option). */
typedef enum {
    SPD_OPT_LOOKAHEAD = 1,
    SPD_OPT_TWO_STEP = 2,
    SPD_OPT_PAIR_ROWS = 3,
    SPD_OPT_SYRK_DEEP_ROWS = 4,
    SPD_OPT_RECT_TALL_ROWS = 5,
    SPD_OPT_TILE_LAUNCH = 6,
    SPD_OPT_TILE_WAIT_US = 7,
    SPD_OPT_COLUMN_FIRST_ROWS = 8,
    SPD_OPT_TILE_HOLD_ROWS = 9,
    SPD_OPT_SUBST_LAUNCH = 10,
    SPD_OPT_TILE_UPDATE_ROWS = 11,
    SPD_OPT_TRIPLE_ROWS = 12
} spd_option_t;
#define SPD_OPT_DEFAULT INT64_MIN
int spd_set_option(spd_option_t opt, int64_t value);
int64_t spd_get_option(spd_option_t opt);

/* Wait for the work on the calling thread's auxiliary streams (on every
 * device it used) to finish, then destroy those streams and their events.
 * The next call that needs them creates them again.  Returns 0, or
 * SPD_ERR_HIP (spd_last_error() says which call failed; the thread's set is
 * forgotten either way). */
int spd_release(void);

/* Launch validation, a debugging aid for callers and tests.
 *   mode 0  off (default)
 *   mode 1  before each kernel is enqueued, replay on the host every address
 *           each of its threads would read or write, and require each to lie
 *           inside the buffers passed to the entry point (the matrix, B, the
 *           workspace, info, logdet; writes only to buffers that call may
 *           modify); a violation returns SPD_ERR_CHECK without enqueueing it
 *   mode 2  the same replay with nothing enqueued and no HIP call made at all
 *           ("dry run"): pointers are never dereferenced, so any addresses
 *           may be passed, and the launch sequence of any shape can be
 *           checked on a machine without a GPU
 * The replay visits every thread of every workgroup, so its host cost grows
 * with the problem's work; it is meant for small and medium shapes.  The
 * setting is process-wide.  Returns 0, or -1 for an unknown mode. */
int spd_debug_validate(int mode);

/* Kernel timing for measurement harnesses.  While enabled (mask != 0), every
 * launch of the selected kernel classes is bracketed by HIP events recorded
 * on its stream; spd_profile_read synchronises on those events and returns,
 * for one class, the summed kernel time in milliseconds, the number of
 * launches and their algorithmic flop count (real-equivalent flops: a complex
 * multiply-add counts 8), then forgets that class's events.
 * Classes: bit 0 = trailing update (A22 -= L21 L21^H) on the caller's stream,
 * bit 5 = the trailing update's launches on potrf's auxiliary stream (the
 * next tile columns), bit 1 = panel solve,
 * bit 2 = diagonal-tile factorization and inversion, bit 3 = substitution
 * (each whole call) and spd_sygst's two triangular products (itypes 2 and 3,
 * each launch), bit 4 = the substitutions' block-update kernel (real
 * types: B_rows -= L_panel X_k, each launch).
 * Returns 0, or -1 for an unknown class, SPD_ERR_HIP on a HIP error. */
int spd_profile_enable(int mask);
int spd_profile_read(int kernel_class, double *ms, int64_t *launches, double *flops);

#ifdef __cplusplus
}
#endif

#endif /* SPD_H */
