// Self-test of the host-side launch replay (spd_check.hpp): the replay must
// accept a launch whose buffers cover every access exactly, and must reject
// the same launch when a buffer is registered one element short (so that the
// last 16-byte vector load of an operand crosses its end) or when a
// vectorised operand is misaligned.  Built and run on the CPU by
// test_replay_selftest.py; no HIP call is made.  Prints one line per case and
// exits non-zero on the first case that does not behave as stated.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <string>

#include "spd_check.hpp"

using namespace spd;

static int failures = 0;

static void expect(bool ok, bool want, const spd::Checker &c, const char *what, const char *needle)
{
    bool good = ok == want;
    if (good && !want && needle != nullptr)
        good = c.err.find(needle) != std::string::npos;
    std::printf("%s: %s%s%s\n", good ? "ok" : "FAIL", what, want ? "" : " -> ", want ? "" : c.err.c_str());
    if (!good)
        ++failures;
}

// Fake, far-apart device addresses: the replay never dereferences them.
static const uintptr_t BASE = uintptr_t(1) << 40;

// The substitutions' block update C(m x n) -= P Q^T with 16-byte loads of P
// (fp64, 64 x 64 tiles, 16-deep slices): m = 128 rows, n = 64 columns, one
// 16-deep slice, P column-major with ldp = m.
static void rect_cases()
{
    constexpr int BM = 64, BN = 64, KB = 16, WM = 2, WN = 2;
    const int m = 128, n = 64, kp = 16;
    RectArgs a{};
    a.P = (const void *)BASE;
    a.ldp = m;
    a.Q = (const void *)(2 * BASE);
    a.ldq = 64;
    a.C = (void *)(3 * BASE);
    a.ldc = m;
    a.m = m;
    a.n = n;
    a.kp = kp;
    a.kvalid = kp;
    a.tiles_m = m / BM;
    a.ntiles = a.tiles_m * (n / BN);
    a.info = nullptr;
    const dim3 grid(a.ntiles);
    const size_t pbytes = sizeof(double) * m * kp, qbytes = sizeof(double) * a.ldq * kp,
                 cbytes = sizeof(double) * m * n;
    auto run = [&](size_t p_registered, const void *P) {
        Checker c;
        c.begin();
        c.add(P, p_registered, false, "P");
        c.add(a.Q, qbytes, false, "Q");
        c.add(a.C, cbytes, true, "C");
        RectArgs b = a;
        b.P = P;
        const bool ok = check_rect<double, BM, BN, KB, WM, WN, false, true, false>(b, grid, c);
        return std::make_pair(ok, c);
    };
    auto r = run(pbytes, a.P);
    expect(r.first, true, r.second, "block update, buffers exactly covering every access", nullptr);
    r = run(pbytes - sizeof(double), a.P);
    expect(r.first, false, r.second, "block update, P registered one element short", "reads 16 bytes");
    r = run(pbytes + sizeof(double), (const void *)(BASE + sizeof(double)));
    expect(r.first, false, r.second, "block update, P misaligned for 16-byte loads", "unaligned vector load");
    // the output registered read-only: the epilogue's stores must be caught
    Checker c;
    c.begin();
    c.add(a.P, pbytes, false, "P");
    c.add(a.Q, qbytes, false, "Q");
    c.add(a.C, cbytes, false, "C");
    const bool ok = check_rect<double, BM, BN, KB, WM, WN, false, true, false>(a, grid, c);
    expect(ok, false, c, "block update, C not writable", "writes");
}

// The trailing update C -= W W^T over the lower tiles (fp64, 128-row tiles,
// 8-deep slices): order m = 256, a panel of 16 columns with ldw = 256.
static void syrk_cases()
{
    constexpr int BM = 128, KB = 8, WM = 2, WN = 4;
    const int m = 256, kp = 16;
    SyrkArgs a{};
    a.W = a.V = (const void *)BASE;
    a.ldw = m;
    a.C = (void *)(3 * BASE);
    a.ldc = m;
    a.m = m;
    a.kp = kp;
    a.tiles = m / BM;
    a.ntiles = a.tiles * (a.tiles + 1) / 2;
    a.krange = SYRK_K_ALL;
    a.info = nullptr;
    const dim3 grid(a.ntiles);
    const size_t wbytes = sizeof(double) * m * kp, cbytes = sizeof(double) * m * m;
    auto run = [&](size_t w_registered) {
        Checker c;
        c.begin();
        c.add(a.W, w_registered, false, "W");
        c.add(a.C, cbytes, true, "C");
        const bool ok = check_syrk<double, false, BM, KB, WM, WN, false>(a, grid, c);
        return std::make_pair(ok, c);
    };
    auto r = run(wbytes);
    expect(r.first, true, r.second, "trailing update, buffers exactly covering every access", nullptr);
    r = run(wbytes - sizeof(double));
    expect(r.first, false, r.second, "trailing update, panel registered one element short", "reads 16 bytes");
}

int main()
{
    rect_cases();
    syrk_cases();
    std::printf("%s\n", failures == 0 ? "all cases behaved" : "some cases failed");
    return failures == 0 ? 0 : 1;
}
