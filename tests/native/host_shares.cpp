// host_shares.cpp -- the balanced schedule's split of positions among
// workgroups (internal.h: Shares and XcdShares), run on the host under
// the sanitizers (tests/test_sanitizers.py) for every grid size up to 300 and
// a spread of totals:
// - share_of is a bijection of [0, n); numbered XCD by XCD (requested, and
//   every share holds a position) it gives each XCD (workgroup index mod 8)
//   one run of consecutive shares, else it is the identity;
// - the shares that hold a position are consecutive (the merges walk a
//   pair's pieces share by share);
// - the shares tile [0, total) in order; each holds q or q + 1 positions, the
//   longer ones being exactly the total % n workgroups with the lowest indices;
// - wg_of(p) is the share whose range holds p;
// - numbered XCD by XCD, the XCDs' runs differ by at most one position
//   beyond q times their workgroup counts.
#include <climits>
#include <cstdio>
#include <vector>

#include "internal.h"

using namespace kvc;

static long failures = 0;
#define CHECK(c)                                                                           \
    do {                                                                                   \
        if (!(c)) {                                                                        \
            if (failures < 20) std::fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                                    \
        }                                                                                  \
    } while (0)

template <bool XCD>
static void check(long total, int n) {
    bool numbered_by_xcd = false;
    auto split = [&]() {
        if constexpr (XCD) {
            const XcdShares x = xcd_shares_of(total, n);
            numbered_by_xcd = x.xcd;
            return x;
        } else {
            return shares_of(total, n);
        }
    };
    const auto sh = split();
    CHECK(numbered_by_xcd == (XCD && total >= n));
    const long q = total / n, r = total % n;
    std::vector<int> owner(n, -1);  // workgroup of each share
    for (int i = 0; i < n; ++i) {
        const int w = sh.share_of(i);
        CHECK(w >= 0 && w < n);
        if (w < 0 || w >= n) return;
        CHECK(owner[w] == -1);
        owner[w] = i;
    }
    CHECK(sh.start(0) == 0);
    CHECK(sh.start(n) == total);
    std::vector<long> per_xcd(8, 0);
    std::vector<int> wgs_xcd(8, 0);
    for (int w = 0; w < n; ++w) {
        const int i = owner[w];
        if (!numbered_by_xcd) CHECK(w == i);
        if (numbered_by_xcd && w > 0) CHECK(owner[w - 1] % 8 <= i % 8);  // one run per XCD, in XCD order
        if (numbered_by_xcd && w > 0 && owner[w - 1] % 8 == i % 8) CHECK(owner[w - 1] + 8 == i);
        const long len = sh.start(w + 1) - sh.start(w);
        if (w > 0 && len > 0) CHECK(sh.start(w) > sh.start(w - 1));  // no empty share before a nonempty one
        CHECK(len == q + (i < r ? 1 : 0));
        per_xcd[i % 8] += len;
        wgs_xcd[i % 8] += 1;
    }
    long lo = LONG_MAX, hi = LONG_MIN;
    for (int x = 0; x < 8; ++x) {
        const long extra = per_xcd[x] - q * wgs_xcd[x];
        lo = extra < lo ? extra : lo;
        hi = extra > hi ? extra : hi;
    }
    if (numbered_by_xcd) CHECK(hi - lo <= 1);
    // wg_of: every position when the total is small, else samples
    const long step = total <= 20000 ? 1 : total / 9973 + 1;
    for (long p = 0; p < total; p += step) {
        const int w = sh.wg_of(p);
        CHECK(w >= 0 && w < n && sh.start(w) <= p && p < sh.start(w + 1));
    }
    if (total > 0) {
        const int w = sh.wg_of(total - 1);
        CHECK(w >= 0 && w < n && sh.start(w) <= total - 1 && total - 1 < sh.start(w + 1));
    }
}

int main() {
    const long totals[] = {0, 1, 2, 7, 8, 9, 63, 64, 65, 255, 1000, 4099, 77777, 262144 + 2048 * 3, 2147483647L * 8};
    const int grids[] = {512, 1024, 2048, 3072, 4096, 8192};
    for (int n = 1; n <= 300; ++n)
        for (long t : totals) check<false>(t, n), check<true>(t, n);
    for (int n : grids)
        for (long t : totals) check<false>(t, n), check<true>(t, n);
    if (failures) {
        std::fprintf(stderr, "%ld failures\n", failures);
        return 1;
    }
    std::printf("host shares ok\n");
    return 0;
}
