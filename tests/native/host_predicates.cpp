// host_predicates.cpp -- the length predicates the kernels apply to device
// metadata (internal.h: length_after, append_fits, ctx_of, seq_range,
// window_released), run
// on the host at the int32 limits, under the sanitizers
// (tests/test_sanitizers.py): a corrupt length near INT32_MAX must read as
// invalid, never wrap into a valid one.
#include <climits>
#include <cstdio>

#include "internal.h"
#include "window.h"

using namespace kvc;

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            std::fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

int main() {
    const int mb = INT_MAX / kBlock;  // the widest table the library accepts
    // length after an append
    CHECK(length_after(INT_MAX, 1) == -1);
    CHECK(length_after(INT_MAX - 1, 1) == INT_MAX);
    CHECK(length_after(INT_MAX, 0) == INT_MAX);
    CHECK(length_after(-1, 1) == -1);
    CHECK(length_after(INT_MIN, 5) == -1);
    CHECK(length_after(37, 1) == 38);
    // an append must fit the table
    CHECK(!append_fits(INT_MAX, 1, mb));
    CHECK(!append_fits(INT_MAX - 3, 4, mb));
    CHECK(append_fits(mb * kBlock - 1, 1, mb));
    CHECK(!append_fits(mb * kBlock, 1, mb));
    CHECK(!append_fits(mb * kBlock - 4, 5, mb));
    CHECK(!append_fits(-1, 1, 10));
    CHECK(append_fits(0, 16, 1) && !append_fits(0, 17, 1) && append_fits(15, 1, 1) && !append_fits(16, 1, 1));
    // the attended length of a decode step
    int L = INT_MAX;
    AttnParams p{};
    p.ctx_lens = &L;
    p.ctx_add = 1;
    CHECK(ctx_of(p, 0) == -1);
    L = 100;
    CHECK(ctx_of(p, 0) == 101);
    p.ctx_add = 0;
    L = INT_MAX;
    CHECK(ctx_of(p, 0) == INT_MAX);
    // a length beyond the table is bad, however large
    CHECK(seq_range(INT_MAX, mb, 0, mb, 1, 1).bad);
    CHECK(seq_range(INT_MAX, 1, 0, 1, 1, 1).bad);
    CHECK(seq_range(-1, 4, 0, 4, 1, 1).bad);
    CHECK(!seq_range(64, 4, 0, 4, 1, 1).bad && seq_range(65, 4, 0, 4, 1, 1).bad);
    CHECK(!seq_range(mb * kBlock, mb, 0, mb, 1, 1).bad);
    // blocks released by a limited window, at the int32 limits
    CHECK(window_released(INT_MAX, 1) == (int)(2147483647LL / kBlock));  // tokens 0 .. INT_MAX - 1 dead
    CHECK(window_released(INT_MAX, INT_MAX) == 0);
    CHECK(window_released(INT_MAX, 0) == 0);
    CHECK(window_released(-1, 16) == -1 && window_released(INT_MIN, 0) == -1);
    CHECK(window_released(100, 16) == 5 && window_released(15, 1) == 0 && window_released(16, 1) == 1);
    if (failures) return 1;
    std::printf("host predicates ok\n");
    return 0;
}
