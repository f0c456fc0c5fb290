// Host check of the launch geometry the library builds (zero_internal.h):
// for every grid, the XCD remap must be a bijection onto the grid, every
// quad (and the ragged tail) must have a thread, each XCD must get runs of
// `group` consecutive logical blocks, and the padding must stay under one
// round of runs.  Prints one line per failure and "all checks passed".
#include <cstdio>
#include <vector>

#include "zero_internal.h"

using namespace zero;

static int failures = 0;
#define CHECK(cond, ...)                        \
    do {                                        \
        if (!(cond)) {                          \
            std::printf("FAIL " __VA_ARGS__);   \
            std::printf("\n");                  \
            ++failures;                         \
        }                                       \
    } while (0)

// units: work items (quads, or 8-element vectors for flatten), one per thread.
static void check_grid(int64_t n, int64_t units, int threads, int64_t blocks, int32_t group,
                       const char* what) {
    CHECK(group >= 1 && blocks % (static_cast<int64_t>(kXcds) * group) == 0,
          "%s n=%lld: %lld blocks not a multiple of 8 x %d", what, (long long)n, (long long)blocks, group);
    CHECK(blocks * threads >= units && blocks >= 1,
          "%s n=%lld: %lld blocks of %d do not cover %lld items", what, (long long)n,
          (long long)blocks, threads, (long long)units);
    int64_t needed = (units + threads - 1) / threads;
    if (needed < 1) needed = 1;
    CHECK(blocks - needed < static_cast<int64_t>(kXcds) * group,
          "%s n=%lld: %lld blocks for %lld needed", what, (long long)n, (long long)blocks, (long long)needed);
    std::vector<unsigned char> seen(static_cast<size_t>(blocks), 0);
    for (int64_t b = 0; b < blocks; ++b) {
        const int64_t l = xcd_logical_block(static_cast<uint32_t>(b), static_cast<uint32_t>(group));
        if (l < 0 || l >= blocks || seen[l]) {
            CHECK(false, "%s n=%lld: block %lld maps to %lld (out of range or taken)", what,
                  (long long)n, (long long)b, (long long)l);
            return;
        }
        seen[l] = 1;
        // within an XCD (b and b + 8), logical blocks advance by one inside a run
        const int64_t j = b / kXcds;
        if (b + kXcds < blocks && (j + 1) % group != 0) {
            const int64_t next = xcd_logical_block(static_cast<uint32_t>(b + kXcds),
                                                   static_cast<uint32_t>(group));
            CHECK(next == l + 1, "%s n=%lld: XCD run broken at block %lld", what, (long long)n,
                  (long long)b);
        }
    }
}

int main() {
    const int64_t sizes[] = {0, 1, 3, 4, 5, 1023, 1024, 1025, 4095, 196992, 524287, 524288, 524289,
                             2097151, 2097152, 2097153, 8390656, 12500096, 273013248,
                             (1LL << 31) + (1LL << 20) + 8, 1625000064LL};
    for (int64_t n : sizes) {
        for (int threads : {kReduceThreads, kApplyThreads}) {
            const Grid g = grid_for(n, threads);
            check_grid(n, quads_of(n), threads, g.blocks, g.group,
                       threads == kReduceThreads ? "reduce" : "apply");
        }
        // a flatten launch of one aligned tensor: one 8-element vector per
        // thread, blocks of 256, the grid rounded up to a multiple of 8 with
        // one share per XCD
        const int64_t body = n / 8, nb = body > 0 ? (body + 255) / 256 : 1;
        const int64_t fb = (nb + kXcds - 1) / kXcds * kXcds;
        if (fb <= (1LL << 24)) check_grid(n, body, 256, fb, static_cast<int32_t>(fb / kXcds), "flatten");
    }
    if (failures == 0) std::printf("all checks passed\n");
    return failures == 0 ? 0 : 1;
}
