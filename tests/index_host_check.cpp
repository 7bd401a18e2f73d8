// Host check of the packed-layout index arithmetic (gdn2_index.h) that the
// kernels use: on well-formed cu_seqlens the slots are unique and the owner
// search inverts them; on malformed arrays (entries past T, negative,
// decreasing) every derived token range, checkpoint slot and segment index
// stays inside the buffers the library sizes from T and N alone.
// Built with g++ by tests/test_index_host.py; prints "ok" and exits 0.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <set>
#include <vector>

#include "gdn2_index.h"

using namespace gdn2;

static int failures = 0;
#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            if (failures++ < 20) fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); \
        }                                                                         \
    } while (0)

template <typename I>
static void check_case(const std::vector<I> &cu, int64_t T, bool well_formed)
{
    const int N = (int)cu.size() - 1;
    const int cu64 = sizeof(I) == 8;
    const void *c = cu.data();
    const int64_t nslots = slot_count(T, N);
    std::set<int64_t> seen;
    for (int n = 0; n < N; ++n) {
        const SeqRange r = seq_range(c, cu64, T, n);
        CHECK(0 <= r.b && r.b <= r.e && r.e <= T);
        if (well_formed) CHECK(r.b == (int64_t)cu[n] && r.e == (int64_t)cu[n + 1]);
        for (int64_t ch = 0; ch < chunks_of(r); ++ch) {
            const int64_t s = chunk_slot(r.b, n, ch);
            CHECK(0 <= s && s < nslots);
            const int64_t t0 = r.b + CHUNK * ch;
            CHECK(0 <= t0 && t0 < r.e);
            if (well_formed) {
                CHECK(seen.insert(s).second);  // unique
                int on;
                int64_t oc;
                CHECK(slot_owner(c, cu64, T, N, s, &on, &oc) && on == n && oc == ch);
            }
        }
        for (int L = 1; L <= 9; L += 4) {
            const int64_t nseg = seg_count(T, L);
            const int last = seg_last(r, L);
            CHECK(last >= 0 && (chunks_of(r) == 0 || last < nseg));
            for (int j = 0; j <= last && chunks_of(r) > 0; ++j) {
                const int64_t tb = r.b + (int64_t)j * L * CHUNK;
                CHECK(0 <= tb && tb < r.e);
            }
        }
    }
    // every slot the chunk-parallel grid visits maps to an in-range chunk or
    // is skipped
    for (int64_t s = 0; s < nslots; ++s) {
        int on;
        int64_t oc;
        if (slot_owner(c, cu64, T, N, s, &on, &oc)) {
            CHECK(0 <= on && on < N);
            const SeqRange r = seq_range(c, cu64, T, on);
            CHECK(0 <= oc && oc < chunks_of(r));
            CHECK(r.b + CHUNK * oc < r.e && r.e <= T);
            if (well_formed) CHECK(seen.count(s) == 1);
        } else if (well_formed) {
            CHECK(seen.count(s) == 0);
        }
    }
}

int main()
{
    std::mt19937_64 rng(12345);
    for (int trial = 0; trial < 3000; ++trial) {
        const int N = 1 + (int)(rng() % 9);
        const int64_t T = (int64_t)(rng() % 700);
        // well-formed: sorted cuts of [0, T]
        std::vector<int64_t> cuts(N + 1);
        cuts[0] = 0;
        cuts[N] = T;
        for (int i = 1; i < N; ++i) cuts[i] = T ? (int64_t)(rng() % (T + 1)) : 0;
        std::sort(cuts.begin() + 1, cuts.begin() + N);
        std::vector<int32_t> c32(cuts.begin(), cuts.end());
        check_case(c32, T, true);
        check_case(cuts, T, true);
        // malformed: arbitrary entries, including negative, past T and
        // decreasing, in both element types
        std::vector<int64_t> bad(N + 1);
        for (int i = 0; i <= N; ++i) {
            const int kind = (int)(rng() % 5);
            bad[i] = kind == 0 ? -(int64_t)(rng() % 1000) - 1
                     : kind == 1 ? T + (int64_t)(rng() % 5000) + 1
                     : kind == 2 ? (int64_t)(rng() % (T + 1))
                     : kind == 3 ? (i ? bad[i - 1] - (int64_t)(rng() % 200) : 0)
                                 : (int64_t)0x7fffffff;
        }
        check_case(bad, T, false);
        std::vector<int32_t> b32(N + 1);
        for (int i = 0; i <= N; ++i) b32[i] = (int32_t)bad[i];
        check_case(b32, T, false);
        bad[0] = INT64_MIN / 2;
        bad[N] = INT64_MAX / 2;
        check_case(bad, T, false);
    }
    // no cu_seqlens: one sequence of T tokens
    const SeqRange r = seq_range(nullptr, 0, 1000, 0);
    CHECK(r.b == 0 && r.e == 1000);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
