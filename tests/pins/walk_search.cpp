// Host check of the gather walk's request searches (find_request and, for
// batch <= 64, bisect_request64 in gather_concat_cache_amd/csrc/gcache_device.h)
// against a linear scan, on random non-decreasing workspace_starts with
// empty requests, single requests, one-row requests and long requests; on
// invalid workspace_starts (not starting at 0, decreasing, random) both must
// stop with a request in [0, batch); row_entry must reject positions outside
// the block-table row and block ids outside the cache.  Exit status 0 = all
// pass.
#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>
#include "../../gather_concat_cache_amd/csrc/gcache_device.h"

int main() {
    std::mt19937_64 rng(7);
    long long checked = 0;
    for (int trial = 0; trial < 4000; trial++) {
        const int batch = 1 + (int)(rng() % (trial % 4 == 0 ? 9000 : 70));
        std::vector<int32_t> ws(batch);
        int64_t pos = 0;
        const int mode = trial % 5;
        for (int b = 0; b < batch; b++) {
            ws[b] = (int32_t)pos;
            int64_t len;
            if (mode == 0) len = 1;                                   // one row per request
            else if (mode == 1) len = rng() % 3;                      // many empty requests
            else if (mode == 2) len = (rng() % 4 == 0) ? 0 : 1 + rng() % 40000;
            else if (mode == 3) len = rng() % 2 ? 0 : 1 + rng() % 5;
            else len = 1 + rng() % 700;
            pos += len;
        }
        int64_t total = pos + (int64_t)(rng() % 3);                   // trailing rows of the last request
        if (total == 0) total = 1;
        for (int q = 0; q < 300; q++) {
            const int64_t r = (q < 3) ? (q == 0 ? 0 : total - q) : (int64_t)(rng() % total);
            if (r < 0) continue;
            int want = 0;
            for (int b = 0; b < batch; b++) if (ws[b] <= r) want = b;
            const int got = gcache::find_request(ws.data(), batch, r, total);
            if (got != want) {
                std::printf("mismatch: trial %d batch %d total %lld r %lld got %d want %d\n", trial, batch,
                            (long long)total, (long long)r, got, want);
                return 1;
            }
            if (batch <= 64) {
                const int got64 = gcache::bisect_request64([&](int i) { return (int64_t)ws[i]; }, batch, r);
                if (got64 != want) {
                    std::printf("bisect64 mismatch: trial %d batch %d r %lld got %d want %d\n", trial, batch,
                                (long long)r, got64, want);
                    return 1;
                }
            }
            checked++;
        }
    }
    // invalid workspace_starts: the searches must stop inside [0, batch)
    long long invalid = 0;
    for (int trial = 0; trial < 3000; trial++) {
        const int batch = 1 + (int)(rng() % (trial % 2 ? 64 : 300));
        std::vector<int32_t> ws(batch);
        for (int b = 0; b < batch; b++) {
            const int mode = trial % 3;
            ws[b] = mode == 0 ? (int32_t)(5 + b * 3)                          // ws[0] > 0
                  : mode == 1 ? (int32_t)((batch - b) * 7)                    // decreasing
                              : (int32_t)(rng() % 2000) - 300;                // anything
        }
        const int64_t total = 1 + (int64_t)(rng() % 3000);
        for (int q = 0; q < 50; q++) {
            const int64_t r = (int64_t)(rng() % total);
            const int a = gcache::find_request(ws.data(), batch, r, total);
            if (a < 0 || a >= batch) {
                std::printf("find_request left [0, batch) on invalid ws: %d of %d\n", a, batch);
                return 1;
            }
            if (batch <= 64) {
                const int c = gcache::bisect_request64([&](int i) { return (int64_t)ws[i]; }, batch, r);
                if (c < 0 || c >= batch) {
                    std::printf("bisect_request64 left [0, batch) on invalid ws: %d of %d\n", c, batch);
                    return 1;
                }
            }
            invalid++;
        }
    }
    // row_entry bounds: 2 requests x 3 block-table columns, 4 blocks of 8
    {
        const int32_t bt[6] = {0, 3, 9, 2, -1, 1};
        const gcache::BlockDiv d8{8, 3}, d6{6, -1};
        struct Case { int b; int64_t ws_b, ss_b, r; const gcache::BlockDiv* d; int64_t want; };
        const Case cases[] = {
            {0, 0, 0, 0, &d8, 0},                 // block 0, offset 0
            {0, 0, 5, 6, &d8, 3 * 1000 + 3 * 10}, // pos 11 -> block bt[1] = 3, offset 3
            {0, 0, 0, 16, &d8, -1},               // pos 16 -> bt[2] = 9 >= 4 blocks
            {0, 0, 0, 24, &d8, -1},               // pos 24 -> column 3 >= stride 3
            {1, 10, 0, 10, &d8, 2 * 1000},        // request 1, pos 0 -> block 2
            {1, 10, 0, 18, &d8, -1},              // pos 8 -> bt[4] = -1
            {1, 10, 2, 29, &d8, 1 * 1000 + 5 * 10}, // pos 21 -> bt[5] = 1, offset 5
            {1, 10, -5, 12, &d8, -1},             // pos -3
            {0, 0, 0, 7, &d6, 3 * 1000 + 1 * 10}, // block size 6: pos 7 -> bt[1] = 3, offset 1
            {0, 0, 0, 13, &d6, -1},               // pos 13 -> bt[2] = 9 >= 4 blocks
        };
        int k = 0;
        for (const Case& c : cases) {
            const int64_t want = c.want;
            const int64_t got = gcache::row_entry(bt, 3, c.b, c.ws_b, c.ss_b, c.r, *c.d, 4, 1000, 10);
            if (got != want) {
                std::printf("row_entry case %d: got %lld want %lld\n", k, (long long)got, (long long)want);
                return 1;
            }
            k++;
        }
    }
    std::printf("request searches agree with a linear scan on %lld queries; %lld queries on invalid "
                "workspace_starts stayed in range; row_entry bounds hold\n", checked, invalid);
    return 0;
}
