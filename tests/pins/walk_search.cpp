// Host check of the gather walk's request search (find_request in
// gather_concat_cache_amd/csrc/gcache_device.h) against a linear scan, on
// random non-decreasing workspace_starts with empty requests, single
// requests, one-row requests and long requests.  Exit status 0 = all agree.
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
            checked++;
        }
    }
    std::printf("find_request agrees with a linear scan on %lld queries\n", checked);
    return 0;
}
