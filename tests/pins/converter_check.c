/*
 * converter_check.c -- host side of the GPU converter sweep: compares what
 * the gfx950 conversion helpers and divisions returned (tests/pins/
 * converter_sweep.hip) with the CPU oracle's encoders and decoders and with
 * IEEE binary32 C arithmetic (built with the oracle's flags: no contraction,
 * no fast-math, SSE arithmetic).
 *
 * Inputs: every binary32 pattern in a chunk [base, base + count).  NaN inputs
 * are skipped for the encoders (the kernels never convert a NaN: inputs are
 * finite and every product they form is finite); the divisions compare NaN
 * results by NaN-ness only.
 *
 * Test infrastructure: links the oracle library.  Each check splits its
 * chunk over `threads` POSIX threads and returns the number of mismatches;
 * *first_bad receives the first mismatching pattern (lowest index of the
 * first thread that saw one) and *what a code naming the converter.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#include "../../oracle/gcache_oracle.h"

enum { W_FP4 = 1, W_FP4_SEL = 2, W_FP8 = 3, W_BF16 = 4, W_DIV6 = 5, W_DIV448 = 6, W_RECIP = 7, W_SCALE_DIV = 8 };

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

typedef struct {
    uint32_t base;
    int64_t lo, hi;                /* index range of this thread */
    const uint8_t* fp4;            /* 1 byte per input (see the sweep kernel) */
    const uint8_t* fp8;            /* 1 byte per input */
    const uint16_t* bf16;          /* 1 per input */
    const uint32_t* div6;
    const uint32_t* div448;
    const uint32_t* recip;
    const float* a;                /* scale-division pairs */
    const float* b;
    const uint32_t* q;
    int64_t bad;
    uint32_t first;
    int what;
} job;

static void note(job* j, uint32_t pattern, int what) {
    if (j->bad++ == 0) { j->first = pattern; j->what = what; }
}

static int same_div(uint32_t got, float want) {
    if (isnan(want)) return isnan(f_of(got));
    return got == u_of(want);
}

static void* run_codes(void* arg) {
    job* j = (job*)arg;
    for (int64_t i = j->lo; i < j->hi; i++) {
        const uint32_t u = j->base + (uint32_t)i;
        const float x = f_of(u);
        if (isnan(x)) continue;
        /* fp4: word i/4 holds byte 0 = (x0, x1), byte 1 = (x2, x3) from
         * selectors 0, 1 and bytes 2, 3 the same pairs from selectors 2, 3 */
        const int64_t w = i / 4, k = i % 4;
        const uint8_t byte = j->fp4[4 * w + k / 2];
        const uint8_t twin = j->fp4[4 * w + 2 + k / 2];
        const uint8_t code = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        if (code != orc_e2m1_encode(x)) note(j, u, W_FP4);
        else if (twin != byte) note(j, u, W_FP4_SEL);
        if (j->fp8[i] != orc_e4m3_encode(x)) note(j, u, W_FP8);
        if (j->bf16[i] != orc_f32_to_bf16_rne(x)) note(j, u, W_BF16);
    }
    return 0;
}

static void* run_divs(void* arg) {
    job* j = (job*)arg;
    for (int64_t i = j->lo; i < j->hi; i++) {
        const uint32_t u = j->base + (uint32_t)i;
        const float x = f_of(u);
        if (!same_div(j->div6[i], x / 6.0f)) note(j, u, W_DIV6);
        if (!same_div(j->div448[i], x / 448.0f)) note(j, u, W_DIV448);
        if (!same_div(j->recip[i], 1.0f / x)) note(j, u, W_RECIP);
    }
    return 0;
}

static void* run_scale_div(void* arg) {
    job* j = (job*)arg;
    for (int64_t i = j->lo; i < j->hi; i++)
        if (!same_div(j->q[i], (j->a[i] / 6.0f) / j->b[i])) note(j, (uint32_t)i, W_SCALE_DIV);
    return 0;
}

static int64_t run(job proto, int64_t count, int threads, void* (*fn)(void*), uint32_t* first_bad, int* what) {
    enum { kMaxThreads = 64 };
    if (threads < 1) threads = 1;
    if (threads > kMaxThreads) threads = kMaxThreads;
    job jobs[kMaxThreads];
    pthread_t tid[kMaxThreads];
    int started[kMaxThreads] = {0};
    for (int t = 0; t < threads; t++) {
        jobs[t] = proto;
        jobs[t].lo = count * t / threads;
        jobs[t].hi = count * (t + 1) / threads;
        jobs[t].bad = 0;
        jobs[t].first = 0;
        jobs[t].what = 0;
        started[t] = pthread_create(&tid[t], 0, fn, &jobs[t]) == 0;
        if (!started[t]) fn(&jobs[t]);
    }
    int64_t bad = 0;
    for (int t = 0; t < threads; t++) {
        if (started[t]) pthread_join(tid[t], 0);
        if (jobs[t].bad && bad == 0) { *first_bad = jobs[t].first; *what = jobs[t].what; }
        bad += jobs[t].bad;
    }
    return bad;
}

int64_t check_codes(uint32_t base, int64_t count, const uint8_t* fp4, const uint8_t* fp8, const uint16_t* bf16,
                    int threads, uint32_t* first_bad, int* what) {
    job p;
    memset(&p, 0, sizeof p);
    p.base = base;
    p.fp4 = fp4;
    p.fp8 = fp8;
    p.bf16 = bf16;
    return run(p, count, threads, run_codes, first_bad, what);
}

int64_t check_divs(uint32_t base, int64_t count, const uint32_t* div6, const uint32_t* div448,
                   const uint32_t* recip, int threads, uint32_t* first_bad, int* what) {
    job p;
    memset(&p, 0, sizeof p);
    p.base = base;
    p.div6 = div6;
    p.div448 = div448;
    p.recip = recip;
    return run(p, count, threads, run_divs, first_bad, what);
}

int64_t check_scale_div(const float* a, const float* b, const uint32_t* q, int64_t count, int threads,
                        uint32_t* first_bad, int* what) {
    job p;
    memset(&p, 0, sizeof p);
    p.a = a;
    p.b = b;
    p.q = q;
    return run(p, count, threads, run_scale_div, first_bad, what);
}

/* Decoders: e4m3[5c + k] must all equal the oracle's decode of code c (NaN
 * codes: NaN), e2m1[8c + 2s], e2m1[8c + 2s + 1] the decodes of the low and
 * high nibble of byte c.  Returns the number of mismatches. */
int64_t check_decoders(const float* e4m3, const float* e2m1) {
    int64_t bad = 0;
    for (int c = 0; c < 256; c++) {
        const float want = orc_e4m3_decode((uint8_t)c);
        for (int k = 0; k < 5; k++) {
            const float got = e4m3[5 * c + k];
            if (isnan(want) ? !isnan(got) : u_of(got) != u_of(want)) bad++;
        }
        const float lo = orc_e2m1_decode((uint8_t)(c & 0xF)), hi = orc_e2m1_decode((uint8_t)(c >> 4));
        for (int s = 0; s < 4; s++)
            if (u_of(e2m1[8 * c + 2 * s]) != u_of(lo) || u_of(e2m1[8 * c + 2 * s + 1]) != u_of(hi)) bad++;
    }
    return bad;
}
