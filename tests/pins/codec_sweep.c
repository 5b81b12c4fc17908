/*
 * Exhaustive pin of the oracle's scalar codecs: every one of the 2^32
 * binary32 bit patterns (NaNs excluded) is encoded by the oracle and by an
 * independent formulation written here from the OCP MX definitions:
 *
 *   e2m1: the grid spacing is 0.5 on [0,2), 1 on [2,4) and 2 on [4,6], so the
 *         nearest value with ties to the even code is rint(|y| / spacing) with
 *         the current (round-to-nearest-even) rounding mode; |y| >= 6 saturates.
 *   e4m3: quantum 2^-9 below 2^-6 (subnormals), else 2^(E-3) for the binade
 *         2^E <= |y| < 2^(E+1); code = rint(|y| / quantum) re-packed, and
 *         anything above code 0x7E (448) saturates to 0x7E.
 *   bf16: the binary32 pattern plus 0x7FFF plus the kept LSB, shifted.
 *
 * Test infrastructure: links the oracle library.  Usage:
 *   codec_sweep <threads> [lo_hex hi_hex]     (range of patterns, default all)
 * Prints mismatch counts and exits 0 only when all of them are 0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/gcache_oracle.h"

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static uint8_t ref_e2m1(float y) {
    uint8_t s = signbit(y) ? 8 : 0;
    double d = fabs((double)y);
    int code;
    if (d >= 6) code = 7;
    else if (d < 2) code = (int)rint(d * 2);        /* 0..4 -> codes 0..4 */
    else if (d < 4) code = (int)rint(d) + 2;        /* 2,3,4 -> codes 4,5,6 */
    else code = (int)rint(d / 2) + 4;               /* 2,3 -> codes 6,7 (4.0, 6.0) */
    return (uint8_t)(s | code);
}

static uint8_t ref_e4m3(float y) {
    uint8_t s = signbit(y) ? 0x80 : 0;
    double d = fabs((double)y);
    int code;
    if (d < ldexp(1.0, -6)) {
        code = (int)rint(ldexp(d, 9));              /* 8 is the first normal, code 8 */
    } else {
        int e;
        frexp(d, &e);                               /* d = f * 2^e, f in [0.5, 1) */
        int E = e - 1;
        if (E > 9) E = 9;                           /* far above 448 anyway */
        int k = (int)rint(ldexp(d, 3 - E));         /* 8 .. 16 */
        if (k == 16) { k = 8; E++; }
        code = ((E + 7) << 3) | (k - 8);
    }
    if (code > 0x7E) code = 0x7E;                   /* satfinite */
    return (uint8_t)(s | code);
}

static uint16_t ref_bf16(uint32_t u) { return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16); }

typedef struct { uint64_t lo, hi, bad2, bad4, badb, first2, first4, firstb; } job_t;

static void* run(void* p) {
    job_t* j = (job_t*)p;
    for (uint64_t v = j->lo; v < j->hi; v++) {
        uint32_t u = (uint32_t)v;
        float y = f_of(u);
        if (isnan(y)) continue;
        if (orc_e2m1_encode(y) != ref_e2m1(y)) { if (!j->bad2++) j->first2 = u; }
        if (orc_e4m3_encode(y) != ref_e4m3(y)) { if (!j->bad4++) j->first4 = u; }
        if (orc_f32_to_bf16_rne(y) != ref_bf16(u)) { if (!j->badb++) j->firstb = u; }
    }
    return NULL;
}

int main(int argc, char** argv) {
    int nt = argc > 1 ? atoi(argv[1]) : 8;
    uint64_t lo = argc > 3 ? strtoull(argv[2], NULL, 16) : 0;
    uint64_t hi = argc > 3 ? strtoull(argv[3], NULL, 16) : (1ull << 32);
    if (nt < 1) nt = 1;
    if (nt > 64) nt = 64;
    pthread_t th[64];
    job_t jobs[64];
    uint64_t per = (hi - lo + nt - 1) / nt;
    for (int i = 0; i < nt; i++) {
        memset(&jobs[i], 0, sizeof jobs[i]);
        jobs[i].lo = lo + per * i;
        jobs[i].hi = lo + per * (i + 1) < hi ? lo + per * (i + 1) : hi;
        pthread_create(&th[i], NULL, run, &jobs[i]);
    }
    uint64_t b2 = 0, b4 = 0, bb = 0;
    for (int i = 0; i < nt; i++) {
        pthread_join(th[i], NULL);
        if (jobs[i].bad2 && !b2) printf("first e2m1 mismatch at 0x%08llx\n", (unsigned long long)jobs[i].first2);
        if (jobs[i].bad4 && !b4) printf("first e4m3 mismatch at 0x%08llx\n", (unsigned long long)jobs[i].first4);
        if (jobs[i].badb && !bb) printf("first bf16 mismatch at 0x%08llx\n", (unsigned long long)jobs[i].firstb);
        b2 += jobs[i].bad2; b4 += jobs[i].bad4; bb += jobs[i].badb;
    }
    printf("patterns [0x%llx, 0x%llx): e2m1 mismatches %llu, e4m3 mismatches %llu, bf16 mismatches %llu\n",
           (unsigned long long)lo, (unsigned long long)hi, (unsigned long long)b2,
           (unsigned long long)b4, (unsigned long long)bb);
    return (b2 || b4 || bb) ? 1 : 0;
}
