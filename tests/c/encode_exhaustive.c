/* Every one of the 2^32 fp32 bit patterns through three fp32 -> fp16 and
 * fp32 -> bf16 encoders that share no code:
 *   - a reference written here from the IEEE-754 definition with integer
 *     arithmetic only (the value is M * 2^E exactly; it is cut to the
 *     format's quantum and rounded to nearest, ties to the even code);
 *   - the oracle's encoders (liboracle.so);
 *   - the library's host cast, reached through zero_host_adamw with lr = 0,
 *     weight decay 0 and a zero gradient, where the update leaves every
 *     master unchanged (p * 1 - 0 * 0), so its output is the cast alone.
 * NaN inputs must give a NaN code in all three (payloads may differ).
 * Usage: encode_exhaustive [threads].  Prints a summary; exit 0 when all
 * agree. */
#include <pthread.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero.h"
#include "zero_oracle.h"

static uint16_t ref_bf16(uint32_t u) {
    const uint32_t sign = (u >> 16) & 0x8000u, a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7fc0u);
    /* bf16 keeps the upper 16 bits: round on the lower 16 (a carry out of
     * the largest finite value reaches the infinity code, as it should) */
    uint32_t keep = a >> 16;
    const uint32_t rest = a & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)(sign | keep);
}

static uint16_t ref_f16(uint32_t u) {
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);
    if (a == 0x7f800000u) return (uint16_t)(sign | 0x7c00u);
    if (a == 0) return sign;
    const int e = (int)(a >> 23);
    const uint64_t M = (a & 0x7fffffu) | (e ? 0x800000u : 0u);   /* value = M * 2^E */
    const int E = (e ? e : 1) - 150;
    const int L = 63 - __builtin_clzll(M);                        /* leading bit of M */
    const int lead = L + E;                                       /* floor(log2 value) */
    const int qexp = (lead < -14 ? -14 : lead) - 10;              /* fp16 quantum 2^qexp */
    const int sh = qexp - E;                                      /* > 0 for every input */
    if (sh >= 40) return sign;                                    /* below half a quantum */
    uint64_t units = M >> sh;
    const uint64_t rem = M & ((1ull << sh) - 1ull), half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (units & 1ull))) units += 1ull;
    if (qexp == -24)             /* quantum of the subnormals and of the first binade */
        return (uint16_t)(sign | units);      /* units <= 2048: the code is the count */
    int exp16 = qexp + 10;
    if (units == 2048u) {
        units = 1024u;
        exp16 += 1;
    }
    if (exp16 > 15) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)(((exp16 + 15) << 10) | (uint32_t)(units - 1024u)));
}

static int is_nan16(uint16_t c, int bf) {
    return bf ? ((c & 0x7f80u) == 0x7f80u && (c & 0x7fu)) : ((c & 0x7c00u) == 0x7c00u && (c & 0x3ffu));
}

enum { CHUNK = 1 << 20 };

typedef struct {
    uint64_t lo, hi;
    uint64_t bad[2][2];   /* [oracle, library][f16, bf16] */
    int error;
} Job;

static void* run(void* arg) {
    Job* j = (Job*)arg;
    float* x = malloc(CHUNK * sizeof(float));
    float* zero = calloc(CHUNK, sizeof(float));
    float* mm = malloc(CHUNK * sizeof(float));
    float* vv = malloc(CHUNK * sizeof(float));
    uint16_t* got = malloc(CHUNK * sizeof(uint16_t));
    if (!x || !zero || !mm || !vv || !got) {
        j->error = 1;
        return NULL;
    }
    for (uint64_t base = j->lo; base < j->hi; base += CHUNK) {
        const int64_t n = (int64_t)((j->hi - base) < CHUNK ? (j->hi - base) : CHUNK);
        for (int bf = 0; bf < 2; ++bf) {
            for (int impl = 0; impl < 2; ++impl) {
                for (int64_t i = 0; i < n; ++i) {
                    const uint32_t u = (uint32_t)(base + (uint64_t)i);
                    memcpy(&x[i], &u, 4);
                }
                if (impl == 0) {
                    if (bf) oracle_f32_to_bf16_array(n, x, got);
                    else oracle_f32_to_f16_array(n, x, got);
                } else {
                    memset(mm, 0, (size_t)n * sizeof(float));
                    memset(vv, 0, (size_t)n * sizeof(float));
                    if (zero_host_adamw(n, zero, 1.0f, x, mm, vv, got, bf ? ZERO_BF16 : ZERO_FP16,
                                        0.0, 0.9, 0.999, 1e-8, 0.0, 1, 1) != ZERO_OK) {
                        j->error = 2;
                        return NULL;
                    }
                }
                for (int64_t i = 0; i < n; ++i) {
                    const uint32_t u = (uint32_t)(base + (uint64_t)i);
                    const uint16_t want = bf ? ref_bf16(u) : ref_f16(u);
                    const int ok = is_nan16(want, bf) ? is_nan16(got[i], bf) : got[i] == want;
                    if (!ok) {
                        if (j->bad[impl][bf] < 3)
                            printf("%s %s: pattern 0x%08x gives 0x%04x, reference 0x%04x\n",
                                   impl ? "library" : "oracle", bf ? "bf16" : "f16", u, got[i], want);
                        j->bad[impl][bf]++;
                    }
                }
            }
        }
    }
    free(x); free(zero); free(mm); free(vv); free(got);
    return NULL;
}

int main(int argc, char** argv) {
    int nt = argc > 1 ? atoi(argv[1]) : 8;
    if (nt < 1 || nt > 256) nt = 8;
    const uint64_t total = 1ull << 32;
    pthread_t th[256];
    Job jobs[256];
    const uint64_t per = (total / (uint64_t)nt + CHUNK - 1) / CHUNK * CHUNK;
    for (int t = 0; t < nt; ++t) {
        memset(&jobs[t], 0, sizeof jobs[t]);
        jobs[t].lo = per * (uint64_t)t < total ? per * (uint64_t)t : total;
        jobs[t].hi = per * (uint64_t)(t + 1) < total ? per * (uint64_t)(t + 1) : total;
        pthread_create(&th[t], NULL, run, &jobs[t]);
    }
    uint64_t bad[2][2] = {{0, 0}, {0, 0}};
    int error = 0;
    for (int t = 0; t < nt; ++t) {
        pthread_join(th[t], NULL);
        error |= jobs[t].error;
        for (int a = 0; a < 2; ++a)
            for (int b = 0; b < 2; ++b) bad[a][b] += jobs[t].bad[a][b];
    }
    printf("mismatches: oracle f16 %llu, oracle bf16 %llu, library f16 %llu, library bf16 %llu\n",
           (unsigned long long)bad[0][0], (unsigned long long)bad[0][1],
           (unsigned long long)bad[1][0], (unsigned long long)bad[1][1]);
    if (error) {
        printf("error %d\n", error);
        return 2;
    }
    if (bad[0][0] | bad[0][1] | bad[1][0] | bad[1][1]) return 1;
    printf("all %llu patterns agree\n", (unsigned long long)total);
    return 0;
}
