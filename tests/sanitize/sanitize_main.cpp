// Drives the libswa C ABI (host side, kernel launches stubbed) and the fp64
// oracle through valid and invalid calls under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Device pointers are fake addresses the host
// code never dereferences.  Prints "sanitize ok" and exits 0 when every
// expectation holds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>

#include "swa.h"

extern int g_launches;

extern "C" {
int64_t swa_oracle_attended(int64_t w, int64_t s, int64_t t, int64_t *out);
int swa_oracle_prefill_lsink(const float *Q, const float *K, const float *V, double *O, double *lse,
                             const double *sink, int B, int L, int Hq, int Hkv, int d, int64_t w, int64_t s,
                             int nthreads);
int swa_oracle_decode_lsink(const float *Q, const int64_t *pos, int64_t npos, const float *Kh, const float *Vh,
                            double *O, double *lse, const double *sink, int B, int Hq, int Hkv, int d, int64_t n,
                            int64_t w, int64_t s, int nthreads);
}

static int failures = 0;
#define EXPECT(c)                                                                  \
    do {                                                                           \
        if (!(c)) {                                                                \
            fprintf(stderr, "expectation failed: %s (line %d): %s\n", #c, __LINE__, swa_last_error()); \
            ++failures;                                                            \
        }                                                                          \
    } while (0)

static void *const DEV = (void *)0x10000;         // 16-byte aligned fake device address
static void *const DEV_MIS = (void *)0x10004;     // misaligned

static void prefill_calls()
{
    const int ws[] = {1, 5, 64, 129, 4096};
    const int ss[] = {0, 1, 4, 40};
    for (int w : ws)
        for (int s : ss) {
            if (s >= w) continue;
            for (int G : {1, 2, 4, 8})
                for (int d : {64, 128}) {
                    EXPECT(swa_prefill(DEV, DEV, DEV, DEV, nullptr, 2, 77, 4 * G, G, d, w, s, SWA_BF16, SWA_BF16,
                                       nullptr) == SWA_OK);
                    EXPECT(swa_prefill(DEV, DEV, DEV, DEV, (float *)DEV, 1, 1, G, G, d, w, s, SWA_F32, SWA_F32,
                                       nullptr) == SWA_OK);
                    EXPECT(swa_prefill_lsink(DEV, DEV, DEV, DEV, nullptr, (const float *)DEV, 1, 300, 2 * G, G, d, w,
                                             s, SWA_BF16, SWA_F32, nullptr) == SWA_OK);
                }
        }
    EXPECT(swa_prefill(DEV, DEV, DEV, DEV, nullptr, 1, 0, 4, 4, 128, 8, 4, SWA_BF16, SWA_BF16, nullptr) == SWA_OK);
    EXPECT(swa_prefill(nullptr, DEV, DEV, DEV, nullptr, 1, 8, 4, 4, 128, 8, 4, SWA_BF16, SWA_BF16, nullptr) ==
           SWA_ERR_INVALID_ARG);
    EXPECT(swa_prefill(DEV, DEV_MIS, DEV, DEV, nullptr, 1, 8, 4, 4, 128, 8, 4, SWA_BF16, SWA_BF16, nullptr) ==
           SWA_ERR_INVALID_ARG);
    EXPECT(swa_prefill(DEV, DEV, DEV, DEV, nullptr, 1, 8, 4, 4, 96, 8, 4, SWA_BF16, SWA_BF16, nullptr) ==
           SWA_ERR_UNSUPPORTED);
    EXPECT(swa_prefill(DEV, DEV, DEV, DEV, nullptr, 1, 8, 4, 4, 128, 4, 4, SWA_BF16, SWA_BF16, nullptr) ==
           SWA_ERR_INVALID_ARG);
    EXPECT(swa_prefill(DEV, DEV, DEV, DEV, nullptr, 1, 8, 6, 4, 128, 8, 4, SWA_BF16, SWA_BF16, nullptr) ==
           SWA_ERR_INVALID_ARG);
    EXPECT(swa_prefill(DEV, DEV, DEV, DEV, nullptr, 1, 8, 4, 4, 128, 8, 4, SWA_F32, SWA_BF16, nullptr) ==
           SWA_ERR_UNSUPPORTED);
    EXPECT(swa_prefill(DEV, DEV, DEV, DEV, nullptr, 1, 1 << 30, 8, 1, 128, 8, 4, SWA_BF16, SWA_BF16, nullptr) ==
           SWA_ERR_UNSUPPORTED);
    // varlen
    EXPECT(swa_prefill_varlen(DEV, DEV, DEV, DEV, nullptr, (const int32_t *)DEV, 3, 1000, 600, 32, 4, 128, 512, 4,
                              SWA_BF16, SWA_BF16, nullptr) == SWA_OK);
    EXPECT(swa_prefill_varlen(DEV, DEV, DEV, DEV, nullptr, (const int32_t *)DEV, 3, 100, 600, 32, 4, 128, 512, 4,
                              SWA_BF16, SWA_BF16, nullptr) == SWA_ERR_INVALID_ARG);
}

static void cache_calls()
{
    for (int w : {1, 2, 33, 64, 512, 576, 16384, 262144})
        for (int s : {0, 1, 4, 31}) {
            if (s >= w) continue;
            for (int B : {1, 3, 16, 64}) {
                swa_cache c;
                EXPECT(swa_cache_init(&c, DEV, DEV, B, 8, 128, w, s, SWA_BF16) == SWA_OK);
                EXPECT(swa_decode(&c, DEV, DEV, 4, nullptr, 0, nullptr) == SWA_ERR_STATE);
                const size_t ws = swa_decode_workspace_bytes(&c, 4);
                void *wsp = ws ? DEV : nullptr;
                const int steps[] = {1, 3, w - s + 3, 2 * w + 1, 1};
                for (int n_new : steps) {
                    if (n_new < 1) continue;
                    EXPECT(swa_cache_append(&c, DEV, DEV, n_new, nullptr) == SWA_OK);
                    EXPECT(swa_decode(&c, DEV, DEV, 4, wsp, ws, nullptr) == SWA_OK);
                    EXPECT(swa_decode_lsink(&c, DEV, DEV, (const float *)DEV, 8, wsp ? wsp : nullptr,
                                            swa_decode_workspace_bytes(&c, 8), nullptr) == SWA_OK ||
                           swa_decode_workspace_bytes(&c, 8) > 0);
                    const swa_status na = swa_decode_noalloc(&c, DEV, DEV, 4, nullptr);
                    EXPECT(na == SWA_OK || na == SWA_ERR_UNSUPPORTED);
                    EXPECT(swa_decode_step(&c, DEV, DEV, DEV, DEV, nullptr, 4, wsp, ws, nullptr) == SWA_OK);
                    EXPECT(swa_prefill_chunk(&c, DEV, DEV, DEV, DEV, nullptr, 5, 4, SWA_BF16, nullptr) == SWA_OK);
                    // C * G <= 16: the multi-query decode when the cache needs no split
                    EXPECT(swa_prefill_chunk(&c, DEV, DEV, DEV, DEV, nullptr, 4, 4, SWA_BF16, nullptr) == SWA_OK);
                    EXPECT(swa_prefill_chunk(&c, DEV, DEV, DEV, DEV, nullptr, 16, 1, SWA_BF16, nullptr) == SWA_OK);
                }
                if (ws) EXPECT(swa_decode(&c, DEV, DEV, 4, DEV, ws - 1, nullptr) == SWA_ERR_INVALID_ARG);
                EXPECT(swa_cache_append(&c, DEV, DEV, 0, nullptr) == SWA_ERR_INVALID_ARG);
                EXPECT(swa_cache_append(&c, DEV_MIS, DEV, 1, nullptr) == SWA_ERR_INVALID_ARG);
                const int64_t n0 = c.n;
                c.n = INT64_MAX;
                EXPECT(swa_cache_append(&c, DEV, DEV, 1, nullptr) == SWA_ERR_STATE);
                c.n = n0;
            }
            // fp8 cache
            swa_cache f;
            EXPECT(swa_cache_init(&f, DEV, DEV, 4, 8, 128, w, s, SWA_FP8_E4M3) == SWA_OK);
            EXPECT(swa_cache_append(&f, DEV, DEV, 1, nullptr) == SWA_ERR_UNSUPPORTED);
            EXPECT(swa_cache_append_fp8(&f, DEV, DEV, 2 * w + 7, (const float *)DEV, nullptr) == SWA_OK);
            EXPECT(swa_decode_fp8(&f, DEV, DEV, (const float *)DEV, nullptr, 4, DEV,
                                  swa_decode_workspace_bytes(&f, 4), nullptr) == SWA_OK);
            EXPECT(swa_decode(&f, DEV, DEV, 4, DEV, 1 << 30, nullptr) == SWA_ERR_UNSUPPORTED);
        }
    EXPECT(swa_cache_init(nullptr, DEV, DEV, 1, 1, 64, 8, 4, SWA_BF16) == SWA_ERR_INVALID_ARG);
    swa_cache c;
    EXPECT(swa_cache_init(&c, DEV, DEV, 1, 1, 64, 4, 4, SWA_BF16) == SWA_ERR_INVALID_ARG);
    EXPECT(swa_cache_init(&c, DEV, DEV, 1, 1, 80, 8, 4, SWA_BF16) == SWA_ERR_UNSUPPORTED);
}

static void paged_calls()
{
    for (int page : {32, 64, 256})
        for (int w : {64, 512, 4096}) {
            swa_paged_cache p;
            const int pps = (w + page - 1) / page;
            EXPECT(swa_paged_cache_init(&p, DEV, DEV, (const int32_t *)DEV, (int64_t *)DEV, 6, 6 * pps + 3, page, 8,
                                        128, w, 4, SWA_BF16) == SWA_OK);
            EXPECT(swa_paged_append(&p, DEV, DEV, (const int32_t *)DEV, 1234, nullptr) == SWA_OK);
            const size_t ws = swa_paged_decode_workspace_bytes(&p, 4);
            EXPECT(swa_paged_decode(&p, DEV, DEV, nullptr, 4, ws ? DEV : nullptr, ws, nullptr) == SWA_OK);
            for (swa_dtype od : {SWA_BF16, SWA_F32})
                EXPECT(swa_paged_prefill_chunk(&p, DEV, DEV, DEV, DEV, (float *)DEV, (const int32_t *)DEV, 1234,
                                               700, 4, od, nullptr) == SWA_OK);
            EXPECT(swa_paged_prefill_chunk(&p, DEV, DEV, DEV, DEV, nullptr, (const int32_t *)DEV, 0, 0, 4, SWA_BF16,
                                           nullptr) == SWA_OK);
            EXPECT(swa_paged_prefill_chunk(&p, DEV, DEV, DEV, DEV, nullptr, (const int32_t *)DEV, 10, 11, 4,
                                           SWA_BF16, nullptr) == SWA_ERR_INVALID_ARG);
            EXPECT(swa_paged_prefill_chunk(&p, DEV, DEV, DEV, DEV, nullptr, nullptr, 10, 5, 4, SWA_BF16,
                                           nullptr) == SWA_ERR_INVALID_ARG);
            EXPECT(swa_paged_prefill_chunk(&p, DEV, DEV, DEV, DEV, nullptr, (const int32_t *)DEV, 10, 5, 3,
                                           SWA_BF16, nullptr) == SWA_ERR_UNSUPPORTED);
            EXPECT(swa_paged_prefill_chunk(&p, DEV, DEV, DEV, DEV, nullptr, (const int32_t *)DEV, 10, 5, 4,
                                           SWA_FP8_E4M3, nullptr) == SWA_ERR_UNSUPPORTED);
        }
    swa_paged_cache p;
    EXPECT(swa_paged_cache_init(&p, DEV, DEV, (const int32_t *)DEV, (int64_t *)DEV, 6, 30, 48, 8, 128, 512, 4,
                                SWA_BF16) == SWA_ERR_UNSUPPORTED);
}

static void host_functions()
{
    for (int w = 1; w <= 40; ++w)
        for (int s = 0; s < w; ++s)
            for (int64_t p = 1; p <= 200; ++p) {
                const int64_t j = swa_cache_slot(w, s, p);
                EXPECT(j >= 0 && j < w);
                EXPECT(swa_attended_count(w, s, p) == (p < w ? p : w));
            }
    EXPECT(swa_cache_slot(8, 8, 3) == -1 && swa_attended_count(4, -1, 3) == -1);
    EXPECT(swa_cache_slot(262144, 4, INT64_MAX) >= 4);
}

static double urand(uint64_t *st)
{
    *st = *st * 6364136223846793005ull + 1442695040888963407ull;
    return ((double)(*st >> 11) / 9007199254740992.0) * 2.0 - 1.0;
}

static void oracle_calls()
{
    uint64_t rng = 12345;
    const int B = 2, L = 70, Hq = 8, Hkv = 2, d = 64;
    float *Q = (float *)malloc(sizeof(float) * B * L * Hq * d);
    float *K = (float *)malloc(sizeof(float) * B * L * Hkv * d);
    float *V = (float *)malloc(sizeof(float) * B * L * Hkv * d);
    double *O = (double *)malloc(sizeof(double) * B * L * Hq * d);
    double *lse = (double *)malloc(sizeof(double) * B * Hq * L);
    double sink[Hq];
    for (int i = 0; i < B * L * Hq * d; ++i) Q[i] = (float)urand(&rng);
    for (int i = 0; i < B * L * Hkv * d; ++i) {
        K[i] = (float)urand(&rng);
        V[i] = (float)urand(&rng);
    }
    for (int h = 0; h < Hq; ++h) sink[h] = h == 0 ? -INFINITY : urand(&rng) * 4.0;
    for (int w : {1, 7, 33, 100})
        for (int s : {0, 3}) {
            if (s >= w) continue;
            EXPECT(swa_oracle_prefill_lsink(Q, K, V, O, lse, nullptr, B, L, Hq, Hkv, d, w, s, 3) == 0);
            EXPECT(swa_oracle_prefill_lsink(Q, K, V, O, lse, sink, B, L, Hq, Hkv, d, w, s, 2) == 0);
            for (int i = 0; i < B * L * Hq * d; ++i) EXPECT(isfinite(O[i]));
            // decode at the last position from the full history
            int64_t pos[L];
            for (int p = 0; p < L; ++p) pos[p] = p + 1;
            double Od[B * Hq * d], ld[B * Hq];
            EXPECT(swa_oracle_decode_lsink(Q, pos, L, K, V, Od, ld, sink, B, Hq, Hkv, d, L, w, s, 2) == 0);
            // a history missing a member of S_n is reported, not read past
            EXPECT(swa_oracle_decode_lsink(Q, pos, L - 1, K, V, Od, ld, nullptr, B, Hq, Hkv, d, L, w, s, 1) != 0);
        }
    int64_t out[300];
    for (int64_t t = 1; t <= 300; ++t) EXPECT(swa_oracle_attended(64, 4, t, out) == (t < 64 ? t : 64));
    EXPECT(swa_oracle_attended(4, 4, 3, out) < 0);
    free(Q);
    free(K);
    free(V);
    free(O);
    free(lse);
}

int main()
{
    prefill_calls();
    cache_calls();
    paged_calls();
    host_functions();
    oracle_calls();
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("sanitize ok: %d stubbed launches checked\n", g_launches);
    return 0;
}
