/*
 * selftest.c -- drives every oracle entry point on seeded inputs so that a
 * build with -fsanitize=address,undefined can flag any out-of-bounds access,
 * leak or undefined operation in the oracle (the notes' host ASan/UBSan
 * lanes, AFN-016 capsule evidence).  TEST INFRASTRUCTURE ONLY.
 * Exit status 0 = every structural check held.
 */
#include "qsa_oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void)
{
    /* splitmix64 (Steele, Lea, Flood 2014) */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static float next_grid(void) { return (float)((int)(next_u64() % 5) - 2) / 8.0f; }

static int run_case(int64_t n, int32_t h_i, int32_t d_i, int32_t k, int32_t h_q,
                    int32_t h_kv, int32_t d)
{
    int64_t g = n / 4;
    int32_t wmax = 4 * k + 4;
    float *raw = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1) * d_i);
    float *pooled = malloc(sizeof(float) * (size_t)(g > 0 ? g : 1) * d_i);
    float *pooled2 = malloc(sizeof(float) * (size_t)(g > 0 ? g : 1) * d_i);
    float *partial = malloc(sizeof(float) * d_i);
    float *qi = malloc(sizeof(float) * h_i * d_i);
    float *q = malloc(sizeof(float) * h_q * d);
    float *kc = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1) * h_kv * d);
    float *vc = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1) * h_kv * d);
    int32_t *map = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    float *scores = malloc(sizeof(float) * (size_t)(g > 0 ? g : 1));
    int64_t *chosen = malloc(sizeof(int64_t) * (size_t)(k > 0 ? k : 1));
    int32_t *ids = malloc(sizeof(int32_t) * wmax);
    int32_t *ids2 = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int32_t *slots = malloc(sizeof(int32_t) * (size_t)(n > wmax ? n : wmax));
    float *kx = malloc(sizeof(float) * (size_t)(n > wmax ? n : wmax) * h_kv * d);
    float *vx = malloc(sizeof(float) * (size_t)(n > wmax ? n : wmax) * h_kv * d);
    float *out = malloc(sizeof(float) * h_q * d);
    float *out2 = malloc(sizeof(float) * h_q * d);
    float *lse = malloc(sizeof(float) * h_q);
    double *oute = malloc(sizeof(double) * h_q * d);
    double *lsee = malloc(sizeof(double) * h_q);
    int bad = 0;

    for (int64_t i = 0; i < n * d_i; ++i) raw[i] = next_grid();
    for (int32_t i = 0; i < h_i * d_i; ++i) qi[i] = next_grid();
    for (int32_t i = 0; i < h_q * d; ++i) q[i] = next_grid();
    for (int64_t i = 0; i < n * h_kv * d; ++i) { kc[i] = next_grid(); vc[i] = next_grid(); }
    for (int64_t i = 0; i < n; ++i) map[i] = (int32_t)(n - 1 - i);

    oracle_pool_full(raw, n, d_i, pooled);
    oracle_pool_incremental(raw, n, d_i, pooled2, partial);
    for (int64_t i = 0; i < g * d_i; ++i) bad |= (pooled[i] != pooled2[i]);

    int32_t w = oracle_decode_row(qi, pooled, n, h_i, d_i, k, map, n, n, kc, vc, h_kv, d,
                                  q, h_q, 0.125f, scores, chosen, ids, slots, kx, vx, out, lse);
    int64_t m = g < k ? g : k;
    bad |= (w != (int32_t)(4 * m + n % 4));
    for (int32_t i = 1; i < w; ++i) bad |= (ids[i] <= ids[i - 1]);
    oracle_attend_exact(q, kx, vx, w, h_q, h_kv, d, 0.125, oute, lsee);
    for (int32_t i = 0; i < h_q * d; ++i) bad |= (w > 0 && fabs(out[i] - oute[i]) > 1e-3);

    if (g <= k) {
        int32_t wd = oracle_dense_row(n, map, n, n, kc, vc, h_kv, d, q, h_q, 0.125f, ids2,
                                      slots, kx, vx, out2, lse);
        bad |= (wd != w);
        for (int32_t i = 0; i < h_q * d; ++i) bad |= (out[i] != out2[i]);
    }
    /* an out-of-range slot map entry is reported, not dereferenced */
    if (n > 0) {
        map[0] = (int32_t)n;
        int32_t probe = 0;
        bad |= (oracle_resolve(&probe, 1, map, n, n, slots) != -1);
    }

    free(raw); free(pooled); free(pooled2); free(partial); free(qi); free(q); free(kc);
    free(vc); free(map); free(scores); free(chosen); free(ids); free(ids2); free(slots);
    free(kx); free(vx); free(out); free(out2); free(lse); free(oute); free(lsee);
    return bad;
}

int main(void)
{
    int bad = 0;
    const int64_t lens[] = {0, 1, 3, 4, 5, 7, 64, 2047, 2051, 2052, 2055, 5000};
    for (size_t i = 0; i < sizeof(lens) / sizeof(lens[0]); ++i) {
        bad |= run_case(lens[i], 4, 32, 512, 1, 1, 64);
        bad |= run_case(lens[i], 2, 16, 8, 4, 2, 16);
    }
    printf("oracle selftest: %s\n", bad ? "FAIL" : "ok");
    return bad;
}
