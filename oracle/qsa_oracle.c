/*
 * qsa_oracle.c -- sequential CPU oracle for physically sparse QSA attention.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
 * benchmark).  Plain C11, one thread, no blocking, fusion or reordering
 * beyond what each step's definition states.  Build with
 *   gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 *
 * Sources:
 *   [SET]  AFN-017 "Top-k chooses the set; time chooses the order"
 *   [MASK] AFN-016 "A sparse mask is not sparse attention"
 *
 * What pins each function (tests/test_oracle_*.py, all CPU):
 *   oracle_pool_full / _incremental: grid-valued raw keys give pooled values
 *     that are exact multiples of 1/32, recomputed in integers; full and
 *     incremental pooling agree bit for bit; hand-worked golden example.
 *   oracle_score: grid-valued keys and queries make every score exact, and
 *     an integer recomputation must match it bit for bit; Gaussian inputs
 *     must sit within the closed-form rounding bound of a float64
 *     evaluation; hand-worked golden example.
 *   oracle_select: an independent O(G^2) rank count on small inputs; all
 *     scores equal selects groups 0..k-1; g <= k selects everything; a tied
 *     block at the threshold keeps its lowest positions; golden tie example.
 *   oracle_emit: strictly ascending IDs, runs of four aligned to multiples
 *     of four, tail equal to 4G..N-1; the dense-parity sweep (ids = 0..N-1
 *     whenever N <= 4k+3).
 *   oracle_resolve / oracle_gather: identity, ring-offset and permutation
 *     closed forms; bitwise equality with direct cache indexing.
 *   oracle_attend_online: one row gives that V row exactly; identical keys
 *     give the mean of V; within a derived bound of oracle_attend_exact.
 *   oracle_attend_exact: numpy float64 softmax-weighted sum (library
 *     routine) to 1e-12.
 *   oracle_decode_row vs oracle_dense_row: equal bit for bit below budget.
 */
#include "qsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- O1 -- */

void oracle_pool_full(const float *raw, int64_t n_tokens, int32_t d_i, float *pooled)
{
    int64_t groups = n_tokens / ORACLE_GROUP;
    for (int64_t g = 0; g < groups; ++g) {
        const float *r = raw + (g * ORACLE_GROUP) * (int64_t)d_i;
        for (int32_t d = 0; d < d_i; ++d) {
            float s = r[d];
            s = s + r[(int64_t)d_i + d];
            s = s + r[2 * (int64_t)d_i + d];
            s = s + r[3 * (int64_t)d_i + d];
            pooled[g * d_i + d] = s * 0.25f;
        }
    }
}

void oracle_pool_incremental(const float *raw, int64_t n_tokens, int32_t d_i,
                             float *pooled, float *partial)
{
    for (int64_t t = 0; t < n_tokens; ++t) {
        const float *r = raw + t * (int64_t)d_i;
        int64_t j = t % ORACLE_GROUP;
        for (int32_t d = 0; d < d_i; ++d) {
            if (j == 0)
                partial[d] = r[d];
            else
                partial[d] = partial[d] + r[d];
        }
        if (j == ORACLE_GROUP - 1) {
            int64_t g = t / ORACLE_GROUP;
            for (int32_t d = 0; d < d_i; ++d)
                pooled[g * d_i + d] = partial[d] * 0.25f;
        }
    }
}

/* ---------------------------------------------------------------- O2 -- */

void oracle_score(const float *qi, const float *pooled, int64_t g, int32_t h_i,
                  int32_t d_i, float *scores)
{
    for (int64_t j = 0; j < g; ++j) {
        const float *k = pooled + j * d_i;
        float s = 0.0f;
        for (int32_t h = 0; h < h_i; ++h) {
            const float *qh = qi + (int64_t)h * d_i;
            float a = 0.0f;
            for (int32_t d = 0; d < d_i; ++d)
                a = fmaf(qh[d], k[d], a);
            s = s + ((a > 0.0f) ? a : 0.0f);
        }
        scores[j] = s;
    }
}

/* ---------------------------------------------------------------- O3 -- */

typedef struct {
    float score;
    int64_t pos;
} ranked;

/* Total order of the notes: higher score first; equal scores, lower
 * logical group position first. */
static int rank_cmp(const void *pa, const void *pb)
{
    const ranked *a = (const ranked *)pa;
    const ranked *b = (const ranked *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    if (a->pos < b->pos) return -1;
    if (a->pos > b->pos) return 1;
    return 0;
}

int64_t oracle_select(const float *scores, int64_t g, int32_t k, int64_t *chosen)
{
    int64_t m = (g < (int64_t)k) ? g : (int64_t)k;
    if (m <= 0) return 0;
    ranked *all = (ranked *)malloc((size_t)g * sizeof(ranked));
    if (!all) return -1;
    for (int64_t j = 0; j < g; ++j) {
        all[j].score = scores[j];
        all[j].pos = j;
    }
    qsort(all, (size_t)g, sizeof(ranked), rank_cmp);
    for (int64_t i = 0; i < m; ++i) chosen[i] = all[i].pos;
    free(all);
    return m;
}

/* ------------------------------------------------------------- O4-O6 -- */

static int pos_cmp(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    return (a > b) - (a < b);
}

int32_t oracle_emit(const int64_t *chosen, int64_t m, int64_t n_tokens, int32_t *ids)
{
    int64_t *order = NULL;
    if (m > 0) {
        order = (int64_t *)malloc((size_t)m * sizeof(int64_t));
        if (!order) return -1;
        memcpy(order, chosen, (size_t)m * sizeof(int64_t));
        qsort(order, (size_t)m, sizeof(int64_t), pos_cmp);           /* O4 */
    }
    int32_t w = 0;
    for (int64_t i = 0; i < m; ++i)                                   /* O5 */
        for (int32_t j = 0; j < ORACLE_GROUP; ++j)
            ids[w++] = (int32_t)(order[i] * ORACLE_GROUP + j);
    int64_t full = (n_tokens / ORACLE_GROUP) * ORACLE_GROUP;
    for (int64_t t = full; t < n_tokens; ++t)                         /* O6 */
        ids[w++] = (int32_t)t;
    free(order);
    return w;
}

/* ------------------------------------------------------------- O7-O8 -- */

int32_t oracle_resolve(const int32_t *ids, int32_t w, const int32_t *slot_map,
                       int64_t map_len, int64_t kv_slots, int32_t *slots)
{
    for (int32_t i = 0; i < w; ++i) {
        if (ids[i] < 0 || (int64_t)ids[i] >= map_len) return -1;
        int32_t s = slot_map[ids[i]];
        if (s < 0 || (int64_t)s >= kv_slots) return -1;
        slots[i] = s;
    }
    return 0;
}

void oracle_gather(const int32_t *slots, int32_t w, const float *k_cache,
                   const float *v_cache, int64_t row_elems, float *k_out, float *v_out)
{
    for (int32_t i = 0; i < w; ++i) {
        memcpy(k_out + (int64_t)i * row_elems, k_cache + (int64_t)slots[i] * row_elems,
               (size_t)row_elems * sizeof(float));
        memcpy(v_out + (int64_t)i * row_elems, v_cache + (int64_t)slots[i] * row_elems,
               (size_t)row_elems * sizeof(float));
    }
}

/* ---------------------------------------------------------------- O9 -- */

void oracle_attend_online(const float *q, const float *kx, const float *vx, int32_t w,
                          int32_t h_q, int32_t h_kv, int32_t d, float scale,
                          float *out, float *lse)
{
    int32_t group = h_q / h_kv;
    float *acc = (float *)malloc((size_t)d * sizeof(float));
    for (int32_t hq = 0; hq < h_q; ++hq) {
        int32_t hk = hq / group;
        const float *qh = q + (int64_t)hq * d;
        float m = -INFINITY, l = 0.0f;
        for (int32_t c = 0; c < d; ++c) acc[c] = 0.0f;
        for (int32_t i = 0; i < w; ++i) {
            const float *kr = kx + ((int64_t)i * h_kv + hk) * d;
            const float *vr = vx + ((int64_t)i * h_kv + hk) * d;
            float dot = 0.0f;
            for (int32_t c = 0; c < d; ++c) dot = fmaf(qh[c], kr[c], dot);
            float s = dot * scale;
            float m_new = fmaxf(m, s);
            float alpha = expf(m - m_new);    /* 0 on the first row: exp(-inf) */
            float p = expf(s - m_new);
            l = l * alpha;
            l = l + p;
            for (int32_t c = 0; c < d; ++c) {
                float a = acc[c] * alpha;
                float b = p * vr[c];
                acc[c] = a + b;
            }
            m = m_new;
        }
        for (int32_t c = 0; c < d; ++c)
            out[(int64_t)hq * d + c] = (w > 0) ? acc[c] / l : 0.0f;
        if (lse) lse[hq] = (w > 0) ? m + logf(l) : -INFINITY;
    }
    free(acc);
}

void oracle_attend_exact(const float *q, const float *kx, const float *vx, int32_t w,
                         int32_t h_q, int32_t h_kv, int32_t d, double scale,
                         double *out, double *lse)
{
    int32_t group = h_q / h_kv;
    double *s = (double *)malloc((size_t)(w > 0 ? w : 1) * sizeof(double));
    for (int32_t hq = 0; hq < h_q; ++hq) {
        int32_t hk = hq / group;
        const float *qh = q + (int64_t)hq * d;
        double mx = -INFINITY;
        for (int32_t i = 0; i < w; ++i) {
            const float *kr = kx + ((int64_t)i * h_kv + hk) * d;
            double dot = 0.0;
            for (int32_t c = 0; c < d; ++c) dot += (double)qh[c] * (double)kr[c];
            s[i] = dot * scale;
            if (s[i] > mx) mx = s[i];
        }
        double den = 0.0;
        for (int32_t i = 0; i < w; ++i) den += exp(s[i] - mx);
        for (int32_t c = 0; c < d; ++c) {
            double num = 0.0;
            for (int32_t i = 0; i < w; ++i)
                num += exp(s[i] - mx) * (double)vx[((int64_t)i * h_kv + hk) * d + c];
            out[(int64_t)hq * d + c] = (w > 0) ? num / den : 0.0;
        }
        if (lse) lse[hq] = (w > 0) ? mx + log(den) : -INFINITY;
    }
    free(s);
}

/* ----------------------------------------------------------- O2-O10 -- */

int32_t oracle_decode_row(const float *qi, const float *pooled, int64_t n_tokens,
                          int32_t h_i, int32_t d_i, int32_t k,
                          const int32_t *slot_map, int64_t map_len, int64_t kv_slots,
                          const float *k_cache, const float *v_cache, int32_t h_kv,
                          int32_t d, const float *q, int32_t h_q, float scale,
                          float *scores, int64_t *chosen, int32_t *ids, int32_t *slots,
                          float *kx, float *vx, float *out, float *lse)
{
    int64_t g = n_tokens / ORACLE_GROUP;
    oracle_score(qi, pooled, g, h_i, d_i, scores);
    int64_t m = oracle_select(scores, g, k, chosen);
    if (m < 0) return -1;
    int32_t w = oracle_emit(chosen, m, n_tokens, ids);
    if (w < 0) return -1;
    if (oracle_resolve(ids, w, slot_map, map_len, kv_slots, slots) != 0) return -1;
    oracle_gather(slots, w, k_cache, v_cache, (int64_t)h_kv * d, kx, vx);
    oracle_attend_online(q, kx, vx, w, h_q, h_kv, d, scale, out, lse);
    return w;
}

int32_t oracle_dense_row(int64_t n_tokens, const int32_t *slot_map, int64_t map_len,
                         int64_t kv_slots, const float *k_cache, const float *v_cache,
                         int32_t h_kv, int32_t d, const float *q, int32_t h_q, float scale,
                         int32_t *ids, int32_t *slots, float *kx, float *vx,
                         float *out, float *lse)
{
    int32_t w = (int32_t)n_tokens;
    for (int32_t i = 0; i < w; ++i) ids[i] = i;
    if (oracle_resolve(ids, w, slot_map, map_len, kv_slots, slots) != 0) return -1;
    oracle_gather(slots, w, k_cache, v_cache, (int64_t)h_kv * d, kx, vx);
    oracle_attend_online(q, kx, vx, w, h_q, h_kv, d, scale, out, lse);
    return w;
}
