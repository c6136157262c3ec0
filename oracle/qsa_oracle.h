/*
 * qsa_oracle.h -- sequential CPU oracle for physically sparse QSA attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The HIP product
 * path never links, includes or calls it, and it shares no code with that
 * path.
 *
 * Sources (the two notes of the Hebrus project, Phase 6):
 *   [SET]  AFN-017 "Top-k chooses the set; time chooses the order"
 *   [MASK] AFN-016 "A sparse mask is not sparse attention"
 *
 * Every floating-point step is single precision with an explicit, fixed
 * operation order (the notes state that the path is F32), except the
 * *_exact functions, which evaluate the plain mathematical definition in
 * double precision.  Compile with -ffp-contract=off and without fast-math.
 *
 * Pins: each function is checked against closed forms, brute force or the
 * double-precision definition by the CPU tests; see the header of
 * qsa_oracle.c for the list.
 */
#ifndef QSA_ORACLE_H
#define QSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Group size: QSA ranks complete four-token groups ([SET] §Decision). */
#define ORACLE_GROUP 4

/* O1. Full pooling.  raw is [n_tokens][d_i] (logical order); pooled receives
 * [floor(n_tokens/4)][d_i]: the mean of each complete group's four raw index
 * keys, evaluated as (((r0 + r1) + r2) + r3) * 0.25f ([MASK] §Why a sparse
 * mask can still be dense: complete groups are pooled, the raw cache is kept). */
void oracle_pool_full(const float *raw, int64_t n_tokens, int32_t d_i, float *pooled);

/* O1'. Incremental pooling: tokens arrive one at a time; a running partial
 * sum (partial, [d_i]) is carried between arrivals and a pooled row is
 * written when the fourth token of a group arrives.  Must equal
 * oracle_pool_full bit for bit ([SET] capsule evidence: full-raw/incremental
 * identity). */
void oracle_pool_incremental(const float *raw, int64_t n_tokens, int32_t d_i,
                             float *pooled, float *partial);

/* O2. Group scores.  qi is [h_i][d_i], pooled is [g][d_i], scores [g].
 * score = sum over heads h (ascending) of ReLU(dot_h), dot_h a sequential
 * fmaf chain over d ascending starting from +0 ([MASK] §Decision: groups are
 * scored; §Why a sparse mask can still be dense: the sum(ReLU(dot_h))
 * ordering, ReLU per head before the head sum). */
void oracle_score(const float *qi, const float *pooled, int64_t g, int32_t h_i,
                  int32_t d_i, float *scores);

/* O3. Top-k membership by (score descending, group position ascending)
 * ([SET] §Decision and §Tie handling belongs to membership).  Writes the
 * min(g, k) chosen groups to chosen[] in rank order and returns that count.
 * Scores must not be NaN. */
int64_t oracle_select(const float *scores, int64_t g, int32_t k, int64_t *chosen);

/* O4-O6. Emission ([SET] §Decision): the chosen groups sorted by logical
 * position, each expanded to four consecutive token IDs, then the raw tail
 * (n_tokens mod 4 tokens, starting at 4*floor(n_tokens/4)).  ids receives
 * the row; the return value is its width 4m + tail. */
int32_t oracle_emit(const int64_t *chosen, int64_t m, int64_t n_tokens, int32_t *ids);

/* O7. One-time slot resolution through the shared slot map ([MASK]
 * §Decision: only the gather crosses into physical layout).  Returns 0, or
 * -1 if an ID is outside [0, map_len) or a slot outside [0, kv_slots). */
int32_t oracle_resolve(const int32_t *ids, int32_t w, const int32_t *slot_map,
                       int64_t map_len, int64_t kv_slots, int32_t *slots);

/* O8. Compact gather of the selected K/V rows ([MASK] §Why compact gather
 * comes before fusion).  A cache row is row_elems = h_kv*d floats. */
void oracle_gather(const int32_t *slots, int32_t w, const float *k_cache,
                   const float *v_cache, int64_t row_elems, float *k_out, float *v_out);

/* O9. F32 online softmax over the compact row in the given (chronological)
 * order: running maximum, rescale, exponent, denominator and accumulator
 * updates ([SET] §Floating point makes order observable).  q is [h_q][d],
 * kx/vx are [w][h_kv][d]; query head hq reads KV head hq / (h_q/h_kv).
 * out is [h_q][d]; lse [h_q] may be NULL.  w == 0 gives out = +0, lse = -inf. */
void oracle_attend_online(const float *q, const float *kx, const float *vx, int32_t w,
                          int32_t h_q, int32_t h_kv, int32_t d, float scale,
                          float *out, float *lse);

/* O9-exact. The definition softmax(scale * q . k) . v evaluated in double
 * precision with a two-pass (max, then sum) softmax.  Same layouts as O9. */
void oracle_attend_exact(const float *q, const float *kx, const float *vx, int32_t w,
                         int32_t h_q, int32_t h_kv, int32_t d, double scale,
                         double *out, double *lse);

/* O2-O9 for one decode row over a plain [g][d_i] pooled buffer and a host
 * K/V cache.  ids must hold 4k+4 entries, slots the same; kx/vx hold
 * (4k+3)*h_kv*d floats.  Returns the width, or -1 on a resolution error. */
int32_t oracle_decode_row(const float *qi, const float *pooled, int64_t n_tokens,
                          int32_t h_i, int32_t d_i, int32_t k,
                          const int32_t *slot_map, int64_t map_len, int64_t kv_slots,
                          const float *k_cache, const float *v_cache, int32_t h_kv,
                          int32_t d, const float *q, int32_t h_q, float scale,
                          float *scores, int64_t *chosen, int32_t *ids, int32_t *slots,
                          float *kx, float *vx, float *out, float *lse);

/* O10. The bounded dense causal row: every visible token 0..n_tokens-1 in
 * order, resolved, gathered and attended exactly like O7-O9 (the dense
 * oracle the notes keep for rows up to 2,051 keys).  Returns n_tokens or -1. */
int32_t oracle_dense_row(int64_t n_tokens, const int32_t *slot_map, int64_t map_len,
                         int64_t kv_slots, const float *k_cache, const float *v_cache,
                         int32_t h_kv, int32_t d, const float *q, int32_t h_q, float scale,
                         int32_t *ids, int32_t *slots, float *kx, float *vx,
                         float *out, float *lse);

#ifdef __cplusplus
}
#endif
#endif
