/*
 * qsa.h -- physically sparse QSA attention for decode on AMD Instinct MI355X
 * (gfx950): the C ABI of libqsa.so.
 *
 * For one query row the path is
 *   1. score every complete four-token group of the visible history,
 *   2. choose the top-k set by (score descending, group position ascending),
 *   3. emit the chosen group IDs in ascending logical position,
 *   4. expand each group to its four consecutive token IDs,
 *   5. append the raw tail of up to three tokens,
 *   6. resolve the logical token IDs once through the slot map,
 *   7. gather only those K/V rows into bounded compact scratch,
 *   8. run an F32 online softmax over the (at most 4k+3) compact rows.
 * No buffer of size rows x tokens (a dense mask) exists anywhere.
 *
 * Sources (Hebrus Phase 6 notes):
 *   [SET]  AFN-017 "Top-k chooses the set; time chooses the order"
 *   [MASK] AFN-016 "A sparse mask is not sparse attention"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named *_host are host memory; every other pointer is DEVICE
 *   memory owned by the caller.  The library allocates no device memory in
 *   these calls, keeps no state between calls and enqueues its kernels
 *   asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 * - Rows: the call covers batch*queries rows; row r = b*queries + j is query
 *   j of sequence b and sees N = seq_len[b] - queries + 1 + j tokens
 *   (decode: queries = 1, N = seq_len[b]).  It has G = floor(N/4) complete
 *   groups and a tail of N mod 4 tokens.
 * - Return value: QSA_OK, or a qsa_status code.  Host-side validation runs
 *   before anything is enqueued, so on an error no output is touched.
 *   QSA_ERR_HIP reports a failed launch (hipGetLastError).
 * - Device-side data errors never fault: a row whose N is negative or whose
 *   G exceeds shape->max_groups gets width -1, token IDs -1 and NaN outputs;
 *   a logical ID outside [0, seq_len[b]) or a mapped slot outside
 *   [0, kv_slots) yields NaN compact rows and phys slot -1.
 * - Calls are thread-safe given distinct output buffers and workspaces.
 * - All floating point is IEEE single precision, round to nearest even,
 *   denormals kept.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define QSA_API __attribute__((visibility("default")))
#else
#define QSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_GROUP 4          /* tokens per group ([SET] §Decision)                 */
#define QSA_MAX_BUDGET 1024  /* largest supported k (the notes use k = 512)        */
#define QSA_KEY_TILE 64      /* groups per pooled-key tile (layout below)          */
#define QSA_DECODE_STAGES 5  /* stages timed by qsa_timer in one qsa_decode call:
                                score, select+emit, resolve+gather, attention
                                chunks, merge of the range partials               */

typedef void *qsa_stream; /* a hipStream_t */

typedef enum {
    QSA_OK = 0,
    QSA_ERR_NULL = 1,        /* a required pointer is NULL                      */
    QSA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent          */
    QSA_ERR_BUDGET = 3,      /* budget_groups outside [1, QSA_MAX_BUDGET]       */
    QSA_ERR_WORKSPACE = 4,   /* workspace smaller than qsa_workspace_bytes()    */
    QSA_ERR_HIP = 5,         /* a HIP call or kernel launch failed              */
    QSA_ERR_UNSUPPORTED = 6, /* a valid shape this build has no kernel for      */
    QSA_ERR_STATIC_WORKSPACE = 7 /* qsa_decode_noalloc: the shape needs more than
                                    QSA_NOALLOC_WORKSPACE_BYTES of workspace      */
} qsa_status;

/* Problem shape.  Supported: index_dim in {32, 64, 128}; index_heads in
 * {1, 2, 4, 8, 16}; head_dim in {64, 128}; q_heads = g * kv_heads with
 * g in {1, 2, 4, 8, 16}. */
typedef struct qsa_shape {
    int32_t batch;          /* B sequences                                          */
    int32_t queries;        /* Q causal query rows per sequence (1 = decode)        */
    int32_t index_heads;    /* H_I indexer heads                                    */
    int32_t index_dim;      /* D_I indexer head dimension                           */
    int32_t q_heads;        /* H_q attention query heads                            */
    int32_t kv_heads;       /* H_kv attention KV heads (GQA: head hq reads KV head  */
                            /* hq / (H_q/H_kv))                                     */
    int32_t head_dim;       /* D attention head dimension                           */
    int32_t budget_groups;  /* k, groups kept per row ([SET] §Decision: 512)        */
    int64_t max_groups;     /* G_max >= G of every row, a multiple of 64: the      */
                            /* stride of score rows                                 */
    int64_t kv_slots;       /* S >= 1, physical slots of the K/V cache              */
    int32_t rows_in_flight; /* qsa_decode only: rows per pass, bounding the         */
                            /* workspace; 0 = all rows in one pass                  */
    int32_t reserved;       /* must be 0                                            */
} qsa_shape;

/* Byte ownership ledger ([MASK] §What the checkpoint measures). */
typedef struct qsa_bytes {
    int64_t raw_key;     /* raw index-key cache, total_tokens x D_I x 4          */
    int64_t pooled_key;  /* pooled-key tiles for batch sequences of max_groups   */
    int64_t kv;          /* K and V caches, 2 x S x H_kv x D x 4                 */
    int64_t workspace;   /* qsa_workspace_bytes(shape)                           */
    int64_t total;       /* sum of the above                                     */
    int64_t dense_mask;  /* always 0: no rows x tokens buffer exists             */
} qsa_bytes;

/* Layouts
 * -------
 * index_q     [rows][H_I][D_I] f32.
 * raw_keys    [tokens][D_I] f32, logical order; sequence b starts at token
 *             raw_off[b].
 * pooled      per sequence, ceil(G_b/64) tiles of 64 groups starting at
 *             element pooled_off[b] (a multiple of 4).  Within a tile, the
 *             pooled key of group g = 64t + i, dimension d, is element
 *             t*64*D_I + (d/4)*256 + i*4 + (d%4): four dimensions of 64
 *             consecutive groups are 1 KiB contiguous, so one wavefront load
 *             of a tile is fully coalesced.  Unused slots of the last tile
 *             are read but never used.
 * scores      [rows][max_groups] f32; entries at or past G are untouched.
 * sel_bitmap  [rows][ceil(max_groups/32)] u32; bit g%32 of word g/32 set iff
 *             group g is chosen.
 * token_ids   [rows][4k+4] int32: the width chronological logical IDs, then
 *             -1 padding.  width [rows] int32.
 * slot_map    int32 per logical token; sequence b's entry for token t is
 *             slot_map[slot_off[b] + t].
 * k_cache,    [S][H_kv][D] f32.
 * v_cache
 * k_compact,  [rows][H_kv][4k+4][D] f32: each KV head's selected rows of a
 * v_compact   query row are contiguous; positions at or past width untouched.
 * q           [rows][H_q][D] f32.  out [rows][H_q][D] f32; lse [rows][H_q].
 *
 * Buffers moved with 16-byte vector accesses must be 16-byte aligned:
 * raw_keys, pooled, scores, token_ids, k_cache, v_cache, k_compact,
 * v_compact, q, out, the workspace, and index_q wherever chunk scoring may
 * run (qsa_score_groups_chunk and the qsa_decode entry points).  A
 * misaligned pointer returns QSA_ERR_SHAPE before anything is enqueued.
 */

/* Workspace bytes qsa_decode needs for this shape (also enough for
 * qsa_select_topk and qsa_online_attend).  Grows with rows_in_flight x
 * (max_groups + 4k+4): per row in flight, one score per candidate group and
 * the selected width's K/V rows, and no buffer spanning rows x tokens
 * ([MASK] §What the checkpoint measures).  0 on an invalid shape. */
QSA_API size_t qsa_workspace_bytes(const qsa_shape *shape);

/* Pool complete groups into the tiled pooled-key buffer: for every
 * sequence b and group g in [first_group[b], floor(seq_len[b]/4)), pooled
 * key = (((r0 + r1) + r2) + r3) * 0.25 of the group's four raw index keys
 * ([MASK] §Why a sparse mask can still be dense: complete groups are
 * pooled and the raw index-key cache is kept).  first_group may be NULL
 * (all groups); passing the previous group count pools only the groups
 * completed since, which is the incremental append.  Uses shape->batch,
 * index_dim and max_groups only (G <= max_groups is required per
 * sequence; larger sequences are clamped). */
QSA_API int qsa_pool_groups(const qsa_shape *shape, const float *raw_keys, const int64_t *raw_off,
                    const int32_t *seq_len, const int32_t *first_group, float *pooled,
                    const int64_t *pooled_off, qsa_stream stream);

/* Step 1: score every complete group of every row ([MASK] §Decision:
 * complete groups are scored in bounded tiles; §Why a sparse mask can still
 * be dense: score = sum over index heads h of ReLU(q_h . pooled_k)).  The
 * order is fixed: each head's dot product is a chain of fused multiply-adds
 * over d ascending starting from +0, and the head terms are added in
 * ascending h starting from +0, so scores are bit-reproducible. */
QSA_API int qsa_score_groups(const qsa_shape *shape, const float *index_q, const float *pooled,
                     const int64_t *pooled_off, const int32_t *seq_len, float *scores,
                     qsa_stream stream);

/* Step 1 for causal chunks (queries > 1), on MFMA: approx[r][g] is an
 * approximation of the step-1 score of row r, group g, and bound[r][g] a
 * certified bound on its distance to the exact (chained) score, derived from
 * the standard floating-point summation error bounds and Cauchy-Schwarz.
 * qsa_decode uses the same kernel for chunk rows and then rescores the
 * groups the bounds cannot rule out with the exact chain, so its selection
 * is identical to one decode per row (AFN-017 capsule evidence: chunk/decode
 * equality).  Supported when index_heads is 4, 8 or 16 and queries is a
 * multiple of 64/index_heads; QSA_ERR_UNSUPPORTED otherwise. */
QSA_API int qsa_score_groups_chunk(const qsa_shape *shape, const float *index_q,
                                   const float *pooled, const int64_t *pooled_off,
                                   const int32_t *seq_len, float *approx, float *bound,
                                   qsa_stream stream);

/* Step 2: top-k membership per row by (score descending, group position
 * ascending); ties are resolved while choosing the set ([SET] §Decision and
 * §Tie handling belongs to membership).  Rows with G <= k keep every group.
 * -0 and +0 are equal scores; NaN scores are outside the contract.  Needs a
 * workspace of qsa_workspace_bytes(shape). */
QSA_API int qsa_select_topk(const qsa_shape *shape, const float *scores, const int32_t *seq_len,
                    uint32_t *sel_bitmap, void *workspace, size_t workspace_bytes,
                    qsa_stream stream);

/* Steps 3-5: emit the chosen groups in ascending logical position, four
 * consecutive token IDs each, then the raw tail; width = 4m + (N mod 4)
 * ([SET] §Decision; §The dense-parity property: at or below budget the row
 * is exactly 0..N-1). */
QSA_API int qsa_emit_chronological(const qsa_shape *shape, const uint32_t *sel_bitmap,
                           const int32_t *seq_len, int32_t *token_ids, int32_t *width,
                           qsa_stream stream);

/* Steps 6-7: resolve each logical ID once through the slot map and copy
 * only those K and V rows into compact scratch, in row order ([MASK]
 * §Decision: only the gather crosses into physical layout; §Why compact
 * gather comes before fusion).  phys_slots ([rows][4k+4], may be NULL)
 * receives the resolved slots. */
QSA_API int qsa_resolve_gather(const qsa_shape *shape, const int32_t *token_ids, const int32_t *width,
                       const int32_t *seq_len, const int32_t *slot_map, const int64_t *slot_off,
                       const float *k_cache, const float *v_cache, float *k_compact,
                       float *v_compact, int32_t *phys_slots, qsa_stream stream);

/* Step 8: F32 online softmax attention over the width compact rows of each
 * row, out = softmax(scale * q . k) . v per query head ([SET] §Floating
 * point makes order observable; [MASK] §Decision).  Rows are visited in
 * chronological order in fixed slices of consecutive rows whose online
 * softmax states (max, denominator, accumulator) are folded in ascending
 * order, one state per range of consecutive rows, the range states then
 * merged in ascending order, so results depend on the width alone and are
 * run-to-run bit-identical.  width 0 gives out = +0
 * and lse = -inf.  lse may be NULL. */
QSA_API int qsa_online_attend(const qsa_shape *shape, const float *q, const float *k_compact,
                      const float *v_compact, const int32_t *width, float softmax_scale,
                      float *out, float *lse, void *workspace, size_t workspace_bytes,
                      qsa_stream stream);

/* Stage timer for qsa_decode and its variants: HIP events recorded on the
 * call's stream around the stages in stage_mask (bit s = stage s, nonzero,
 * below 1 << QSA_DECODE_STAGES) of up to max_calls calls; with several
 * passes of rows_in_flight rows, around the first pass.  Each recorded event
 * costs the stream a few microseconds, so time only the stages needed. */
#define QSA_TIMER_ALL ((1u << QSA_DECODE_STAGES) - 1u)
typedef struct qsa_timer qsa_timer;
QSA_API int qsa_timer_create(int32_t max_calls, uint32_t stage_mask, qsa_timer **timer);
/* Waits for the recorded calls and writes ms[call][stage] for the n calls
 * made since creation or the last reset (n returned in *calls); stages not
 * in the mask read -1. */
QSA_API int qsa_timer_read(qsa_timer *timer, float *ms_host, int32_t *calls_host);
QSA_API void qsa_timer_reset(qsa_timer *timer);
QSA_API void qsa_timer_destroy(qsa_timer *timer);

/* Steps 1-8 in one call: scores and per-16-group maxima, selection and
 * chronological emission (token_ids, width), resolve and compact gather,
 * online attention (out, lse).  With queries > 1 and a shape that
 * qsa_score_groups_chunk supports, step 1 runs on MFMA with certified bounds
 * and the candidates are rescored exactly, so every row's result equals a
 * decode of that row alone.  Workspace >= qsa_workspace_bytes(shape)
 * holds scores, maxima, tile error widths (causal chunks), compact K/V
 * and attention partials.  timer may be
 * NULL.  Intermediate scratch contents are undefined after the call. */
QSA_API int qsa_decode(const qsa_shape *shape, const float *index_q, const float *pooled,
               const int64_t *pooled_off, const int32_t *seq_len, const int32_t *slot_map,
               const int64_t *slot_off, const float *k_cache, const float *v_cache,
               const float *q, float softmax_scale, int32_t *token_ids, int32_t *width,
               float *out, float *lse, void *workspace, size_t workspace_bytes,
               qsa_timer *timer, qsa_stream stream);

/* Steps 1-8 with steps 6-8 fused: the attention kernel resolves each
 * selected logical ID once through the slot map and reads the K/V rows
 * straight from the cache, so no compact scratch is written or read.  The
 * note names this as the step after the compact gather, once measured, with
 * the logical-ID interface and the absence of any dense mask unchanged
 * ([MASK] §Why compact gather comes before fusion).  Same arguments,
 * workspace and results as qsa_decode, bit for bit; the timer's gather stage
 * is empty. */
QSA_API int qsa_decode_fused(const qsa_shape *shape, const float *index_q, const float *pooled,
                             const int64_t *pooled_off, const int32_t *seq_len,
                             const int32_t *slot_map, const int64_t *slot_off,
                             const float *k_cache, const float *v_cache, const float *q,
                             float softmax_scale, int32_t *token_ids, int32_t *width, float *out,
                             float *lse, void *workspace, size_t workspace_bytes,
                             qsa_timer *timer, qsa_stream stream);

/* The bounded dense causal row on the GPU: every visible token 0..N-1, in
 * order, resolved through the slot map and attended with exactly the
 * reduction order of step 8, for rows with N <= 4k+3 ([SET] §The
 * dense-parity property: at or below the budget the sparse row is this row,
 * so qsa_decode and this call return the same bits there; [MASK] §Failure
 * boundary: the dense oracle is bounded at 2,051 keys for k = 512).  Rows
 * with more visible tokens get width -1 and NaN outputs.  Writes token_ids
 * ([rows][4k+4], the dense row) and width; needs qsa_workspace_bytes. */
QSA_API int qsa_dense_attend(const qsa_shape *shape, const int32_t *seq_len,
                             const int32_t *slot_map, const int64_t *slot_off,
                             const float *k_cache, const float *v_cache, const float *q,
                             float softmax_scale, int32_t *token_ids, int32_t *width, float *out,
                             float *lse, void *workspace, size_t workspace_bytes,
                             qsa_stream stream);

/* Steps 6-7 once per chunk instead of once per row.  The queries of a
 * causal chunk choose nearly the same groups, so the union of the groups
 * their IDs touch (selected groups and each row's raw-tail group) is
 * resolved through the slot map and copied once, into a union scratch
 * ([MASK] §Decision: only the gather crosses into physical layout; §Why
 * compact gather comes before fusion: one explicit copy into bounded
 * scratch; [SET] capsule evidence: chunk/decode equality).  All rows form one
 * union, so rows_in_flight must be 0 or at least batch x queries
 * (QSA_ERR_UNSUPPORTED otherwise).
 *   k_union, v_union  [rows x (4k+4)][H_kv][D] f32 (the compact capacity; a
 *                     union never needs more).  Union group u (groups
 *                     ordered by sequence, then position) occupies rows
 *                     4u..4u+3, token 4g+e at row 4u+e.  Tokens that no row
 *                     of the sequence can see are left unwritten; an
 *                     out-of-range slot gives a NaN row.
 *   union_pos         [rows][4k+4] int32: row i of a query row is scratch row
 *                     union_pos[row][i]; -1 past the width and for IDs the
 *                     row cannot see.
 *   union_groups      device int32, receives the union's group count; may be
 *                     NULL.
 * Needs qsa_workspace_bytes(shape). */
QSA_API int qsa_union_gather(const qsa_shape *shape, const int32_t *token_ids,
                             const int32_t *width, const int32_t *seq_len,
                             const int32_t *slot_map, const int64_t *slot_off,
                             const float *k_cache, const float *v_cache, float *k_union,
                             float *v_union, int32_t *union_pos, int32_t *union_groups,
                             void *workspace, size_t workspace_bytes, qsa_stream stream);

/* Step 8 over rows read through a position list: row i of query row r is
 * k_rows/v_rows row row_pos[r][i] ([rows][4k+4] int32; rows [n_rows][H_kv][D]
 * f32).  A position outside [0, n_rows) makes that row NaN.  Same chunked
 * chronological order and bits as qsa_online_attend over the equivalent
 * compact rows.  Needs qsa_workspace_bytes(shape). */
QSA_API int qsa_online_attend_indexed(const qsa_shape *shape, const float *q,
                                      const float *k_rows, const float *v_rows, int64_t n_rows,
                                      const int32_t *row_pos, const int32_t *width,
                                      float softmax_scale, float *out, float *lse,
                                      void *workspace, size_t workspace_bytes,
                                      qsa_stream stream);

/* Steps 1-8 with the union gather: per pass of rows_in_flight rows, one
 * union of the rows' K/V (as qsa_union_gather, per pass) replaces the
 * per-row compact copies, and the attention reads each row through its
 * position list.  Same arguments, workspace and results as qsa_decode, bit
 * for bit; for decode rows (queries = 1) the union is each row's own rows. */
QSA_API int qsa_decode_dedup(const qsa_shape *shape, const float *index_q, const float *pooled,
                             const int64_t *pooled_off, const int32_t *seq_len,
                             const int32_t *slot_map, const int64_t *slot_off,
                             const float *k_cache, const float *v_cache, const float *q,
                             float softmax_scale, int32_t *token_ids, int32_t *width, float *out,
                             float *lse, void *workspace, size_t workspace_bytes,
                             qsa_timer *timer, qsa_stream stream);

/* qsa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * workspace is the library's own static device buffer of
 * QSA_NOALLOC_WORKSPACE_BYTES (64 MiB), which each device the library runs on
 * holds until the process ends; the call allocates nothing.  Same arguments
 * as qsa_decode minus the workspace, same results bit for bit.  A shape
 * whose qsa_workspace_bytes exceeds the buffer returns
 * QSA_ERR_STATIC_WORKSPACE before anything is enqueued: lower rows_in_flight
 * (at 262,144 visible tokens, indexer 16 x 128 and attention 32 / 4 x 128,
 * budget 512, up to 7 rows fit).  Nothing in the buffer has to start at zero
 * (every call writes what it reads); calls that overlap on one device share
 * the buffer and race, so calls on one device must be ordered (one stream, or
 * streams joined by events). */
#define QSA_NOALLOC_WORKSPACE_BYTES (64ull << 20)
QSA_API int qsa_decode_noalloc(const qsa_shape *shape, const float *index_q, const float *pooled,
                               const int64_t *pooled_off, const int32_t *seq_len,
                               const int32_t *slot_map, const int64_t *slot_off,
                               const float *k_cache, const float *v_cache, const float *q,
                               float softmax_scale, int32_t *token_ids, int32_t *width,
                               float *out, float *lse, qsa_timer *timer, qsa_stream stream);

/* Host-only byte ledger for a cache of total_tokens tokens ([MASK] §What
 * the checkpoint measures; the dense-mask count is always 0). */
QSA_API int qsa_accounting(const qsa_shape *shape, int64_t total_tokens, qsa_bytes *out_host);

/* Static description of a status code. */
QSA_API const char *qsa_status_string(int status);

/* Library version, e.g. "qsa 0.1.0 gfx950". */
QSA_API const char *qsa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QSA_H */
