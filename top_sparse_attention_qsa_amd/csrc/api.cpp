// api.cpp -- host side of libqsa.so: validation, workspace layout, launch
// chains, stage timer and byte accounting.  Every entry point validates its
// arguments on the host and returns a qsa_status before enqueueing anything.
// No C++ exception crosses the ABI; no device memory is allocated.
//
// Plain C++: the kernels are reached only through the launchers of
// qsa_launch.h, so this file builds with a host compiler alone (and, for the
// sanitizer tests, against a stub that records the launches).
#include <stdint.h>
#include <string.h>

#include <new>

#include "qsa.h"
#include "qsa_launch.h"

using namespace qsa;

namespace {

inline bool is_pow2_in(int32_t v, int32_t lo, int32_t hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t row_count(const qsa_shape* s) { return (int64_t)s->batch * s->queries; }

int64_t rows_per_pass(const qsa_shape* s) {
  const int64_t rows = row_count(s);
  return (s->rows_in_flight > 0 && s->rows_in_flight < rows) ? s->rows_in_flight : rows;
}

int32_t token_stride(const qsa_shape* s) { return 4 * s->budget_groups + 4; }

int32_t attn_chunks(const qsa_shape* s) {
  return (4 * s->budget_groups + 3 + kAttnChunk - 1) / kAttnChunk;
}

// What each entry point needs from the shape.
enum Need { kNeedIndex = 1, kNeedAttn = 2, kNeedBudget = 4 };

int validate(const qsa_shape* s, int need) {
  if (!s) return QSA_ERR_NULL;
  if (s->reserved != 0) return QSA_ERR_SHAPE;
  if (s->batch < 1 || s->queries < 1) return QSA_ERR_SHAPE;
  if (row_count(s) > 65535) return QSA_ERR_UNSUPPORTED;  // rows ride a grid dimension
  if (s->max_groups < 0 || (s->max_groups % 64) != 0) return QSA_ERR_SHAPE;
  if (s->max_groups > ((int64_t)1 << 28)) return QSA_ERR_UNSUPPORTED;
  if (s->rows_in_flight < 0) return QSA_ERR_SHAPE;
  if (need & kNeedBudget) {
    if (s->budget_groups < 1 || s->budget_groups > QSA_MAX_BUDGET) return QSA_ERR_BUDGET;
  }
  if (need & kNeedIndex) {
    if (s->index_heads < 1 || s->index_dim < 1) return QSA_ERR_SHAPE;
    if (!is_pow2_in(s->index_heads, 1, 16)) return QSA_ERR_UNSUPPORTED;
    if (!is_pow2_in(s->index_dim, 32, 128)) return QSA_ERR_UNSUPPORTED;
  }
  if (need & kNeedAttn) {
    if (s->q_heads < 1 || s->kv_heads < 1 || s->head_dim < 1) return QSA_ERR_SHAPE;
    if (s->q_heads % s->kv_heads != 0) return QSA_ERR_SHAPE;
    if (!is_pow2_in(s->q_heads / s->kv_heads, 1, 16)) return QSA_ERR_UNSUPPORTED;
    if (s->head_dim != 64 && s->head_dim != 128) return QSA_ERR_UNSUPPORTED;
    if (s->kv_heads > 65535) return QSA_ERR_UNSUPPORTED;
    if (s->kv_slots < 1 || s->kv_slots > INT32_MAX) return QSA_ERR_SHAPE;
  }
  return QSA_OK;
}

struct Layout {
  size_t scores, maxima, widths, kc, vc, pacc, pml;
  size_t rbm, ubm, upre, ublk, ulist, upos;  // union gather (chunk dedup)
  size_t total;
};

Layout layout(const qsa_shape* s) {
  Layout L{};
  const int64_t R = rows_per_pass(s);
  const int64_t g = s->max_groups;
  size_t off = 0;
  L.scores = off;
  off = align256(off + (size_t)R * g * sizeof(float));
  L.maxima = off;
  off = align256(off + (size_t)R * (g / kSegment) * sizeof(uint32_t));
  L.widths = off;  // certified (causal chunk) rows only: one per 64-group tile
  off = align256(off + (size_t)R * (g / 64) * sizeof(float));
  const size_t compact = (size_t)R * token_stride(s) * s->kv_heads * s->head_dim * sizeof(float);
  L.kc = off;
  off = align256(off + compact);
  L.vc = off;
  off = align256(off + compact);
  const size_t slots = (size_t)R * s->q_heads * attn_parts(attn_chunks(s));
  L.pacc = off;
  off = align256(off + slots * s->head_dim * sizeof(float));
  L.pml = off;
  off = align256(off + slots * 2 * sizeof(float));
  const int64_t wps = union_words_per_seq(g);
  const int64_t useq = union_seqs_per_pass(R, s->queries, s->batch);
  L.rbm = off;
  off = align256(off + (size_t)R * wps * sizeof(uint32_t));
  L.ubm = off;
  off = align256(off + (size_t)useq * wps * sizeof(uint32_t));
  L.upre = off;
  off = align256(off + (size_t)useq * wps * sizeof(uint32_t));
  L.ublk = off;
  off = align256(off + (size_t)(union_scan_blocks(useq * wps) + 1) * sizeof(uint32_t));
  L.ulist = off;
  off = align256(off + (size_t)R * (s->budget_groups + 1) * 2 * sizeof(int32_t));
  L.upos = off;
  off = align256(off + (size_t)R * token_stride(s) * sizeof(int32_t));
  L.total = off;
  return L;
}

inline int hip_status(int e) { return e == 0 ? QSA_OK : QSA_ERR_HIP; }

}  // namespace

struct qsa_timer {
  int32_t max_calls;
  int32_t calls;
  uint32_t mask;   // stages timed (bit s: stage s)
  void** ev;       // hipEvent_t [max_calls][QSA_DECODE_STAGES + 1]
};

extern "C" {

const char* qsa_version(void) { return "qsa 0.2.0 gfx950"; }

const char* qsa_status_string(int status) {
  switch (status) {
    case QSA_OK: return "ok";
    case QSA_ERR_NULL: return "a required pointer is NULL";
    case QSA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case QSA_ERR_BUDGET: return "budget_groups outside [1, QSA_MAX_BUDGET]";
    case QSA_ERR_WORKSPACE: return "workspace smaller than qsa_workspace_bytes()";
    case QSA_ERR_HIP: return "a HIP call or kernel launch failed";
    case QSA_ERR_UNSUPPORTED: return "shape not supported by this build";
    case QSA_ERR_STATIC_WORKSPACE:
      return "the shape needs more workspace than the library's static buffer "
             "(QSA_NOALLOC_WORKSPACE_BYTES); lower rows_in_flight";
    default: return "unknown status";
  }
}

size_t qsa_workspace_bytes(const qsa_shape* s) {
  if (validate(s, kNeedBudget | kNeedAttn) != QSA_OK) return 0;
  return layout(s).total;
}

int qsa_accounting(const qsa_shape* s, int64_t total_tokens, qsa_bytes* out) {
  if (!out) return QSA_ERR_NULL;
  const int rc = validate(s, kNeedIndex | kNeedAttn | kNeedBudget);
  if (rc != QSA_OK) return rc;
  if (total_tokens < 0) return QSA_ERR_SHAPE;
  qsa_bytes b{};
  b.raw_key = total_tokens * s->index_dim * (int64_t)sizeof(float);
  b.pooled_key = (int64_t)s->batch * ((s->max_groups + 63) / 64) * 64 * s->index_dim *
                 (int64_t)sizeof(float);
  b.kv = 2 * s->kv_slots * s->kv_heads * (int64_t)s->head_dim * (int64_t)sizeof(float);
  b.workspace = (int64_t)layout(s).total;
  b.dense_mask = 0;
  b.total = b.raw_key + b.pooled_key + b.kv + b.workspace + b.dense_mask;
  *out = b;
  return QSA_OK;
}

int qsa_pool_groups(const qsa_shape* s, const float* raw_keys, const int64_t* raw_off,
                    const int32_t* seq_len, const int32_t* first_group, float* pooled,
                    const int64_t* pooled_off, qsa_stream stream) {
  int rc = validate(s, kNeedIndex);
  if (rc != QSA_OK) return rc;
  if (!raw_keys || !raw_off || !seq_len || !pooled || !pooled_off) return QSA_ERR_NULL;
  if (!aligned16(raw_keys) || !aligned16(pooled)) return QSA_ERR_SHAPE;
  PoolArgs a{raw_keys, raw_off, seq_len, first_group, pooled, pooled_off, s->batch,
             s->index_dim, s->max_groups};
  return hip_status(launch_pool(a, stream));
}

int qsa_score_groups(const qsa_shape* s, const float* index_q, const float* pooled,
                     const int64_t* pooled_off, const int32_t* seq_len, float* scores,
                     qsa_stream stream) {
  int rc = validate(s, kNeedIndex);
  if (rc != QSA_OK) return rc;
  if (!index_q || !pooled || !pooled_off || !seq_len || !scores) return QSA_ERR_NULL;
  if (!aligned16(pooled) || !aligned16(scores)) return QSA_ERR_SHAPE;
  ScoreArgs a{index_q, pooled, pooled_off, seq_len, s->queries, s->max_groups,
              0, row_count(s), scores, nullptr};
  return hip_status(launch_score(a, s->index_heads, s->index_dim, stream));
}

int qsa_score_groups_chunk(const qsa_shape* s, const float* index_q, const float* pooled,
                           const int64_t* pooled_off, const int32_t* seq_len, float* approx,
                           float* bound, qsa_stream stream) {
  int rc = validate(s, kNeedIndex);
  if (rc != QSA_OK) return rc;
  if (!index_q || !pooled || !pooled_off || !seq_len || !approx || !bound) return QSA_ERR_NULL;
  if (!aligned16(index_q) || !aligned16(pooled)) return QSA_ERR_SHAPE;
  if (!chunk_supported(s->index_heads, s->queries, row_count(s))) return QSA_ERR_UNSUPPORTED;
  ChunkArgs a{index_q, pooled, pooled_off, seq_len, s->queries, s->max_groups, 0, row_count(s),
              approx, bound, nullptr, nullptr};
  return hip_status(launch_chunk(a, s->index_heads, s->index_dim, stream));
}

int qsa_select_topk(const qsa_shape* s, const float* scores, const int32_t* seq_len,
                    uint32_t* sel_bitmap, void* ws, size_t ws_bytes, qsa_stream stream) {
  int rc = validate(s, kNeedBudget | kNeedAttn);
  if (rc != QSA_OK) return rc;
  if (!scores || !seq_len || !sel_bitmap || !ws) return QSA_ERR_NULL;
  if (!aligned16(scores)) return QSA_ERR_SHAPE;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return QSA_ERR_WORKSPACE;
  uint32_t* maxima = reinterpret_cast<uint32_t*>((char*)ws + L.maxima);
  const int64_t rows = row_count(s), R = rows_per_pass(s);
  void* st = stream;
  for (int64_t r0 = 0; r0 < rows; r0 += R) {
    const int64_t n = (rows - r0) < R ? (rows - r0) : R;
    const float* sc = scores + r0 * s->max_groups;
    int e = launch_segment_maxima(sc, seq_len, s->queries, s->max_groups, r0, n, maxima, st);
    if (e != 0) return QSA_ERR_HIP;
    SelectArgs a{sc, maxima, seq_len, s->queries, s->max_groups, s->budget_groups,
                 r0, n, sel_bitmap, nullptr, nullptr};
    e = launch_select(a, st);
    if (e != 0) return QSA_ERR_HIP;
  }
  return QSA_OK;
}

int qsa_emit_chronological(const qsa_shape* s, const uint32_t* sel_bitmap, const int32_t* seq_len,
                           int32_t* token_ids, int32_t* width, qsa_stream stream) {
  int rc = validate(s, kNeedBudget);
  if (rc != QSA_OK) return rc;
  if (!sel_bitmap || !seq_len || !token_ids || !width) return QSA_ERR_NULL;
  if (!aligned16(token_ids)) return QSA_ERR_SHAPE;
  return hip_status(launch_emit(sel_bitmap, seq_len, s->queries, s->max_groups,
                                s->budget_groups, row_count(s), token_ids, width,
                                stream));
}

int qsa_resolve_gather(const qsa_shape* s, const int32_t* token_ids, const int32_t* width,
                       const int32_t* seq_len, const int32_t* slot_map, const int64_t* slot_off,
                       const float* k_cache, const float* v_cache, float* k_compact,
                       float* v_compact, int32_t* phys_slots, qsa_stream stream) {
  int rc = validate(s, kNeedBudget | kNeedAttn);
  if (rc != QSA_OK) return rc;
  if (!token_ids || !width || !seq_len || !slot_map || !slot_off || !k_cache || !v_cache ||
      !k_compact || !v_compact)
    return QSA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_compact) ||
      !aligned16(v_compact))
    return QSA_ERR_SHAPE;
  GatherArgs a{token_ids, width, seq_len, slot_map, slot_off, k_cache, v_cache, s->queries,
               s->kv_heads, s->head_dim, token_stride(s), s->kv_slots, 0, row_count(s),
               k_compact, v_compact, phys_slots};
  return hip_status(launch_gather(a, stream));
}

int qsa_online_attend(const qsa_shape* s, const float* q, const float* k_compact,
                      const float* v_compact, const int32_t* width, float softmax_scale,
                      float* out, float* lse, void* ws, size_t ws_bytes, qsa_stream stream) {
  int rc = validate(s, kNeedBudget | kNeedAttn);
  if (rc != QSA_OK) return rc;
  if (!q || !k_compact || !v_compact || !width || !out || !ws) return QSA_ERR_NULL;
  if (!aligned16(k_compact) || !aligned16(v_compact) || !aligned16(q) || !aligned16(out))
    return QSA_ERR_SHAPE;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return QSA_ERR_WORKSPACE;
  const int64_t rows = row_count(s), R = rows_per_pass(s);
  const int64_t compact_row = (int64_t)token_stride(s) * s->kv_heads * s->head_dim;
  void* st = stream;
  for (int64_t r0 = 0; r0 < rows; r0 += R) {
    const int64_t n = (rows - r0) < R ? (rows - r0) : R;
    AttendArgs a{q, k_compact + r0 * compact_row, v_compact + r0 * compact_row, width,
                 s->q_heads, s->kv_heads, s->head_dim, token_stride(s), attn_chunks(s),
                 softmax_scale, r0, n,
                 reinterpret_cast<float*>((char*)ws + L.pacc),
                 reinterpret_cast<float*>((char*)ws + L.pml), out, lse};
    if (launch_attend(a, st) != 0) return QSA_ERR_HIP;
    if (launch_merge(a, st) != 0) return QSA_ERR_HIP;
  }
  return QSA_OK;
}

int qsa_timer_create(int32_t max_calls, uint32_t stage_mask, qsa_timer** timer) {
  if (!timer) return QSA_ERR_NULL;
  if (max_calls < 1 || max_calls > (1 << 20)) return QSA_ERR_SHAPE;
  if (stage_mask == 0 || (stage_mask >> QSA_DECODE_STAGES) != 0) return QSA_ERR_SHAPE;
  qsa_timer* t = new (std::nothrow) qsa_timer;
  if (!t) return QSA_ERR_HIP;
  const int32_t n = max_calls * (QSA_DECODE_STAGES + 1);
  t->ev = new (std::nothrow) void*[n];
  t->max_calls = max_calls;
  t->calls = 0;
  t->mask = stage_mask;
  if (!t->ev) {
    delete t;
    return QSA_ERR_HIP;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (event_create(&t->ev[i]) != 0) {
      for (int32_t j = 0; j < i; ++j) (void)event_destroy(t->ev[j]);
      delete[] t->ev;
      delete t;
      return QSA_ERR_HIP;
    }
  }
  *timer = t;
  return QSA_OK;
}

int qsa_timer_read(qsa_timer* t, float* ms, int32_t* calls) {
  if (!t || !ms || !calls) return QSA_ERR_NULL;
  for (int32_t c = 0; c < t->calls; ++c) {
    void** e = t->ev + (size_t)c * (QSA_DECODE_STAGES + 1);
    int last = QSA_DECODE_STAGES;  // the last event recorded for this call
    while (last > 0 && !((t->mask >> (last - 1)) & 1u)) --last;
    if (event_synchronize(e[last]) != 0) return QSA_ERR_HIP;
    for (int st = 0; st < QSA_DECODE_STAGES; ++st) {
      float v = -1.0f;  // stage not timed
      if ((t->mask >> st) & 1u) {
        if (event_elapsed_ms(&v, e[st], e[st + 1]) != 0) return QSA_ERR_HIP;
      }
      ms[(size_t)c * QSA_DECODE_STAGES + st] = v;
    }
  }
  *calls = t->calls;
  return QSA_OK;
}

void qsa_timer_reset(qsa_timer* t) {
  if (t) t->calls = 0;
}

void qsa_timer_destroy(qsa_timer* t) {
  if (!t) return;
  const int32_t n = t->max_calls * (QSA_DECODE_STAGES + 1);
  for (int32_t i = 0; i < n; ++i) (void)event_destroy(t->ev[i]);
  delete[] t->ev;
  delete t;
}

}  // extern "C"

// How steps 6-8 read the selected K/V rows.
enum class Rows { kCompact, kFused, kUnion };

static UnionArgs union_args(const qsa_shape* s, const Layout& L, char* w, const int32_t* token_ids,
                            const int32_t* width, const int32_t* seq_len, const int32_t* slot_map,
                            const int64_t* slot_off, const float* k_cache, const float* v_cache,
                            int64_t r0, int64_t n, float* k_union, float* v_union,
                            int32_t* union_pos, int32_t* count_out) {
  UnionArgs u{};
  u.token_ids = token_ids;
  u.width = width;
  u.seq_len = seq_len;
  u.slot_map = slot_map;
  u.slot_off = slot_off;
  u.k_cache = k_cache;
  u.v_cache = v_cache;
  u.queries = s->queries;
  u.kv_heads = s->kv_heads;
  u.head_dim = s->head_dim;
  u.stride = token_stride(s);
  u.kv_slots = s->kv_slots;
  u.max_groups = s->max_groups;
  u.row0 = r0;
  u.rows = n;
  u.cus = device_cus();
  u.row_bitmap = reinterpret_cast<uint32_t*>(w + L.rbm);
  u.union_bitmap = reinterpret_cast<uint32_t*>(w + L.ubm);
  u.word_prefix = reinterpret_cast<uint32_t*>(w + L.upre);
  u.block_prefix = reinterpret_cast<uint32_t*>(w + L.ublk);
  u.union_list = reinterpret_cast<int32_t*>(w + L.ulist);
  u.k_union = k_union;
  u.v_union = v_union;
  u.union_pos = union_pos;
  u.count_out = count_out;
  return u;
}

static int decode_impl(Rows mode, const qsa_shape* s, const float* index_q, const float* pooled,
               const int64_t* pooled_off, const int32_t* seq_len, const int32_t* slot_map,
               const int64_t* slot_off, const float* k_cache, const float* v_cache,
               const float* q, float softmax_scale, int32_t* token_ids, int32_t* width,
               float* out, float* lse, void* ws, size_t ws_bytes, qsa_timer* timer,
               qsa_stream stream) {
  int rc = validate(s, kNeedIndex | kNeedAttn | kNeedBudget);
  if (rc != QSA_OK) return rc;
  if (!index_q || !pooled || !pooled_off || !seq_len || !slot_map || !slot_off || !k_cache ||
      !v_cache || !q || !token_ids || !width || !out || !ws)
    return QSA_ERR_NULL;
  if (!aligned16(index_q) || !aligned16(pooled) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(q) || !aligned16(out) || !aligned16(token_ids) || !aligned16(ws))
    return QSA_ERR_SHAPE;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return QSA_ERR_WORKSPACE;
  if (timer && timer->calls >= timer->max_calls) return QSA_ERR_SHAPE;

  char* w = (char*)ws;
  float* scores = reinterpret_cast<float*>(w + L.scores);
  uint32_t* maxima = reinterpret_cast<uint32_t*>(w + L.maxima);
  float* widths = reinterpret_cast<float*>(w + L.widths);
  float* kc = reinterpret_cast<float*>(w + L.kc);
  float* vc = reinterpret_cast<float*>(w + L.vc);
  float* pacc = reinterpret_cast<float*>(w + L.pacc);
  float* pml = reinterpret_cast<float*>(w + L.pml);
  void* st = stream;
  void** ev = timer ? timer->ev + (size_t)timer->calls * (QSA_DECODE_STAGES + 1) : nullptr;
  const int64_t rows = row_count(s), R = rows_per_pass(s);
  // causal chunks score on MFMA with certified bounds and an exact rescoring
  // of the candidates; decode rows (or unsupported chunk shapes) use the chain
  const bool chunk = s->queries > 1 && chunk_supported(s->index_heads, s->queries, R);

  for (int64_t r0 = 0; r0 < rows; r0 += R) {
    const int64_t n = (rows - r0) < R ? (rows - r0) : R;
    const bool timed = ev && r0 == 0;  // with several passes the events bracket the first
    // event i opens stage i and closes stage i-1; only those of timed stages
    // are recorded, so an untimed stage adds nothing to the stream
    auto record = [&](int i) -> bool {
      if (!timed) return true;
      const uint32_t m = timer->mask;
      const bool need = ((m >> i) & 1u) || (i > 0 && ((m >> (i - 1)) & 1u));
      return !need || event_record(ev[i], st) == 0;
    };
    if (!record(0)) return QSA_ERR_HIP;
    if (chunk) {
      ChunkArgs ca{index_q, pooled, pooled_off, seq_len, s->queries, s->max_groups, r0, n,
                   nullptr, nullptr, scores, maxima, widths};
      if (launch_chunk(ca, s->index_heads, s->index_dim, st) != 0) return QSA_ERR_HIP;
    } else {
      ScoreArgs sa{index_q, pooled, pooled_off, seq_len, s->queries, s->max_groups, r0, n,
                   scores, maxima};
      if (launch_score(sa, s->index_heads, s->index_dim, st) != 0) return QSA_ERR_HIP;
    }
    if (!record(1)) return QSA_ERR_HIP;
    SelectArgs se{scores, maxima, seq_len, s->queries, s->max_groups, s->budget_groups,
                  r0, n, nullptr, token_ids, width};
    if (chunk) {
      se.widths = widths;
      RescoreArgs ra{index_q, pooled, pooled_off, s->index_heads, s->index_dim};
      if (launch_select_certified(se, ra, st) != 0) return QSA_ERR_HIP;
    } else if (launch_select(se, st) != 0) {
      return QSA_ERR_HIP;
    }
    if (!record(2)) return QSA_ERR_HIP;
    int32_t* upos = reinterpret_cast<int32_t*>(w + L.upos);
    if (mode == Rows::kCompact) {
      GatherArgs ga{token_ids, width, seq_len, slot_map, slot_off, k_cache, v_cache, s->queries,
                    s->kv_heads, s->head_dim, token_stride(s), s->kv_slots, r0, n, kc, vc,
                    nullptr};
      if (launch_gather(ga, st) != 0) return QSA_ERR_HIP;
    } else if (mode == Rows::kUnion) {
      const UnionArgs ua = union_args(s, L, w, token_ids, width, seq_len, slot_map, slot_off,
                                      k_cache, v_cache, r0, n, kc, vc, upos, nullptr);
      if (launch_union(ua, st) != 0) return QSA_ERR_HIP;
    }
    if (!record(3)) return QSA_ERR_HIP;
    AttendArgs aa{q, kc, vc, width, s->q_heads, s->kv_heads, s->head_dim, token_stride(s),
                  attn_chunks(s), softmax_scale, r0, n, pacc, pml, out, lse};
    if (mode == Rows::kUnion) {
      aa.union_pos = upos;
      aa.k_cache = kc;
      aa.v_cache = vc;
      aa.kv_slots = n * (int64_t)token_stride(s);
    } else if (mode == Rows::kFused) {
      aa.token_ids = token_ids;
      aa.seq_len = seq_len;
      aa.slot_map = slot_map;
      aa.slot_off = slot_off;
      aa.k_cache = k_cache;
      aa.v_cache = v_cache;
      aa.kv_slots = s->kv_slots;
      aa.queries = s->queries;
    }
    if (launch_attend(aa, st) != 0) return QSA_ERR_HIP;
    if (!record(4)) return QSA_ERR_HIP;
    if (launch_merge(aa, st) != 0) return QSA_ERR_HIP;
    if (!record(5)) return QSA_ERR_HIP;
  }
  if (timer) timer->calls += 1;
  return QSA_OK;
}


extern "C" {

int qsa_dense_attend(const qsa_shape* s, const int32_t* seq_len, const int32_t* slot_map,
                     const int64_t* slot_off, const float* k_cache, const float* v_cache,
                     const float* q, float softmax_scale, int32_t* token_ids, int32_t* width,
                     float* out, float* lse, void* ws, size_t ws_bytes, qsa_stream stream) {
  int rc = validate(s, kNeedAttn | kNeedBudget);
  if (rc != QSA_OK) return rc;
  if (!seq_len || !slot_map || !slot_off || !k_cache || !v_cache || !q || !token_ids || !width ||
      !out || !ws)
    return QSA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(out) ||
      !aligned16(token_ids) || !aligned16(ws))
    return QSA_ERR_SHAPE;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return QSA_ERR_WORKSPACE;
  void* st = stream;
  const int64_t rows = row_count(s), R = rows_per_pass(s);
  if (launch_dense_ids(seq_len, s->queries, s->budget_groups, rows, token_ids, width, st) != 0)
    return QSA_ERR_HIP;
  char* w = (char*)ws;
  for (int64_t r0 = 0; r0 < rows; r0 += R) {
    const int64_t n = (rows - r0) < R ? (rows - r0) : R;
    AttendArgs aa{q, nullptr, nullptr, width, s->q_heads, s->kv_heads, s->head_dim,
                  token_stride(s), attn_chunks(s), softmax_scale, r0, n,
                  reinterpret_cast<float*>(w + L.pacc), reinterpret_cast<float*>(w + L.pml), out,
                  lse};
    aa.token_ids = token_ids;
    aa.seq_len = seq_len;
    aa.slot_map = slot_map;
    aa.slot_off = slot_off;
    aa.k_cache = k_cache;
    aa.v_cache = v_cache;
    aa.kv_slots = s->kv_slots;
    aa.queries = s->queries;
    if (launch_attend(aa, st) != 0) return QSA_ERR_HIP;
    if (launch_merge(aa, st) != 0) return QSA_ERR_HIP;
  }
  return QSA_OK;
}

int qsa_decode(const qsa_shape* s, const float* index_q, const float* pooled,
               const int64_t* pooled_off, const int32_t* seq_len, const int32_t* slot_map,
               const int64_t* slot_off, const float* k_cache, const float* v_cache,
               const float* q, float softmax_scale, int32_t* token_ids, int32_t* width,
               float* out, float* lse, void* ws, size_t ws_bytes, qsa_timer* timer,
               qsa_stream stream) {
  return decode_impl(Rows::kCompact, s, index_q, pooled, pooled_off, seq_len, slot_map, slot_off, k_cache,
                     v_cache, q, softmax_scale, token_ids, width, out, lse, ws, ws_bytes, timer,
                     stream);
}

int qsa_decode_fused(const qsa_shape* s, const float* index_q, const float* pooled,
                     const int64_t* pooled_off, const int32_t* seq_len, const int32_t* slot_map,
                     const int64_t* slot_off, const float* k_cache, const float* v_cache,
                     const float* q, float softmax_scale, int32_t* token_ids, int32_t* width,
                     float* out, float* lse, void* ws, size_t ws_bytes, qsa_timer* timer,
                     qsa_stream stream) {
  return decode_impl(Rows::kFused, s, index_q, pooled, pooled_off, seq_len, slot_map, slot_off, k_cache,
                     v_cache, q, softmax_scale, token_ids, width, out, lse, ws, ws_bytes, timer,
                     stream);
}

int qsa_decode_dedup(const qsa_shape* s, const float* index_q, const float* pooled,
                     const int64_t* pooled_off, const int32_t* seq_len, const int32_t* slot_map,
                     const int64_t* slot_off, const float* k_cache, const float* v_cache,
                     const float* q, float softmax_scale, int32_t* token_ids, int32_t* width,
                     float* out, float* lse, void* ws, size_t ws_bytes, qsa_timer* timer,
                     qsa_stream stream) {
  return decode_impl(Rows::kUnion, s, index_q, pooled, pooled_off, seq_len, slot_map, slot_off,
                     k_cache, v_cache, q, softmax_scale, token_ids, width, out, lse, ws, ws_bytes,
                     timer, stream);
}

int qsa_union_gather(const qsa_shape* s, const int32_t* token_ids, const int32_t* width,
                     const int32_t* seq_len, const int32_t* slot_map, const int64_t* slot_off,
                     const float* k_cache, const float* v_cache, float* k_union, float* v_union,
                     int32_t* union_pos, int32_t* union_groups, void* ws, size_t ws_bytes,
                     qsa_stream stream) {
  int rc = validate(s, kNeedBudget | kNeedAttn);
  if (rc != QSA_OK) return rc;
  if (!token_ids || !width || !seq_len || !slot_map || !slot_off || !k_cache || !v_cache ||
      !k_union || !v_union || !union_pos || !ws)
    return QSA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_union) || !aligned16(v_union))
    return QSA_ERR_SHAPE;
  if (rows_per_pass(s) != row_count(s)) return QSA_ERR_UNSUPPORTED;  // one union for all rows
  const Layout L = layout(s);
  if (ws_bytes < L.total) return QSA_ERR_WORKSPACE;
  const UnionArgs ua = union_args(s, L, (char*)ws, token_ids, width, seq_len, slot_map, slot_off,
                                  k_cache, v_cache, 0, row_count(s), k_union, v_union, union_pos,
                                  union_groups);
  return hip_status(launch_union(ua, stream));
}

int qsa_online_attend_indexed(const qsa_shape* s, const float* q, const float* k_rows,
                              const float* v_rows, int64_t n_rows, const int32_t* row_pos,
                              const int32_t* width, float softmax_scale, float* out, float* lse,
                              void* ws, size_t ws_bytes, qsa_stream stream) {
  int rc = validate(s, kNeedBudget | kNeedAttn);
  if (rc != QSA_OK) return rc;
  if (!q || !k_rows || !v_rows || !row_pos || !width || !out || !ws) return QSA_ERR_NULL;
  if (!aligned16(k_rows) || !aligned16(v_rows) || !aligned16(q) || !aligned16(out))
    return QSA_ERR_SHAPE;
  if (n_rows < 1 || n_rows > INT32_MAX) return QSA_ERR_SHAPE;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return QSA_ERR_WORKSPACE;
  const int64_t rows = row_count(s), R = rows_per_pass(s);
  void* st = stream;
  for (int64_t r0 = 0; r0 < rows; r0 += R) {
    const int64_t n = (rows - r0) < R ? (rows - r0) : R;
    AttendArgs a{q, nullptr, nullptr, width, s->q_heads, s->kv_heads, s->head_dim,
                 token_stride(s), attn_chunks(s), softmax_scale, r0, n,
                 reinterpret_cast<float*>((char*)ws + L.pacc),
                 reinterpret_cast<float*>((char*)ws + L.pml), out, lse};
    a.union_pos = row_pos + r0 * token_stride(s);
    a.k_cache = k_rows;
    a.v_cache = v_rows;
    a.kv_slots = n_rows;
    if (launch_attend(a, st) != 0) return QSA_ERR_HIP;
    if (launch_merge(a, st) != 0) return QSA_ERR_HIP;
  }
  return QSA_OK;
}

}  // extern "C"
