// qsa_launch.h -- the interface between the host side of libqsa.so (api.cpp:
// validation, workspace layout, launch chains, stage timer, byte accounting)
// and the HIP kernels.  Plain C++ with no HIP types, so the host side builds
// with a host compiler alone, against these launchers or against a stub that
// records the calls.  Not part of the public ABI.
//
// Every launcher enqueues on `stream` (a hipStream_t) and returns 0, or the
// nonzero HIP error code of the failed launch.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace qsa {

constexpr int kSegment = 16;          // groups per maximum used to bound the threshold
constexpr int kAttnChunk = 64;        // compact rows per attention chunk
constexpr int kAttnRange = 8;         // consecutive chunks folded into one partial
constexpr int kUnionScanWords = 4096; // union bitmap words per count/list block

struct ScoreArgs {
  const float* index_q;
  const float* pooled;
  const int64_t* pooled_off;
  const int32_t* seq_len;
  int32_t queries;
  int64_t g_max;
  int64_t row0;       // first global row of this launch
  int64_t rows;       // rows in this launch
  float* scores;      // indexed by local row
  uint32_t* maxima;   // [rows][g_max/16] order keys, may be null
};

struct SelectArgs {
  const float* scores;       // local rows
  const uint32_t* maxima;    // local rows, may be null (no threshold bound)
  const int32_t* seq_len;
  int32_t queries;
  int64_t g_max;
  int32_t k;
  int64_t row0;
  int64_t rows;
  uint32_t* bitmap;          // global rows, may be null
  int32_t* token_ids;        // global rows, may be null
  int32_t* width;            // global rows, may be null
  const float* widths = nullptr;  // certified rows: ChunkArgs::widths, local rows
};

struct GatherArgs {
  const int32_t* token_ids;  // global rows
  const int32_t* width;      // global rows
  const int32_t* seq_len;
  const int32_t* slot_map;
  const int64_t* slot_off;
  const float* k_cache;
  const float* v_cache;
  int32_t queries;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t stride;            // 4k+4
  int64_t kv_slots;
  int64_t row0;
  int64_t rows;
  float* k_compact;          // local rows
  float* v_compact;
  int32_t* phys_slots;       // global rows, may be null
};

struct AttendArgs {
  const float* q;            // global rows
  const float* k_compact;    // local rows (compact path)
  const float* v_compact;
  const int32_t* width;      // global rows
  int32_t q_heads;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t stride;            // 4k+4
  int32_t n_chunks;          // ceil((4k+3)/kAttnChunk)
  float scale;
  int64_t row0;
  int64_t rows;
  float* part_acc;           // [rows][H_q][attn_parts(n_chunks)][D] local rows
  float* part_ml;            // [rows][H_q][attn_parts(n_chunks)][2]
  float* out;                // global rows
  float* lse;                // global rows, may be null
  // fused path (token_ids != null): rows are read from the cache through the
  // slot map instead of the compact scratch
  const int32_t* token_ids = nullptr;  // global rows
  const int32_t* seq_len = nullptr;
  const int32_t* slot_map = nullptr;
  const int64_t* slot_off = nullptr;
  const float* k_cache = nullptr;
  const float* v_cache = nullptr;
  int64_t kv_slots = 0;
  int32_t queries = 1;
  // union path (union_pos != null): row i of a row is k_cache/v_cache row
  // union_pos[row][i] (< kv_slots; negative: invalid), no slot map
  const int32_t* union_pos = nullptr;  // local rows
};

// One pass of the union gather (union.hip).
struct UnionArgs {
  const int32_t* token_ids;  // global rows
  const int32_t* width;      // global rows
  const int32_t* seq_len;
  const int32_t* slot_map;
  const int64_t* slot_off;
  const float* k_cache;
  const float* v_cache;
  int32_t queries;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t stride;            // 4k+4
  int64_t kv_slots;
  int64_t max_groups;
  int64_t row0;
  int64_t rows;
  int32_t cus;               // compute units (gather grid)
  uint32_t* row_bitmap;      // [rows][union_words_per_seq]
  uint32_t* union_bitmap;    // [union_seqs_per_pass][union_words_per_seq]
  uint32_t* word_prefix;     // same shape as union_bitmap
  uint32_t* block_prefix;    // [union_scan_blocks(words) + 1]
  int32_t* union_list;       // [rows * (k+1)] (sequence, group) pairs, 8-byte aligned
  float* k_union;            // [rows * (4k+4)][H_kv][D]
  float* v_union;
  int32_t* union_pos;        // [rows][4k+4] local rows
  int32_t* count_out;        // union groups, may be null
};

struct ChunkArgs {
  const float* index_q;      // global rows
  const float* pooled;
  const int64_t* pooled_off;
  const int32_t* seq_len;
  int32_t queries;
  int64_t g_max;
  int64_t row0;
  int64_t rows;              // a multiple of 4*16/H_I
  // two output sets: approx and bound, or hi, lo_maxima and widths (the
  // pointers of the other set null; any other combination is refused)
  float* approx;             // [rows][g_max] approximate scores
  float* bound;              // [rows][g_max] certified error bounds
  float* hi;                 // [rows][g_max] approx + bound
  uint32_t* lo_maxima;       // [rows][g_max/16] order keys of approx - bound
  float* widths = nullptr;   // [rows][g_max/64] per 64-group tile, an upper bound of
                             // hi - s over its groups (s: the chain score)
};

// Exact rescoring inputs for the certified selection (chunk rows).
struct RescoreArgs {
  const float* index_q;      // global rows
  const float* pooled;
  const int64_t* pooled_off;
  int32_t index_heads;
  int32_t index_dim;
};

struct PoolArgs {
  const float* raw_keys;
  const int64_t* raw_off;
  const int32_t* seq_len;
  const int32_t* first_group;
  float* pooled;
  const int64_t* pooled_off;
  int32_t batch;
  int32_t index_dim;
  int64_t g_max;
};

int launch_score(const ScoreArgs& a, int h_i, int d_i, void* stream);
int launch_segment_maxima(const float* scores, const int32_t* seq_len, int32_t queries,
                          int64_t g_max, int64_t row0, int64_t rows, uint32_t* maxima,
                          void* stream);
int launch_select(const SelectArgs& a, void* stream);
int launch_emit(const uint32_t* bitmap, const int32_t* seq_len, int32_t queries, int64_t g_max,
                int32_t k, int64_t rows, int32_t* token_ids, int32_t* width, void* stream);
int launch_gather(const GatherArgs& a, void* stream);
int launch_attend(const AttendArgs& a, void* stream);
int launch_merge(const AttendArgs& a, void* stream);
int launch_pool(const PoolArgs& a, void* stream);
int launch_dense_ids(const int32_t* seq_len, int32_t queries, int32_t k, int64_t rows,
                     int32_t* token_ids, int32_t* width, void* stream);
int launch_chunk(const ChunkArgs& a, int h_i, int d_i, void* stream);
int launch_select_certified(const SelectArgs& a, const RescoreArgs& r, void* stream);
int launch_union(const UnionArgs& a, void* stream);

// Attention partials per row and query head for n_chunks chunks: one per
// range of kAttnRange consecutive chunks.
inline constexpr int attn_parts(int n_chunks) {
  return (n_chunks + kAttnRange - 1) / kAttnRange;
}

// Compute units of the current device (256 if it cannot be queried).
int device_cus();

// Stage-timer events (hipEvent_t behind void*).  0 on success.
int event_create(void** ev);
int event_destroy(void* ev);
int event_record(void* ev, void* stream);
int event_synchronize(void* ev);
int event_elapsed_ms(float* ms, void* start, void* stop);

// chunk_score_kernel's row blocking: rows per launch must be a multiple of
// 4 * (16 / H_I).
inline bool chunk_supported(int h_i, int queries, int64_t rows_per_launch) {
  if (h_i != 4 && h_i != 8 && h_i != 16) return false;
  const int rb = 4 * (16 / h_i);
  return queries % rb == 0 && rows_per_launch % rb == 0;
}

// Union-gather scratch sizes (per pass).
inline int64_t union_words_per_seq(int64_t max_groups) { return max_groups / 32 + 1; }

inline int64_t union_seqs_per_pass(int64_t rows_per_pass, int32_t queries, int32_t batch) {
  const int64_t s = rows_per_pass / queries + 2;
  return s < batch ? s : batch;
}

inline int64_t union_scan_blocks(int64_t words) {
  return (words + kUnionScanWords - 1) / kUnionScanWords;
}

}  // namespace qsa
