// qsa_internal.h -- device helpers and kernel launchers shared by the HIP
// sources of libqsa.so (gfx950, wave64).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

constexpr int kWave = 64;
constexpr int kScoreWaves = 4;        // waves (one 64-group tile each) per scoring workgroup
constexpr int kSegment = 16;          // groups per maximum used to bound the threshold
constexpr int kSelectThreads = 1024;  // one selection workgroup per row
constexpr int kCandCap = 4096;        // candidates kept in LDS before the streaming path
constexpr int kGatherTokens = 8;      // compact rows per gather workgroup
constexpr int kAttnChunk = 64;        // compact rows per attention partial

// Scores are ordered through a monotone unsigned key: -0 is folded onto +0,
// then non-negative floats get their sign bit set and negative floats are
// bit-inverted, so unsigned comparison equals float comparison.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct RowView {
  int64_t n;     // visible tokens
  int64_t g;     // complete groups
  int32_t tail;  // n mod 4
  int32_t b;     // sequence
  bool valid;
};

__device__ __forceinline__ RowView row_view(const int32_t* __restrict__ seq_len, int64_t row,
                                            int32_t queries, int64_t g_max) {
  RowView v;
  v.b = (int32_t)(row / queries);
  const int32_t j = (int32_t)(row - (int64_t)v.b * queries);
  v.n = (int64_t)seq_len[v.b] - queries + 1 + j;
  v.valid = v.n >= 0;
  v.g = v.valid ? (v.n >> 2) : 0;
  v.tail = v.valid ? (int32_t)(v.n & 3) : 0;
  if (v.g > g_max) v.valid = false;
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Index of this wavefront within its workgroup, as a value the compiler knows
// to be uniform (so addresses derived from it use scalar loads).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t y = __shfl_up(v, o, kWave);
    if (lane >= o) v += y;
  }
  return v;
}

// Wavefront reductions.  Within each 16-lane DPP row, rotations by 1, 2, 4
// and 8 lanes (row_ror) leave every lane holding its row's reduction; lane 0
// of each row is then read into a scalar and the four rows are combined as
// (r0 op r1) op (r2 op r3).  The order is fixed, so a sum is the same bits on
// every run and the result is uniform across the wavefront.  DPP stays in
// the VALU: no LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

__device__ __forceinline__ float read_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kRowRor1>(v));
  v = fmaxf(v, dpp_f32<kRowRor2>(v));
  v = fmaxf(v, dpp_f32<kRowRor4>(v));
  v = fmaxf(v, dpp_f32<kRowRor8>(v));
  return fmaxf(fmaxf(read_lane(v, 0), read_lane(v, 16)), fmaxf(read_lane(v, 32), read_lane(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp_f32<kRowRor1>(v);
  v = v + dpp_f32<kRowRor2>(v);
  v = v + dpp_f32<kRowRor4>(v);
  v = v + dpp_f32<kRowRor8>(v);
  return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

// Exclusive prefix sum over a whole workgroup of NT threads (NT/64 waves);
// `wave_tot` is LDS scratch of NT/64 words.  *total receives the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t x, uint32_t* wave_tot,
                                                        uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int wave = (int)(threadIdx.x / kWave);
  const uint32_t inc = wave_inclusive_sum(x);
  if (lane_id() == kWave - 1) wave_tot[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = wave_tot[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - x;
}

// ---------------------------------------------------------------- launchers
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
  float* part_acc;           // [rows][H_q][n_chunks][D] local rows
  float* part_ml;            // [rows][H_q][n_chunks][2]
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
  int2* union_list;          // [rows * (k+1)]
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
  float* approx;             // [rows][g_max] approximate scores, may be null
  float* bound;              // [rows][g_max] certified error bounds, may be null
  float* hi;                 // [rows][g_max] approx + bound, may be null
  uint32_t* lo_maxima;       // [rows][g_max/16] order keys of approx - bound, may be null
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

hipError_t launch_score(const ScoreArgs& a, int h_i, int d_i, hipStream_t s);
hipError_t launch_segment_maxima(const float* scores, const int32_t* seq_len, int32_t queries,
                                 int64_t g_max, int64_t row0, int64_t rows, uint32_t* maxima,
                                 hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_emit(const uint32_t* bitmap, const int32_t* seq_len, int32_t queries,
                       int64_t g_max, int32_t k, int64_t rows, int32_t* token_ids,
                       int32_t* width, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);
hipError_t launch_merge(const AttendArgs& a, hipStream_t s);
hipError_t launch_pool(const PoolArgs& a, hipStream_t s);
hipError_t launch_dense_ids(const int32_t* seq_len, int32_t queries, int32_t k, int64_t rows,
                            int32_t* token_ids, int32_t* width, hipStream_t s);
bool chunk_supported(int h_i, int queries, int64_t rows_per_launch);
hipError_t launch_chunk(const ChunkArgs& a, int h_i, int d_i, hipStream_t s);
hipError_t launch_select_certified(const SelectArgs& a, const RescoreArgs& r, hipStream_t s);
int64_t union_words_per_seq(int64_t max_groups);
int64_t union_seqs_per_pass(int64_t rows_per_pass, int32_t queries, int32_t batch);
int64_t union_scan_blocks(int64_t words);
hipError_t launch_union(const UnionArgs& a, hipStream_t s);
int device_cus();

}  // namespace qsa
