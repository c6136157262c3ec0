// stub_launch.cpp -- recording implementations of every function of
// qsa_launch.h (see stub.h).
#include "stub.h"

#include "qsa_launch.h"

namespace stub {

std::vector<Call> calls;
int fail_at = -1;
int events_live = 0;

void reset() {
  calls.clear();
  fail_at = -1;
}

int count(const std::string& name) {
  int n = 0;
  for (const Call& c : calls) n += c.name == name;
  return n;
}

static int record(const char* name, int64_t row0, int64_t rows,
                  std::vector<const void*> ptrs, void* stream) {
  Call c;
  c.name = name;
  c.row0 = row0;
  c.rows = rows;
  c.ptrs = std::move(ptrs);
  c.stream = stream;
  calls.push_back(std::move(c));
  return (int)calls.size() - 1 == fail_at ? 98 : 0;  // 98: some nonzero HIP error code
}

}  // namespace stub

namespace qsa {

int launch_score(const ScoreArgs& a, int, int, void* s) {
  return stub::record("score", a.row0, a.rows,
                      {a.index_q, a.pooled, a.pooled_off, a.seq_len, a.scores, a.maxima}, s);
}
int launch_segment_maxima(const float* scores, const int32_t* seq_len, int32_t, int64_t,
                          int64_t row0, int64_t rows, uint32_t* maxima, void* s) {
  return stub::record("segment_maxima", row0, rows, {scores, seq_len, maxima}, s);
}
int launch_select(const SelectArgs& a, void* s) {
  return stub::record("select", a.row0, a.rows,
                      {a.scores, a.maxima, a.seq_len, a.bitmap, a.token_ids, a.width}, s);
}
int launch_emit(const uint32_t* bitmap, const int32_t* seq_len, int32_t, int64_t, int32_t,
                int64_t rows, int32_t* token_ids, int32_t* width, void* s) {
  return stub::record("emit", 0, rows, {bitmap, seq_len, token_ids, width}, s);
}
int launch_gather(const GatherArgs& a, void* s) {
  return stub::record("gather", a.row0, a.rows,
                      {a.token_ids, a.width, a.seq_len, a.slot_map, a.slot_off, a.k_cache,
                       a.v_cache, a.k_compact, a.v_compact, a.phys_slots},
                      s);
}
int launch_attend(const AttendArgs& a, void* s) {
  return stub::record("attend", a.row0, a.rows,
                      {a.q, a.k_compact, a.v_compact, a.width, a.part_acc, a.part_ml,
                       a.token_ids, a.k_cache, a.v_cache, a.union_pos},
                      s);
}
int launch_merge(const AttendArgs& a, void* s) {
  return stub::record("merge", a.row0, a.rows, {a.part_acc, a.part_ml, a.width, a.out, a.lse}, s);
}
int launch_pool(const PoolArgs& a, void* s) {
  return stub::record("pool", 0, a.batch, {a.raw_keys, a.raw_off, a.seq_len, a.first_group,
                                           a.pooled, a.pooled_off}, s);
}
int launch_dense_ids(const int32_t* seq_len, int32_t, int32_t, int64_t rows, int32_t* token_ids,
                     int32_t* width, void* s) {
  return stub::record("dense_ids", 0, rows, {seq_len, token_ids, width}, s);
}
int launch_chunk(const ChunkArgs& a, int, int, void* s) {
  return stub::record("chunk", a.row0, a.rows,
                      {a.index_q, a.pooled, a.approx, a.bound, a.hi, a.lo_maxima, a.widths}, s);
}
int launch_select_certified(const SelectArgs& a, const RescoreArgs& r, void* s) {
  return stub::record("select_certified", a.row0, a.rows,
                      {a.scores, a.maxima, a.token_ids, a.width, r.index_q, r.pooled, a.widths},
                      s);
}
int launch_union(const UnionArgs& a, void* s) {
  return stub::record("union", a.row0, a.rows,
                      {a.row_bitmap, a.union_bitmap, a.word_prefix, a.block_prefix, a.union_list,
                       a.k_union, a.v_union, a.union_pos},
                      s);
}

int device_cus() { return 256; }

int event_create(void** ev) {
  *ev = new int(0);
  ++stub::events_live;
  return 0;
}
int event_destroy(void* ev) {
  delete static_cast<int*>(ev);
  --stub::events_live;
  return 0;
}
int event_record(void* ev, void* s) {
  *static_cast<int*>(ev) += 1;
  stub::Call c;
  c.name = "event";
  c.ptrs = {ev};
  c.stream = s;
  stub::calls.push_back(c);
  return 0;
}
int event_synchronize(void* ev) { return *static_cast<int*>(ev) > 0 ? 0 : 97; }
int event_elapsed_ms(float* ms, void* start, void* stop) {
  if (*static_cast<int*>(start) <= 0 || *static_cast<int*>(stop) <= 0) return 97;
  *ms = 0.25f;
  return 0;
}

}  // namespace qsa
