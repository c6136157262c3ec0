// driver.cpp -- the host side of libqsa.so (api.cpp) against the recording
// stub launchers, built with the host sanitizers (AddressSanitizer and
// UndefinedBehaviorSanitizer) by tests/test_host_sanitized.py.
//
// Checks, for every entry point of include/qsa.h:
//  - shape validation (every field and limit, max_groups up to 2^28),
//  - NULL and misaligned pointers, short workspaces,
//  - that a rejected call enqueues nothing (the non-completion gate on the
//    host side: the stub records no launch),
//  - the launch chain of a valid call: stages in order, passes of
//    rows_in_flight rows covering every row once, and workspace regions that
//    lie inside the workspace without overlapping (recomputed here from the
//    layout's definition, not read from the library),
//  - HIP launch errors propagating as QSA_ERR_HIP with nothing enqueued after
//    the failing launch,
//  - the stage timer's bookkeeping and the byte ledger.
// Device pointers are fake addresses that are never dereferenced; the stub
// touches no memory.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <utility>
#include <vector>

#include "qsa.h"
#include "stub.h"

namespace {

int failures = 0;
int checks = 0;

#define CHECK(cond, ...)                                            \
  do {                                                              \
    ++checks;                                                       \
    if (!(cond)) {                                                  \
      ++failures;                                                   \
      fprintf(stderr, "FAIL %s:%d: %s -- ", __FILE__, __LINE__, #cond); \
      fprintf(stderr, __VA_ARGS__);                                 \
      fprintf(stderr, "\n");                                        \
    }                                                               \
  } while (0)

// Fake device addresses: caller buffer i lives in region i (2^36 bytes each),
// the workspace in region kWsRegion.
constexpr int kRegionShift = 36;
constexpr uintptr_t kWsRegion = 256;

template <class T = float>
T* dev(int region) {
  return reinterpret_cast<T*>((uintptr_t)region << kRegionShift);
}
void* const kWs = reinterpret_cast<void*>(kWsRegion << kRegionShift);
void* const kStream = reinterpret_cast<void*>(0x5000);

template <class T>
T* misalign(T* p) {
  return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(p) + 4);
}

qsa_shape c4_shape() {
  qsa_shape s{};
  s.batch = 32;
  s.queries = 1;
  s.index_heads = 16;
  s.index_dim = 128;
  s.q_heads = 32;
  s.kv_heads = 4;
  s.head_dim = 128;
  s.budget_groups = 512;
  s.max_groups = 65536;
  s.kv_slots = 8388608;
  s.rows_in_flight = 0;
  s.reserved = 0;
  return s;
}

// ---------------------------------------------------------------- decode family
struct DecodeCall {
  qsa_shape s = c4_shape();
  const float* index_q = dev(1);
  const float* pooled = dev(2);
  const int64_t* pooled_off = dev<int64_t>(3);
  const int32_t* seq_len = dev<int32_t>(4);
  const int32_t* slot_map = dev<int32_t>(5);
  const int64_t* slot_off = dev<int64_t>(6);
  const float* k_cache = dev(7);
  const float* v_cache = dev(8);
  const float* q = dev(9);
  float scale = 0.0883883f;
  int32_t* token_ids = dev<int32_t>(10);
  int32_t* width = dev<int32_t>(11);
  float* out = dev(12);
  float* lse = dev(13);
  void* ws = kWs;
  size_t ws_bytes = 0;  // 0: qsa_workspace_bytes(&s)
  qsa_timer* timer = nullptr;
  bool null_shape = false;
};

using DecodeFn = int (*)(const qsa_shape*, const float*, const float*, const int64_t*,
                         const int32_t*, const int32_t*, const int64_t*, const float*,
                         const float*, const float*, float, int32_t*, int32_t*, float*, float*,
                         void*, size_t, qsa_timer*, qsa_stream);

int run(DecodeFn f, const DecodeCall& c) {
  const size_t ws_bytes = c.ws_bytes ? c.ws_bytes : qsa_workspace_bytes(&c.s);
  return f(c.null_shape ? nullptr : &c.s, c.index_q, c.pooled, c.pooled_off, c.seq_len,
           c.slot_map, c.slot_off, c.k_cache, c.v_cache, c.q, c.scale, c.token_ids, c.width,
           c.out, c.lse, c.ws, ws_bytes, c.timer, kStream);
}

struct Named {
  const char* name;
  DecodeFn fn;
  const char* rows_stage;  // the launch that moves K/V rows between select and attend
};
const Named kDecoders[] = {{"qsa_decode", qsa_decode, "gather"},
                           {"qsa_decode_fused", qsa_decode_fused, nullptr},
                           {"qsa_decode_dedup", qsa_decode_dedup, "union"}};

// A rejected call: the expected status and nothing enqueued.
void expect_rejected(DecodeFn f, const DecodeCall& c, int code, const char* what) {
  stub::reset();
  const int rc = run(f, c);
  CHECK(rc == code, "%s: status %d, expected %d", what, rc, code);
  CHECK(stub::calls.empty(), "%s: %zu launches after a rejected call", what, stub::calls.size());
}

// Workspace regions of one pass, recomputed from the layout's definition:
// scores, maxima, compact K, compact V, partial accumulators, partial (m, l),
// and for causal-chunk rows the tile widths of the certified selection.
struct Region {
  const char* name;
  uintptr_t begin, bytes;
};

std::vector<Region> expected_regions(const qsa_shape& s) {
  const int64_t rows = (int64_t)s.batch * s.queries;
  const int64_t R = (s.rows_in_flight > 0 && s.rows_in_flight < rows) ? s.rows_in_flight : rows;
  const int64_t stride = 4 * (int64_t)s.budget_groups + 4;
  // attention partials: one per 8 consecutive chunks of 64 compact rows
  const int64_t chunks = ((4 * (int64_t)s.budget_groups + 3 + 63) / 64 + 7) / 8;
  std::vector<Region> r;
  r.push_back({"scores", 0, (uintptr_t)(R * s.max_groups * 4)});
  r.push_back({"maxima", 0, (uintptr_t)(R * (s.max_groups / 16) * 4)});
  r.push_back({"k_compact", 0, (uintptr_t)(R * stride * s.kv_heads * s.head_dim * 4)});
  r.push_back({"v_compact", 0, (uintptr_t)(R * stride * s.kv_heads * s.head_dim * 4)});
  r.push_back({"part_acc", 0, (uintptr_t)(R * s.q_heads * chunks * s.head_dim * 4)});
  r.push_back({"part_ml", 0, (uintptr_t)(R * s.q_heads * chunks * 2 * 4)});
  r.push_back({"widths", 0, (uintptr_t)(R * (s.max_groups / 64) * 4)});
  return r;
}

bool in_ws(const void* p) { return ((uintptr_t)p >> kRegionShift) == kWsRegion; }

// Checks the recorded launches of one valid decode call.
void check_decode_chain(const Named& d, const qsa_shape& s, bool chunk) {
  const int64_t rows = (int64_t)s.batch * s.queries;
  const int64_t R = (s.rows_in_flight > 0 && s.rows_in_flight < rows) ? s.rows_in_flight : rows;
  const size_t need = qsa_workspace_bytes(&s);
  std::vector<std::string> stages = {chunk ? "chunk" : "score",
                                     chunk ? "select_certified" : "select"};
  if (d.rows_stage) stages.push_back(d.rows_stage);
  stages.push_back("attend");
  stages.push_back("merge");
  const int64_t passes = (rows + R - 1) / R;
  CHECK((int64_t)stub::calls.size() == passes * (int64_t)stages.size(),
        "%s: %zu launches for %lld passes of %zu stages", d.name, stub::calls.size(),
        (long long)passes, stages.size());
  if ((int64_t)stub::calls.size() != passes * (int64_t)stages.size()) return;
  std::vector<Region> reg = expected_regions(s);
  // first-pass pointers of each region (scores from score/chunk, maxima from
  // score/chunk, compact K/V from gather, partials from attend)
  const stub::Call& c0 = stub::calls[0];
  // score and chunk launches both pass (..., scores or hi, maxima) as ptrs 4, 5
  reg[0].begin = (uintptr_t)c0.ptrs[4];
  reg[1].begin = (uintptr_t)c0.ptrs[5];
  const stub::Call& att = stub::calls[stages.size() - 2];
  reg[4].begin = (uintptr_t)att.ptrs[4];
  reg[5].begin = (uintptr_t)att.ptrs[5];
  Region widths = reg[6];
  reg.pop_back();
  size_t nreg = 2;
  if (d.rows_stage && std::string(d.rows_stage) == "gather") {
    reg[2].begin = (uintptr_t)stub::calls[2].ptrs[7];
    reg[3].begin = (uintptr_t)stub::calls[2].ptrs[8];
    nreg = 6;
  } else if (d.rows_stage) {  // the union scratch reuses the compact regions
    reg[2].begin = (uintptr_t)stub::calls[2].ptrs[5];
    reg[3].begin = (uintptr_t)stub::calls[2].ptrs[6];
    nreg = 6;
  } else {
    reg.erase(reg.begin() + 2, reg.begin() + 4);
    nreg = 4;
  }
  if (chunk) {  // the chunk launch passes its segment widths as ptr 6
    widths.begin = (uintptr_t)c0.ptrs[6];
    reg.insert(reg.begin() + nreg, widths);
    ++nreg;
    CHECK(stub::calls[1].ptrs[6] == c0.ptrs[6], "%s: selection reads the chunk's widths", d.name);
  }
  for (size_t i = 0; i < nreg; ++i) {
    CHECK(in_ws((void*)reg[i].begin), "%s: %s outside the workspace", d.name, reg[i].name);
    CHECK(reg[i].begin % 16 == 0, "%s: %s not 16-byte aligned", d.name, reg[i].name);
    CHECK(reg[i].begin + reg[i].bytes <= (uintptr_t)kWs + need,
          "%s: %s ends past the workspace (%zu bytes)", d.name, reg[i].name, need);
    for (size_t j = 0; j < i; ++j) {
      const bool apart = reg[i].begin + reg[i].bytes <= reg[j].begin ||
                         reg[j].begin + reg[j].bytes <= reg[i].begin;
      CHECK(apart, "%s: %s overlaps %s", d.name, reg[i].name, reg[j].name);
    }
  }
  for (int64_t p = 0; p < passes; ++p) {
    const int64_t r0 = p * R, n = std::min(R, rows - r0);
    for (size_t k = 0; k < stages.size(); ++k) {
      const stub::Call& c = stub::calls[p * stages.size() + k];
      CHECK(c.name == stages[k], "%s: pass %lld launch %zu is %s, expected %s", d.name,
            (long long)p, k, c.name.c_str(), stages[k].c_str());
      CHECK(c.row0 == r0 && c.rows == n, "%s: pass %lld %s covers rows [%lld, +%lld), not "
            "[%lld, +%lld)", d.name, (long long)p, c.name.c_str(), (long long)c.row0,
            (long long)c.rows, (long long)r0, (long long)n);
      CHECK(c.stream == kStream, "%s: launch on another stream", d.name);
      for (const void* ptr : c.ptrs)
        if (ptr && in_ws(ptr))
          CHECK((uintptr_t)ptr < (uintptr_t)kWs + need, "%s: %s gets a pointer past the "
                "workspace", d.name, c.name.c_str());
    }
  }
}

void test_decode_family() {
  for (const Named& d : kDecoders) {
    // valid call, one pass and several
    for (int32_t rif : {0, 1, 5, 31, 32, 33}) {
      DecodeCall c;
      c.s.rows_in_flight = rif;
      stub::reset();
      const int rc = run(d.fn, c);
      CHECK(rc == QSA_OK, "%s rows_in_flight %d: status %d", d.name, rif, rc);
      check_decode_chain(d, c.s, false);
    }
    // optional outputs
    {
      DecodeCall c;
      c.lse = nullptr;
      stub::reset();
      CHECK(run(d.fn, c) == QSA_OK, "%s: lse may be NULL", d.name);
    }
    // causal chunks: MFMA scoring and the certified selection
    {
      DecodeCall c;
      c.s.batch = 8;
      c.s.queries = 256;
      c.s.rows_in_flight = 256;
      stub::reset();
      CHECK(run(d.fn, c) == QSA_OK, "%s: chunk shape", d.name);
      check_decode_chain(d, c.s, true);
      // a pass size the MFMA blocking cannot take falls back to the chain
      c.s.rows_in_flight = 6;
      stub::reset();
      CHECK(run(d.fn, c) == QSA_OK, "%s: chunk shape, 6 rows in flight", d.name);
      check_decode_chain(d, c.s, false);
    }
    // NULL arguments, one at a time
    {
      const char* names[] = {"index_q", "pooled", "pooled_off", "seq_len", "slot_map",
                             "slot_off", "k_cache", "v_cache", "q", "token_ids", "width",
                             "out", "ws"};
      for (int i = 0; i < 13; ++i) {
        DecodeCall c;
        switch (i) {
          case 0: c.index_q = nullptr; break;
          case 1: c.pooled = nullptr; break;
          case 2: c.pooled_off = nullptr; break;
          case 3: c.seq_len = nullptr; break;
          case 4: c.slot_map = nullptr; break;
          case 5: c.slot_off = nullptr; break;
          case 6: c.k_cache = nullptr; break;
          case 7: c.v_cache = nullptr; break;
          case 8: c.q = nullptr; break;
          case 9: c.token_ids = nullptr; break;
          case 10: c.width = nullptr; break;
          case 11: c.out = nullptr; break;
          case 12: c.ws = nullptr; break;
        }
        std::string what = std::string(d.name) + " NULL " + names[i];
        expect_rejected(d.fn, c, QSA_ERR_NULL, what.c_str());
      }
      DecodeCall c;
      c.null_shape = true;
      expect_rejected(d.fn, c, QSA_ERR_NULL, "NULL shape");
    }
    // misaligned 16-byte-access buffers
    {
      const char* names[] = {"index_q", "pooled", "k_cache", "v_cache", "q", "out",
                             "token_ids", "ws"};
      for (int i = 0; i < 8; ++i) {
        DecodeCall c;
        switch (i) {
          case 0: c.index_q = misalign(c.index_q); break;
          case 1: c.pooled = misalign(c.pooled); break;
          case 2: c.k_cache = misalign(c.k_cache); break;
          case 3: c.v_cache = misalign(c.v_cache); break;
          case 4: c.q = misalign(c.q); break;
          case 5: c.out = misalign(c.out); break;
          case 6: c.token_ids = misalign(c.token_ids); break;
          case 7: c.ws = misalign(c.ws); break;
        }
        std::string what = std::string(d.name) + " misaligned " + names[i];
        expect_rejected(d.fn, c, QSA_ERR_SHAPE, what.c_str());
      }
    }
    // workspace one byte short
    {
      DecodeCall c;
      c.ws_bytes = qsa_workspace_bytes(&c.s) - 1;
      expect_rejected(d.fn, c, QSA_ERR_WORKSPACE, "workspace one byte short");
      c.s.rows_in_flight = 3;
      c.ws_bytes = qsa_workspace_bytes(&c.s) - 1;
      expect_rejected(d.fn, c, QSA_ERR_WORKSPACE, "workspace one byte short, 3 rows in flight");
    }
    // a failing launch stops the chain
    for (int at : {0, 1, 2, 4}) {
      DecodeCall c;
      c.s.rows_in_flight = 8;
      stub::reset();
      stub::fail_at = at;
      const int rc = run(d.fn, c);
      CHECK(rc == QSA_ERR_HIP, "%s: launch %d fails -> status %d", d.name, at, rc);
      CHECK((int)stub::calls.size() == at + 1, "%s: %zu launches after failing launch %d",
            d.name, stub::calls.size(), at);
      stub::fail_at = -1;
    }
  }
}

// Shape fields one at a time, through qsa_decode (which needs every part of
// the shape) and qsa_workspace_bytes.
void test_shape_validation() {
  struct Case {
    const char* what;
    void (*edit)(qsa_shape&);
    int code;
  };
  const Case cases[] = {
      {"reserved", [](qsa_shape& s) { s.reserved = 1; }, QSA_ERR_SHAPE},
      {"batch 0", [](qsa_shape& s) { s.batch = 0; }, QSA_ERR_SHAPE},
      {"batch -1", [](qsa_shape& s) { s.batch = -1; }, QSA_ERR_SHAPE},
      {"queries 0", [](qsa_shape& s) { s.queries = 0; }, QSA_ERR_SHAPE},
      {"rows 65536", [](qsa_shape& s) { s.batch = 256; s.queries = 256; }, QSA_ERR_UNSUPPORTED},
      {"max_groups -64", [](qsa_shape& s) { s.max_groups = -64; }, QSA_ERR_SHAPE},
      {"max_groups 100", [](qsa_shape& s) { s.max_groups = 100; }, QSA_ERR_SHAPE},
      {"max_groups 2^28+64", [](qsa_shape& s) { s.max_groups = (1ll << 28) + 64; },
       QSA_ERR_UNSUPPORTED},
      {"rows_in_flight -1", [](qsa_shape& s) { s.rows_in_flight = -1; }, QSA_ERR_SHAPE},
      {"budget 0", [](qsa_shape& s) { s.budget_groups = 0; }, QSA_ERR_BUDGET},
      {"budget 1025", [](qsa_shape& s) { s.budget_groups = 1025; }, QSA_ERR_BUDGET},
      {"index_heads 0", [](qsa_shape& s) { s.index_heads = 0; }, QSA_ERR_SHAPE},
      {"index_heads 3", [](qsa_shape& s) { s.index_heads = 3; }, QSA_ERR_UNSUPPORTED},
      {"index_heads 32", [](qsa_shape& s) { s.index_heads = 32; }, QSA_ERR_UNSUPPORTED},
      {"index_dim 0", [](qsa_shape& s) { s.index_dim = 0; }, QSA_ERR_SHAPE},
      {"index_dim 48", [](qsa_shape& s) { s.index_dim = 48; }, QSA_ERR_UNSUPPORTED},
      {"index_dim 256", [](qsa_shape& s) { s.index_dim = 256; }, QSA_ERR_UNSUPPORTED},
      {"q_heads 0", [](qsa_shape& s) { s.q_heads = 0; }, QSA_ERR_SHAPE},
      {"q_heads 30 of 4 kv", [](qsa_shape& s) { s.q_heads = 30; }, QSA_ERR_SHAPE},
      {"gqa 3", [](qsa_shape& s) { s.q_heads = 12; }, QSA_ERR_UNSUPPORTED},
      {"gqa 32", [](qsa_shape& s) { s.q_heads = 128; }, QSA_ERR_UNSUPPORTED},
      {"kv_heads 0", [](qsa_shape& s) { s.kv_heads = 0; }, QSA_ERR_SHAPE},
      {"kv_heads 65536", [](qsa_shape& s) { s.kv_heads = 65536; s.q_heads = 65536; },
       QSA_ERR_UNSUPPORTED},
      {"head_dim 0", [](qsa_shape& s) { s.head_dim = 0; }, QSA_ERR_SHAPE},
      {"head_dim 96", [](qsa_shape& s) { s.head_dim = 96; }, QSA_ERR_UNSUPPORTED},
      {"kv_slots 0", [](qsa_shape& s) { s.kv_slots = 0; }, QSA_ERR_SHAPE},
      {"kv_slots 2^31", [](qsa_shape& s) { s.kv_slots = 1ll << 31; }, QSA_ERR_SHAPE},
  };
  for (const Case& k : cases) {
    DecodeCall c;
    k.edit(c.s);
    c.ws_bytes = (size_t)1 << 40;
    expect_rejected(qsa_decode, c, k.code, k.what);
  }
  // edges that are accepted
  const Case ok[] = {
      {"rows 65535", [](qsa_shape& s) { s.batch = 65535; s.rows_in_flight = 64; }, QSA_OK},
      {"max_groups 0", [](qsa_shape& s) { s.max_groups = 0; }, QSA_OK},
      {"max_groups 2^28", [](qsa_shape& s) { s.max_groups = 1ll << 28; s.rows_in_flight = 1; },
       QSA_OK},
      {"budget 1", [](qsa_shape& s) { s.budget_groups = 1; }, QSA_OK},
      {"budget 1024", [](qsa_shape& s) { s.budget_groups = 1024; }, QSA_OK},
      {"gqa 16", [](qsa_shape& s) { s.q_heads = 64; }, QSA_OK},
      {"gqa 1", [](qsa_shape& s) { s.q_heads = 4; }, QSA_OK},
      {"kv_slots 2^31-1", [](qsa_shape& s) { s.kv_slots = (1ll << 31) - 1; }, QSA_OK},
      {"index 1 x 32", [](qsa_shape& s) { s.index_heads = 1; s.index_dim = 32; }, QSA_OK},
      {"head_dim 64", [](qsa_shape& s) { s.head_dim = 64; }, QSA_OK},
  };
  for (const Case& k : ok) {
    DecodeCall c;
    k.edit(c.s);
    stub::reset();
    const int rc = run(qsa_decode, c);
    CHECK(rc == QSA_OK, "%s: status %d", k.what, rc);
    if (rc == QSA_OK) check_decode_chain(kDecoders[0], c.s, false);
  }
}

// Workspace size: linear in rows in flight and groups, independent of the
// K/V cache size, and no 32-bit overflow at 2^28 groups.
void test_workspace_bytes() {
  qsa_shape s = c4_shape();
  const size_t base = qsa_workspace_bytes(&s);
  CHECK(base > 0, "c4 workspace");
  CHECK(qsa_workspace_bytes(nullptr) == 0, "NULL shape");
  qsa_shape bad = s;
  bad.budget_groups = 0;
  CHECK(qsa_workspace_bytes(&bad) == 0, "invalid shape gives 0");
  qsa_shape big_cache = s;
  big_cache.kv_slots = (1ll << 31) - 1;
  CHECK(qsa_workspace_bytes(&big_cache) == base, "independent of the cache size");
  // per-row regions recomputed from the layout's definition
  size_t per_row = 0;
  qsa_shape one = s;
  one.rows_in_flight = 1;
  for (const Region& r : expected_regions(one)) per_row += r.bytes;
  CHECK(base >= 32 * per_row, "workspace %zu below the %zu bytes of 32 rows", base,
        32 * per_row);
  size_t prev = 0;
  for (int32_t rif = 1; rif <= 32; rif *= 2) {
    qsa_shape t = s;
    t.rows_in_flight = rif;
    const size_t w = qsa_workspace_bytes(&t);
    CHECK(w > prev, "grows with rows in flight (%d)", rif);
    CHECK(w >= (size_t)rif * per_row, "covers %d rows", rif);
    prev = w;
  }
  qsa_shape huge = s;
  huge.max_groups = 1ll << 28;
  huge.rows_in_flight = 1;
  const size_t wh = qsa_workspace_bytes(&huge);
  CHECK(wh >= ((size_t)1 << 28) * 4 + ((size_t)1 << 24) * 4, "2^28 groups: %zu", wh);
  huge.rows_in_flight = 0;
  const size_t wh32 = qsa_workspace_bytes(&huge);
  CHECK(wh32 >= 32 * (((size_t)1 << 28) * 4), "2^28 groups x 32 rows: %zu (no overflow)", wh32);
  // the byte ledger
  qsa_bytes b{};
  CHECK(qsa_accounting(&s, 32ll * 262144, &b) == QSA_OK, "accounting");
  CHECK(b.dense_mask == 0, "no dense mask");
  CHECK(b.raw_key == 32ll * 262144 * 128 * 4, "raw keys");
  CHECK(b.pooled_key == 32ll * 65536 * 128 * 4, "pooled keys");
  CHECK(b.kv == 2ll * 8388608 * 4 * 128 * 4, "K/V");
  CHECK(b.workspace == (int64_t)base, "workspace");
  CHECK(b.total == b.raw_key + b.pooled_key + b.kv + b.workspace, "total");
  CHECK(qsa_accounting(&s, -1, &b) == QSA_ERR_SHAPE, "negative tokens");
  CHECK(qsa_accounting(&s, 1, nullptr) == QSA_ERR_NULL, "NULL out");
  CHECK(qsa_accounting(nullptr, 1, &b) == QSA_ERR_NULL, "NULL shape");
}

// The per-step entry points.
void test_step_entry_points() {
  const qsa_shape s = c4_shape();
  const size_t need = qsa_workspace_bytes(&s);
  // step 1
  stub::reset();
  CHECK(qsa_score_groups(&s, dev(1), dev(2), dev<int64_t>(3), dev<int32_t>(4), dev(5), kStream) ==
            QSA_OK, "score");
  CHECK(stub::calls.size() == 1 && stub::calls[0].name == "score" && stub::calls[0].rows == 32 &&
            stub::calls[0].ptrs[5] == nullptr, "score: one launch, no maxima");
  const char* score_args[] = {"index_q", "pooled", "pooled_off", "seq_len", "scores"};
  for (int i = 0; i < 5; ++i) {
    const void* p[5] = {dev(1), dev(2), dev(3), dev(4), dev(5)};
    p[i] = nullptr;
    stub::reset();
    const int rc = qsa_score_groups(&s, (const float*)p[0], (const float*)p[1],
                                    (const int64_t*)p[2], (const int32_t*)p[3], (float*)p[4],
                                    kStream);
    CHECK(rc == QSA_ERR_NULL && stub::calls.empty(), "score NULL %s", score_args[i]);
  }
  stub::reset();
  CHECK(qsa_score_groups(&s, dev(1), misalign(dev(2)), dev<int64_t>(3), dev<int32_t>(4), dev(5),
                         kStream) == QSA_ERR_SHAPE && stub::calls.empty(), "score misaligned");
  // step 1 on MFMA for chunks
  qsa_shape ch = s;
  ch.batch = 2;
  ch.queries = 16;
  stub::reset();
  CHECK(qsa_score_groups_chunk(&ch, dev(1), dev(2), dev<int64_t>(3), dev<int32_t>(4), dev(5),
                               dev(6), kStream) == QSA_OK &&
            stub::count("chunk") == 1, "chunk scoring");
  qsa_shape ch2 = ch;
  ch2.index_heads = 2;
  stub::reset();
  CHECK(qsa_score_groups_chunk(&ch2, dev(1), dev(2), dev<int64_t>(3), dev<int32_t>(4), dev(5),
                               dev(6), kStream) == QSA_ERR_UNSUPPORTED && stub::calls.empty(),
        "chunk scoring with 2 index heads");
  qsa_shape ch3 = ch;
  ch3.queries = 6;
  stub::reset();
  CHECK(qsa_score_groups_chunk(&ch3, dev(1), dev(2), dev<int64_t>(3), dev<int32_t>(4), dev(5),
                               dev(6), kStream) == QSA_ERR_UNSUPPORTED && stub::calls.empty(),
        "chunk scoring with 6 queries");
  stub::reset();
  CHECK(qsa_score_groups_chunk(&ch, misalign(dev(1)), dev(2), dev<int64_t>(3), dev<int32_t>(4),
                               dev(5), dev(6), kStream) == QSA_ERR_SHAPE && stub::calls.empty(),
        "chunk scoring misaligned index_q");
  stub::reset();
  CHECK(qsa_score_groups_chunk(&ch, dev(1), dev(2), dev<int64_t>(3), dev<int32_t>(4), dev(5),
                               nullptr, kStream) == QSA_ERR_NULL && stub::calls.empty(),
        "chunk scoring NULL bound");
  // step 2, in passes
  for (int32_t rif : {0, 7}) {
    qsa_shape t = s;
    t.rows_in_flight = rif;
    const size_t w = qsa_workspace_bytes(&t);
    stub::reset();
    CHECK(qsa_select_topk(&t, dev(1), dev<int32_t>(2), dev<uint32_t>(3), kWs, w, kStream) ==
              QSA_OK, "select");
    const int64_t R = rif ? rif : 32, passes = (32 + R - 1) / R;
    CHECK((int64_t)stub::calls.size() == 2 * passes, "select: %zu launches", stub::calls.size());
    for (int64_t p = 0; p < passes && (int64_t)stub::calls.size() == 2 * passes; ++p) {
      const stub::Call& m = stub::calls[2 * p];
      const stub::Call& c = stub::calls[2 * p + 1];
      const int64_t r0 = p * R;
      CHECK(m.name == "segment_maxima" && c.name == "select", "select pass order");
      CHECK(c.row0 == r0 && c.rows == std::min<int64_t>(R, 32 - r0), "select pass rows");
      // the pass reads the caller's scores from its first row on
      CHECK(c.ptrs[0] == (const void*)(dev(1) + r0 * t.max_groups), "select pass scores");
      CHECK(in_ws(c.ptrs[1]) && (uintptr_t)c.ptrs[1] < (uintptr_t)kWs + w, "maxima in ws");
    }
    stub::reset();
    CHECK(qsa_select_topk(&t, dev(1), dev<int32_t>(2), dev<uint32_t>(3), kWs, w - 1, kStream) ==
              QSA_ERR_WORKSPACE && stub::calls.empty(), "select short workspace");
  }
  stub::reset();
  CHECK(qsa_select_topk(&s, dev(1), dev<int32_t>(2), nullptr, kWs, need, kStream) ==
            QSA_ERR_NULL && stub::calls.empty(), "select NULL bitmap");
  stub::reset();
  CHECK(qsa_select_topk(&s, misalign(dev(1)), dev<int32_t>(2), dev<uint32_t>(3), kWs, need,
                        kStream) == QSA_ERR_SHAPE && stub::calls.empty(), "select misaligned");
  // steps 3-5
  stub::reset();
  CHECK(qsa_emit_chronological(&s, dev<uint32_t>(1), dev<int32_t>(2), dev<int32_t>(3),
                               dev<int32_t>(4), kStream) == QSA_OK && stub::count("emit") == 1,
        "emit");
  stub::reset();
  CHECK(qsa_emit_chronological(&s, dev<uint32_t>(1), dev<int32_t>(2), misalign(dev<int32_t>(3)),
                               dev<int32_t>(4), kStream) == QSA_ERR_SHAPE && stub::calls.empty(),
        "emit misaligned ids");
  stub::reset();
  CHECK(qsa_emit_chronological(&s, nullptr, dev<int32_t>(2), dev<int32_t>(3), dev<int32_t>(4),
                               kStream) == QSA_ERR_NULL && stub::calls.empty(), "emit NULL");
  // steps 6-7
  stub::reset();
  CHECK(qsa_resolve_gather(&s, dev<int32_t>(1), dev<int32_t>(2), dev<int32_t>(3),
                           dev<int32_t>(4), dev<int64_t>(5), dev(6), dev(7), dev(8), dev(9),
                           nullptr, kStream) == QSA_OK && stub::count("gather") == 1,
        "gather, phys_slots optional");
  for (int i = 0; i < 4; ++i) {
    const float* p[4] = {dev(6), dev(7), dev(8), dev(9)};
    p[i] = misalign(p[i]);
    stub::reset();
    CHECK(qsa_resolve_gather(&s, dev<int32_t>(1), dev<int32_t>(2), dev<int32_t>(3),
                             dev<int32_t>(4), dev<int64_t>(5), p[0], p[1], (float*)p[2],
                             (float*)p[3], nullptr, kStream) == QSA_ERR_SHAPE &&
              stub::calls.empty(), "gather misaligned %d", i);
  }
  stub::reset();
  CHECK(qsa_resolve_gather(&s, dev<int32_t>(1), dev<int32_t>(2), dev<int32_t>(3), nullptr,
                           dev<int64_t>(5), dev(6), dev(7), dev(8), dev(9), nullptr, kStream) ==
            QSA_ERR_NULL && stub::calls.empty(), "gather NULL slot map");
  // step 8, in passes; each pass reads its own rows of the compact scratch
  for (int32_t rif : {0, 5}) {
    qsa_shape t = s;
    t.rows_in_flight = rif;
    const size_t w = qsa_workspace_bytes(&t);
    stub::reset();
    CHECK(qsa_online_attend(&t, dev(1), dev(2), dev(3), dev<int32_t>(4), 0.1f, dev(5), nullptr,
                            kWs, w, kStream) == QSA_OK, "attend");
    const int64_t R = rif ? rif : 32, passes = (32 + R - 1) / R;
    const int64_t compact_row = (4 * 512 + 4) * 4 * 128;
    CHECK((int64_t)stub::calls.size() == 2 * passes, "attend launches");
    for (int64_t p = 0; p < passes && (int64_t)stub::calls.size() == 2 * passes; ++p) {
      const stub::Call& a = stub::calls[2 * p];
      CHECK(a.name == "attend" && stub::calls[2 * p + 1].name == "merge", "attend order");
      CHECK(a.ptrs[1] == (const void*)(dev(2) + p * R * compact_row), "attend pass K rows");
      CHECK(a.ptrs[2] == (const void*)(dev(3) + p * R * compact_row), "attend pass V rows");
    }
    stub::reset();
    CHECK(qsa_online_attend(&t, dev(1), dev(2), dev(3), dev<int32_t>(4), 0.1f, dev(5), nullptr,
                            kWs, w - 1, kStream) == QSA_ERR_WORKSPACE && stub::calls.empty(),
          "attend short workspace");
  }
  stub::reset();
  CHECK(qsa_online_attend(&s, dev(1), dev(2), dev(3), dev<int32_t>(4), 0.1f, misalign(dev(5)),
                          nullptr, kWs, need, kStream) == QSA_ERR_SHAPE && stub::calls.empty(),
        "attend misaligned out");
  // indexed attention
  stub::reset();
  CHECK(qsa_online_attend_indexed(&s, dev(1), dev(2), dev(3), 0, dev<int32_t>(4),
                                  dev<int32_t>(5), 0.1f, dev(6), nullptr, kWs, need, kStream) ==
            QSA_ERR_SHAPE && stub::calls.empty(), "indexed: no rows");
  stub::reset();
  CHECK(qsa_online_attend_indexed(&s, dev(1), dev(2), dev(3), 1ll << 31, dev<int32_t>(4),
                                  dev<int32_t>(5), 0.1f, dev(6), nullptr, kWs, need, kStream) ==
            QSA_ERR_SHAPE && stub::calls.empty(), "indexed: 2^31 rows");
  stub::reset();
  CHECK(qsa_online_attend_indexed(&s, dev(1), dev(2), dev(3), 1000, dev<int32_t>(4),
                                  dev<int32_t>(5), 0.1f, dev(6), nullptr, kWs, need, kStream) ==
            QSA_OK && stub::count("attend") == 1 && stub::count("merge") == 1, "indexed");
  // union gather: one union for all rows
  stub::reset();
  CHECK(qsa_union_gather(&s, dev<int32_t>(1), dev<int32_t>(2), dev<int32_t>(3), dev<int32_t>(4),
                         dev<int64_t>(5), dev(6), dev(7), dev(8), dev(9), dev<int32_t>(10),
                         nullptr, kWs, need, kStream) == QSA_OK && stub::count("union") == 1,
        "union gather");
  qsa_shape split = s;
  split.rows_in_flight = 4;
  stub::reset();
  CHECK(qsa_union_gather(&split, dev<int32_t>(1), dev<int32_t>(2), dev<int32_t>(3),
                         dev<int32_t>(4), dev<int64_t>(5), dev(6), dev(7), dev(8), dev(9),
                         dev<int32_t>(10), nullptr, kWs, (size_t)1 << 40, kStream) ==
            QSA_ERR_UNSUPPORTED && stub::calls.empty(), "union gather in passes");
  stub::reset();
  CHECK(qsa_union_gather(&s, dev<int32_t>(1), dev<int32_t>(2), dev<int32_t>(3), dev<int32_t>(4),
                         dev<int64_t>(5), dev(6), dev(7), dev(8), dev(9), nullptr, nullptr, kWs,
                         need, kStream) == QSA_ERR_NULL && stub::calls.empty(),
        "union gather NULL positions");
  // bounded dense row: IDs once, attention per pass
  qsa_shape dn = s;
  dn.rows_in_flight = 10;
  const size_t wd = qsa_workspace_bytes(&dn);
  stub::reset();
  CHECK(qsa_dense_attend(&dn, dev<int32_t>(1), dev<int32_t>(2), dev<int64_t>(3), dev(4), dev(5),
                         dev(6), 0.1f, dev<int32_t>(7), dev<int32_t>(8), dev(9), nullptr, kWs, wd,
                         kStream) == QSA_OK, "dense");
  CHECK(stub::count("dense_ids") == 1 && stub::count("attend") == 4 && stub::count("merge") == 4,
        "dense: IDs once, four passes");
  stub::reset();
  CHECK(qsa_dense_attend(&dn, dev<int32_t>(1), dev<int32_t>(2), dev<int64_t>(3), dev(4), dev(5),
                         dev(6), 0.1f, dev<int32_t>(7), dev<int32_t>(8), dev(9), nullptr, kWs,
                         wd - 1, kStream) == QSA_ERR_WORKSPACE && stub::calls.empty(),
        "dense short workspace");
  // pooling
  stub::reset();
  CHECK(qsa_pool_groups(&s, dev(1), dev<int64_t>(2), dev<int32_t>(3), nullptr, dev(4),
                        dev<int64_t>(5), kStream) == QSA_OK && stub::count("pool") == 1,
        "pool, first_group optional");
  stub::reset();
  CHECK(qsa_pool_groups(&s, misalign(dev(1)), dev<int64_t>(2), dev<int32_t>(3), nullptr, dev(4),
                        dev<int64_t>(5), kStream) == QSA_ERR_SHAPE && stub::calls.empty(),
        "pool misaligned");
  stub::reset();
  CHECK(qsa_pool_groups(&s, dev(1), dev<int64_t>(2), dev<int32_t>(3), nullptr, dev(4), nullptr,
                        kStream) == QSA_ERR_NULL && stub::calls.empty(), "pool NULL offsets");
}

// Stage timer: events only around timed stages, first pass only, read-back,
// capacity, reset and teardown.
void test_timer() {
  qsa_timer* t = nullptr;
  CHECK(qsa_timer_create(4, 1, nullptr) == QSA_ERR_NULL, "NULL out");
  CHECK(qsa_timer_create(0, 1, &t) == QSA_ERR_SHAPE, "no calls");
  CHECK(qsa_timer_create((1 << 20) + 1, 1, &t) == QSA_ERR_SHAPE, "too many calls");
  CHECK(qsa_timer_create(4, 0, &t) == QSA_ERR_SHAPE, "no stage");
  CHECK(qsa_timer_create(4, 1u << QSA_DECODE_STAGES, &t) == QSA_ERR_SHAPE, "stage past the end");
  const int live0 = stub::events_live;
  // stages 0 and 2 timed: events 0, 1 (around stage 0) and 2, 3 (around stage 2)
  CHECK(qsa_timer_create(3, 0x5u, &t) == QSA_OK && t, "create");
  CHECK(stub::events_live == live0 + 3 * (QSA_DECODE_STAGES + 1), "events created");
  for (int c = 0; c < 3; ++c) {
    DecodeCall d;
    d.s.rows_in_flight = 16;  // two passes: only the first is timed
    d.timer = t;
    stub::reset();
    CHECK(run(qsa_decode, d) == QSA_OK, "timed call %d", c);
    CHECK(stub::count("event") == 4, "call %d: %d events", c, stub::count("event"));
    // the events bracket the first pass's score and gather launches
    std::vector<std::string> seq;
    for (const stub::Call& k : stub::calls) seq.push_back(k.name);
    const std::vector<std::string> first = {"event", "score", "event", "select", "event",
                                            "gather", "event", "attend", "merge"};
    CHECK(seq.size() >= first.size() && std::equal(first.begin(), first.end(), seq.begin()),
          "call %d: event placement", c);
  }
  {
    DecodeCall d;
    d.timer = t;
    expect_rejected(qsa_decode, d, QSA_ERR_SHAPE, "timer full");
  }
  float ms[3 * QSA_DECODE_STAGES];
  int32_t n = -1;
  CHECK(qsa_timer_read(t, ms, &n) == QSA_OK && n == 3, "read %d calls", n);
  for (int c = 0; c < 3; ++c)
    for (int st = 0; st < QSA_DECODE_STAGES; ++st) {
      const float want = (st == 0 || st == 2) ? 0.25f : -1.0f;
      CHECK(ms[c * QSA_DECODE_STAGES + st] == want, "ms[%d][%d] = %g", c, st,
            ms[c * QSA_DECODE_STAGES + st]);
    }
  CHECK(qsa_timer_read(t, nullptr, &n) == QSA_ERR_NULL, "read NULL");
  qsa_timer_reset(t);
  CHECK(qsa_timer_read(t, ms, &n) == QSA_OK && n == 0, "reset");
  qsa_timer_destroy(t);
  qsa_timer_reset(nullptr);
  qsa_timer_destroy(nullptr);
  CHECK(stub::events_live == live0, "events destroyed (%d live)", stub::events_live);
  // every stage timed
  CHECK(qsa_timer_create(1, QSA_TIMER_ALL, &t) == QSA_OK, "create all");
  DecodeCall d;
  d.timer = t;
  stub::reset();
  CHECK(run(qsa_decode_fused, d) == QSA_OK, "fused timed");
  CHECK(stub::count("event") == QSA_DECODE_STAGES + 1, "all stages: %d events",
        stub::count("event"));
  CHECK(qsa_timer_read(t, ms, &n) == QSA_OK && n == 1, "read all");
  qsa_timer_destroy(t);
}

void test_status_strings() {
  std::vector<std::string> seen;
  for (int code = 0; code <= 7; ++code) {
    const char* s = qsa_status_string(code);
    CHECK(s && *s, "status %d has a string", code);
    if (s) seen.push_back(s);
  }
  std::sort(seen.begin(), seen.end());
  CHECK(std::unique(seen.begin(), seen.end()) == seen.end(), "distinct status strings");
  CHECK(strcmp(qsa_status_string(99), "unknown status") == 0, "unknown status");
  CHECK(strstr(qsa_version(), "gfx950") != nullptr, "version names the target");
}

}  // namespace

int main() {
  test_shape_validation();
  test_decode_family();
  test_workspace_bytes();
  test_step_entry_points();
  test_timer();
  test_status_strings();
  printf("host lane: %d checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
