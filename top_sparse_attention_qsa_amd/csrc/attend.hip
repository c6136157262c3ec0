// attend.hip -- step 8: F32 online-softmax attention over the compact row.
//
// Attention over the same rows is permutation invariant only in exact
// arithmetic; in F32 the visit order shows in the last bits, so one canonical
// order is fixed (AFN-017 "Top-k chooses the set; time chooses the order",
// §Floating point makes order observable).  The order used here depends on
// the width alone.  The compact row is cut into chunks of kAttnChunk
// consecutive rows and the chunks into ranges of kAttnRange.  Within a range,
// each of four row slices of a chunk (16 rows) belongs to one wavefront,
// which keeps an online-softmax state per query head over its slices of the
// range's chunks in ascending order: running maximum, weights exp(s - m),
// rescale of the weight sum (a fixed butterfly per chunk) and of the
// accumulators (a chronological accumulation over the slice's rows) when the
// maximum grows.  At the range's end the four states are rescaled to the
// range maximum and added in wavefront order: one partial (max, denominator,
// accumulator) per range, and the range partials are merged the same way in
// ascending range order.  No float atomics: results are run-to-run
// identical.
//
// attend_chunk_kernel: a persistent workgroup walks its (range, KV head, row)
// items chunk by chunk and stores a range's partial after its last chunk, so
// the merge reads one partial per range.  Each chunk serves every query head
// of the KV head's GQA group (query head hq reads KV head hq / (H_q/H_kv)).
// Scores: the chunk's K rows and query heads are staged in LDS; wavefront w
// scores rows 16w..16w+15 for every head of the group on
// v_mfma_f32_16x16x4_f32 (one column per head); the maxima and sums over a
// wavefront's four lane rows use the VALU cross-lane swaps.  P.V: wavefront w
// accumulates its rows in row order with lane = output dimension, reading its
// V rows straight from memory (issued before the score phase), on
// v_mfma_f32_4x4x1_16b_f32 when the group has a multiple of four heads (one
// product per step, the bits of the VALU fused multiply-adds).  The
// wavefronts meet only at the K staging and at range ends: two barriers per
// chunk.  merge_kernel: four wavefronts per (query head, row).
#include <atomic>
#include <type_traits>

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int C = kAttnChunk;
constexpr int RC = kAttnRange;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer resource on this architecture (32-bit data format,
// no swizzle, no index stride): loads past num_records return zeros.
constexpr int kBufferFormat = 0x00020000;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D, int GQ>
struct AttnCfg {
  static constexpr int NW = 4;           // wavefronts; with GQ < 4 some have no score work
  static constexpr int NT = NW * kWave;
  static_assert(GQ <= 16, "one MFMA column per query head");
  static constexpr int KPW = C / NW;     // compact rows per wavefront in the P.V phase
  static constexpr int KP = D + 4;       // padded K row, floats
  static constexpr int DPL = D / kWave;  // output dims per lane
  static constexpr int KV4 = C * D / 4 / NT;  // K float4 per thread per chunk
  static constexpr int QV4 = (GQ * D / 4 + NT - 1) / NT;  // q float4 per thread per item
  static constexpr int OV4 = QV4;                          // partial float4 per thread per item
  static constexpr int KFLOATS = C * KP;
  static constexpr int RFLOATS = NW * GQ * D;  // per-wavefront P.V partials, aliasing K
  static constexpr int SFLOATS = KFLOATS > RFLOATS ? KFLOATS : RFLOATS;
};

// Work item it -> (range, local row, KV head), range-major, so that the items
// of one range index are consecutive and a launch whose grid divides the item
// count of the non-empty ranges gives every workgroup the same amount of
// work.  The `chunk` digit of an item holds its range; a position inside the
// item adds the chunk's offset in the range.
struct Item {
  int chunk;
  int hk;
  int64_t lrow;
};
__device__ __forceinline__ Item item_of(int64_t it, int64_t rows, int kv_heads) {
  Item x;
  const int64_t per_chunk = rows * kv_heads;
  x.chunk = (int)(it / per_chunk);
  const int64_t r = it - (int64_t)x.chunk * per_chunk;
  x.lrow = r / kv_heads;
  x.hk = (int)(r - x.lrow * kv_heads);
  return x;
}

// Stepping a workgroup's item by the grid size adds the grid size's own
// (range, row, head) digits with carries, so the item loop does no 64-bit
// division (which the compiler expands to over a hundred scalar
// instructions).  Digits past the last range are only used behind `it < items`.
__device__ __forceinline__ Item item_step(Item x, const Item& step, int64_t rows, int kv_heads) {
  x.hk += step.hk;
  int64_t carry = 0;
  if (x.hk >= kv_heads) {
    x.hk -= kv_heads;
    carry = 1;
  }
  x.lrow += step.lrow + carry;
  int carry2 = 0;
  if (x.lrow >= rows) {
    x.lrow -= rows;
    carry2 = 1;
  }
  x.chunk += step.chunk + carry2;
  return x;
}

// Where a work item's K and V rows come from.  Compact: the scratch written
// by the gather (row i of the row's compact copy).  Fused: straight from the
// K/V cache; the chunk's logical IDs are resolved through the slot map once,
// inside this kernel, two items ahead of their use, into a three-deep LDS
// ring (wavefront 0: ID loads at the top of an item, slot-map loads after its
// scores, LDS write at its end), so the row loads of the next item can be
// issued as early as in the compact path.  Union: like fused, but the
// positions are read from a per-row list into the union scratch of the chunk
// gather (union.hip) and need no slot map.  All three produce the same bits.
enum Mode { kCompact = 0, kFused = 1, kUnion = 2 };
struct RowSource {
  const float* k_compact;
  const float* v_compact;
  const int32_t* token_ids;  // fused: global rows; union: positions, local rows
  const int32_t* seq_len;
  const int32_t* slot_map;
  const int64_t* slot_off;
  const float* k_cache;
  const float* v_cache;
  int64_t kv_slots;
  int32_t queries;
};

// Three resident workgroups per compute unit (at most 168 VGPRs) where the
// GQA group fits them without spills; two for the compact mode at D * GQ =
// 1024 (measured slightly faster: no spill, more registers for the loads).
template <int D, int GQ, int MODE>
__global__ void __launch_bounds__(4 * kWave)
__attribute__((amdgpu_waves_per_eu((MODE == kCompact ? D * GQ < 1024 : D * GQ <= 1024) ? 3 : 2)))
attend_chunk_kernel(const float* __restrict__ q, RowSource src, const int32_t* __restrict__ width,
                    int32_t q_heads, int32_t kv_heads, int32_t stride, int32_t n_chunks,
                    float scale, int64_t row0, int64_t rows, float* __restrict__ part_acc,
                    float* __restrict__ part_ml) {
  using A = AttnCfg<D, GQ>;
  constexpr bool FUSED = MODE != kCompact;
  constexpr int NW = A::NW, NT = A::NT, KPW = A::KPW, KP = A::KP;
  constexpr int DPL = A::DPL, KV4 = A::KV4, QV4 = A::QV4, OV4 = A::OV4;
  __shared__ float4 smem4[A::SFLOATS / 4];
  __shared__ float4 ql4[GQ * D / 4];          // the item's query heads
  __shared__ float4 ps4[GQ * C / 4];
  __shared__ int32_t ring[FUSED ? 3 : 1][C];  // resolved slots (-1: invalid ID or slot)
  __shared__ float mw_sh[NW][GQ];             // per wavefront and head: max over its 16 rows
  __shared__ float lw_sh[NW][GQ];             // per wavefront and head: sum of its weights
  float* smem = reinterpret_cast<float*>(smem4);
  float* ps = reinterpret_cast<float*>(ps4);

  const int tid = (int)threadIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();
  // range items (range of RC consecutive chunks, local row, KV head),
  // range-major; a workgroup walks the chunks of each of its range items in
  // order and folds their partials into one per range
  const int n_ranges = attn_parts(n_chunks);
  const int64_t items = (int64_t)n_ranges * rows * kv_heads;
  const int64_t rstride = (int64_t)kv_heads * D;  // floats between compact or cache rows

  // Every load is unconditional: rows past a chunk's width read zeros (compact
  // mode, through the item's buffer resource) or the chunk's last valid row
  // (cache and union modes, always in bounds); their scores are replaced by
  // -inf and their weights p are 0, so they add nothing.  No load sits behind
  // a branch.  Prefetches are unconditional as well: an empty or out-of-range
  // next item reads nothing (compact: an empty resource) or row 0 of the last
  // item's chunk, which always exists, and ignores it.
  auto chunk_rows = [&](const Item& x) -> int {  // rows of this chunk, 0 = no work
    const int32_t w = width[row0 + x.lrow];
    const int c0 = x.chunk * C;
    if (w <= 0 || w > stride - 1 || c0 >= w) return 0;
    return (w - c0) < C ? (w - c0) : C;
  };
  // address of row i (< cn) of item x for KV head x.hk, in K or V
  auto row_ptr = [&](const float* compact, const float* cache, const Item& x, int i,
                     int ring_slot) -> const float* {
    if constexpr (FUSED) {
      const int32_t sl = ring[ring_slot][i];
      return cache + (int64_t)(sl >= 0 ? sl : 0) * rstride + (int64_t)x.hk * D;
    } else {
      return compact + ((x.lrow * kv_heads + x.hk) * stride + (int64_t)x.chunk * C + i) *
                           (int64_t)D;
    }
  };
  float4 kst[KV4];
  float4 qst[QV4];
  float vreg[KPW][DPL];
  // K rows and the query heads of item x (q staged in LDS next to K, so the
  // score loop reads it with broadcast LDS loads instead of scalar loads
  // that would each wait on a cache round trip)
  // Compact rows are read through a buffer resource per item that covers
  // only the item's valid rows (the loads return raw 32-bit words, bit-cast
  // to float): rows past the width read as zeros (their
  // scores are replaced by -inf and their weights are 0), so the loads need
  // no clamp and no 64-bit address arithmetic.  The item is uniform across
  // the workgroup, so the descriptor is kept in scalar registers.
  auto item_rsrc = [&](const float* compact, const Item& x, int cn_raw) {
    const float* base =
        compact + ((x.lrow * kv_heads + x.hk) * stride + (int64_t)x.chunk * C) * (int64_t)D;
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const int bytes = __builtin_amdgcn_readfirstlane(cn_raw * D * 4);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                             (short)0, bytes, kBufferFormat);
  };
  auto load_q = [&](const Item& x) {
    const float* qg = q + ((row0 + x.lrow) * q_heads + (int64_t)x.hk * GQ) * D;
#pragma unroll
    for (int r = 0; r < QV4; ++r) {
      const int e = tid + r * NT;
      qst[r] = *reinterpret_cast<const float4*>(qg + 4 * (e < GQ * D / 4 ? e : 0));
    }
  };
  auto load_k = [&](const Item& x, int cn_raw, int ring_slot) {
    if constexpr (MODE == kCompact) {
      const auto rs = item_rsrc(src.k_compact, x, cn_raw);
#pragma unroll
      for (int r = 0; r < KV4; ++r) {  // float4 e of the item's rows is at byte 16e
        const f32x4 v = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (tid + r * NT) * 16, 0, 0));
        kst[r] = make_float4(v.x, v.y, v.z, v.w);
      }
      return;
    }
    const int cn = cn_raw > 0 ? cn_raw : 1;
#pragma unroll
    for (int r = 0; r < KV4; ++r) {
      const int e = tid + r * NT;
      const int i = e / (D / 4);
      const int c = e - i * (D / 4);
      const int ic = i < cn ? i : cn - 1;
      kst[r] = *reinterpret_cast<const float4*>(
          row_ptr(src.k_compact, src.k_cache, x, ic, ring_slot) + 4 * c);
    }
  };
  auto load_v_rows = [&](const Item& x, int cn_raw, int ring_slot, auto J0, auto J1) {
    constexpr int j0 = decltype(J0)::value, j1 = decltype(J1)::value;
    if constexpr (MODE == kCompact) {
      const auto rs = item_rsrc(src.v_compact, x, cn_raw);
#pragma unroll
      for (int j = j0; j < j1; ++j) {
        const int i = wave * KPW + j;
        if constexpr (DPL == 2) {
          const f32x2 v = __builtin_bit_cast(
              f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (i * D + 2 * lane) * 4, 0, 0));
          vreg[j][0] = v.x;
          vreg[j][1] = v.y;
        } else {
          vreg[j][0] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(rs, (i * D + lane) * 4, 0, 0));
        }
      }
      return;
    }
    const int cn = cn_raw > 0 ? cn_raw : 1;
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const int i = wave * KPW + j;
      const int ic = i < cn ? i : cn - 1;
      const float* vp = row_ptr(src.v_compact, src.v_cache, x, ic, ring_slot);
      if constexpr (DPL == 2) {
        const float2 v2 = *reinterpret_cast<const float2*>(vp + 2 * lane);
        vreg[j][0] = v2.x;
        vreg[j][1] = v2.y;
      } else {
        vreg[j][0] = vp[lane];
      }
    }
  };
  auto load_v = [&](const Item& x, int cn_raw, int ring_slot) {
    load_v_rows(x, cn_raw, ring_slot, std::integral_constant<int, 0>{},
                std::integral_constant<int, KPW>{});
  };
  // Fused resolution of item x in three phases on wavefront 0, lane i = row i:
  // IDs loaded (before the next item's K loads, so that waiting for them
  // does not wait for K), the slot map read (its value checked only when the
  // slots are stored, so the load is not waited for at once), and the slots
  // written to the LDS ring at the end of the item.
  int32_t id_reg = -1, len_reg = 0, sl_raw = 0;
  int64_t soff_reg = 0;
  bool id_ok = false;
  auto resolve_ids = [&](const Item& x, int cn_x) {
    if constexpr (FUSED) {
      if (wave == 0) {
        const int64_t row = MODE == kUnion ? x.lrow : row0 + x.lrow;
        id_reg = lane < cn_x ? src.token_ids[row * stride + (int64_t)x.chunk * C + lane] : -1;
        if constexpr (MODE == kFused) {
          const int32_t b = (int32_t)row / src.queries;  // rows fit in 32 bits (validated)
          len_reg = src.seq_len[b];
          soff_reg = src.slot_off[b];
        }
      }
    }
  };
  auto resolve_slots = [&](const Item& x, int cn_x) {
    if constexpr (FUSED) {
      if (wave == 0 && MODE == kUnion) {
        id_ok = lane < cn_x && id_reg >= 0;
        sl_raw = id_reg;
      } else if (wave == 0) {
        const int32_t row = (int32_t)(row0 + x.lrow);
        const int32_t b = row / src.queries;
        const int64_t n = (int64_t)len_reg - src.queries + 1 + (row - b * src.queries);
        id_ok = lane < cn_x && id_reg >= 0 && (int64_t)id_reg < n;
        if (id_ok) sl_raw = src.slot_map[soff_reg + id_reg];
      }
    }
  };
  // rows past the width get slot 0 (a row that exists), invalid IDs or slots -1
  auto resolve_store = [&](int ring_slot, int cn_x) {
    if constexpr (FUSED) {
      if (wave == 0)
        ring[ring_slot][lane] =
            lane < cn_x ? ((id_ok && sl_raw >= 0 && (int64_t)sl_raw < src.kv_slots) ? sl_raw : -1)
                        : 0;
    }
  };

  // positions: range item `it` (digits r: range, row, head) and chunk `sub`
  // of the range; past the last range item, the last range item's first
  // chunk stands in for address computations
  struct Pos {
    int64_t it;
    Item r;
    int sub;
  };
  const Item step = item_of(gridDim.x, rows, kv_heads);
  const Item last = item_of(items - 1, rows, kv_heads);
  auto chunk_of = [&](const Pos& p) -> Item {
    Item x = p.it < items ? p.r : last;
    x.chunk = x.chunk * RC + (p.it < items ? p.sub : 0);
    return x;
  };
  auto rows_of = [&](const Pos& p) -> int { return p.it < items ? chunk_rows(chunk_of(p)) : 0; };
  // the next position: the next chunk of the range while it has rows, else
  // the first chunk of the workgroup's next range item
  auto advance = [&](const Pos& p) -> Pos {
    if (p.it < items && p.sub + 1 < RC) {
      Pos q = p;
      ++q.sub;
      if (rows_of(q) > 0) return q;
    }
    return Pos{p.it + (int64_t)gridDim.x, item_step(p.r, step, rows, kv_heads), 0};
  };
  int j = 0;  // this workgroup's chunk sequence number
  Pos pcur{(int64_t)blockIdx.x, item_of(blockIdx.x, rows, kv_heads), 0};
  Item cur = chunk_of(pcur);
  int cn = rows_of(pcur);
  if constexpr (FUSED) {
    // chunks 0 and 1 of this workgroup are resolved up front
    const Pos p1 = advance(pcur);
    const Item x1 = chunk_of(p1);
    resolve_ids(cur, cn);
    resolve_slots(cur, cn);
    resolve_store(0, cn);
    resolve_ids(x1, rows_of(p1));
    resolve_slots(x1, rows_of(p1));
    resolve_store(1, rows_of(p1));
    __syncthreads();
  }
  // K, then q, then V here as in the loop: the wait for K and q at the top of
  // an item can then leave V (issued after them) in flight on every path into
  // the loop
  load_k(cur, cn, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_q(cur);
  __builtin_amdgcn_sched_barrier(0);
  load_v(cur, cn, 0);
  // this wavefront's running softmax state over the chunks of the current
  // range: per head, the maximum and weight sum over its rows so far (lane
  // (li, lq) tracks head li) and the P.V accumulators (lane = dimensions)
  float m_run = -INFINITY, l_run = 0.0f;
  float acc[GQ][DPL];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int t = 0; t < DPL; ++t) acc[h][t] = 0.0f;
  while (pcur.it < items) {
    const Pos pnx = advance(pcur);
    const Pos pnx2 = advance(pnx);
    const Item nxt = chunk_of(pnx);
    const int cn_next = rows_of(pnx);
    const Item nxt2 = chunk_of(pnx2);
    const int cn_next2 = rows_of(pnx2);
    const int rs_cur = FUSED ? j % 3 : 0, rs_next = FUSED ? (j + 1) % 3 : 0;
    if (cn == 0 && pnx.it >= items) break;
    {
      // stage this item's K in LDS (rows past the width hold a copy of the
      // last row -- their scores are replaced by -inf, so they are never
      // used; rows whose ID or slot was out of range are NaN, as in the
      // compact path)
      __syncthreads();  // the previous item is done with LDS
#pragma unroll
      for (int r = 0; r < KV4; ++r) {
        const int e = tid + r * NT;
        const int i = e / (D / 4);
        const int c = e - i * (D / 4);
        float4 kv = kst[r];
        if constexpr (FUSED) {
          if (i < cn && ring[rs_cur][i] < 0) {
            const float nan = __int_as_float(0x7fc00000);
            kv = make_float4(nan, nan, nan, nan);
          }
        }
        smem4[(i * KP) / 4 + c] = kv;
      }
      // (unconditional when the threads cover q exactly: a store behind a
      // branch leaves the q load possibly pending on the other path, and the
      // next write to its registers would wait for V loads issued after it)
#pragma unroll
      for (int r = 0; r < QV4; ++r) {
        const int e = tid + r * NT;
        if ((GQ * D / 4) % NT == 0 || e < GQ * D / 4) ql4[e] = qst[r];
      }
      __syncthreads();
      // next item's K streams in under this item; the scheduling barriers keep
      // the compiler from hoisting it (or V below) above the last use of the
      // registers it refills, which would double the register footprint
      __builtin_amdgcn_sched_barrier(0);
      resolve_ids(nxt2, cn_next2);
      __builtin_amdgcn_sched_barrier(0);
      load_k(nxt, cn_next, rs_next);
      __builtin_amdgcn_sched_barrier(0);  // issued before the score phase

      // scores on v_mfma_f32_16x16x4_f32: S[row 16w + 4lq + r][head li] in
      // sacc[r] (lane (li, lq) = lane % 16, lane / 16); k-step (c, e) covers
      // dim 16c + 4lq + e in both operands.  Head columns past the group
      // repeat head 0: MFMA columns are independent, and those lanes' scores
      // are never stored or exchanged (a masked operand would put a branch
      // and a full LDS wait into every k-step).  Two independent accumulators
      // (even and odd e), added at the end.
      const int li = lane & 15, lq = lane >> 4;
      const bool hcol = li < GQ;
      f32x4 sp[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) sp[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const float4 a4 = smem4[((16 * wave + li) * KP + 16 * c + 4 * lq) / 4];
        const float4 b4 = ql4[((hcol ? li : 0) * D + 16 * c + 4 * lq) / 4];
        sp[0] = mfma4(a4.x, b4.x, sp[0]);
        sp[1] = mfma4(a4.y, b4.y, sp[1]);
        sp[0] = mfma4(a4.z, b4.z, sp[0]);
        sp[1] = mfma4(a4.w, b4.w, sp[1]);
      }
      const f32x4 sacc = sp[0] + sp[1];
      // softmax, per wavefront: the running maximum per head over this
      // wavefront's rows of the range so far (no exchange between wavefronts
      // until the range ends); the accumulators and the weight sum so far are
      // rescaled by alpha = exp(m_old - m_new)
      const int rbase = 16 * wave + 4 * lq;  // rows rbase .. rbase+3 in this lane
      float sc[4];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = rbase + r < cn ? sacc[r] * scale : -INFINITY;
        mx = fmaxf(mx, sc[r]);
      }
      mx = xor16(mx, MaxOp{});  // over the four lane rows: lq = 0..3
      mx = xor32(mx, MaxOp{});
      resolve_slots(nxt2, cn_next2);
      const float m_new = fmaxf(m_run, mx);
      // a head with no row so far keeps alpha = 1 (its state is all zeros)
      const float alpha = m_new == -INFINITY ? 1.0f : expf(m_run - m_new);
      {
        const int h = hcol ? li : 0;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = rbase + r < cn ? expf(sc[r] - m_new) : 0.0f;
        float l = ((p[0] + p[1]) + p[2]) + p[3];
        l = xor16(l, AddOp{});
        l = xor32(l, AddOp{});
        l_run = l_run * alpha + l;
        m_run = m_new;
        if (hcol) ps4[(h * C + rbase) / 4] = make_float4(p[0], p[1], p[2], p[3]);  // read back below
      }

      // P.V over this wavefront's rows, in row order, onto the rescaled
      // running accumulators; lane owns dims lane*DPL..  (alpha of head h is
      // lane h's)
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float ah = read_lane(alpha, h);
#pragma unroll
        for (int t = 0; t < DPL; ++t) acc[h][t] = acc[h][t] * ah;
      }
      if constexpr (GQ % 4 == 0) {
        // on v_mfma_f32_4x4x1_16b_f32: block b (lanes 4b..4b+3) adds A[i] *
        // B[j] to D[i][j] with one rounding, A[i] from lane 4b+i, B[j] from
        // lane 4b+j, D[i][j] in register i of lane 4b+j.  With A = the weight
        // of head 4hq + (lane mod 4) for the row and B = the lane's V value,
        // register i of lane l accumulates head 4hq + i at the lane's own
        // dimensions: the same fused multiply-adds, in the same row order, as
        // on the VALU, so the same bits.  Rows go in quads; once a quad is
        // done for every head its V registers are refilled with the next
        // chunk's rows, so those loads start a part of P.V earlier.
        typedef float v4f __attribute__((ext_vector_type(4)));
        const int pi = lane & 3;
        v4f pacc[GQ / 4][DPL];
#pragma unroll
        for (int hq = 0; hq < GQ / 4; ++hq)
#pragma unroll
          for (int t = 0; t < DPL; ++t)
            pacc[hq][t] = v4f{acc[4 * hq][t], acc[4 * hq + 1][t], acc[4 * hq + 2][t],
                              acc[4 * hq + 3][t]};
        load_q(nxt);  // the next item's query heads stream in under P.V
        __builtin_amdgcn_sched_barrier(0);
        auto quad = [&](auto J4) {
          constexpr int j4 = decltype(J4)::value;
          float4 p4[GQ / 4];
#pragma unroll
          for (int hq = 0; hq < GQ / 4; ++hq)
            p4[hq] = ps4[((4 * hq + pi) * C + wave * KPW) / 4 + j4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int hq = 0; hq < GQ / 4; ++hq) {
              const float pv = jj == 0 ? p4[hq].x : jj == 1 ? p4[hq].y : jj == 2 ? p4[hq].z : p4[hq].w;
#pragma unroll
              for (int t = 0; t < DPL; ++t)  // rows past the width carry p = 0
                pacc[hq][t] = __builtin_amdgcn_mfma_f32_4x4x1f32(pv, vreg[4 * j4 + jj][t],
                                                                 pacc[hq][t], 0, 0, 0);
            }
          __builtin_amdgcn_sched_barrier(0);
          load_v_rows(nxt, cn_next, rs_next, std::integral_constant<int, 4 * j4>{},
                      std::integral_constant<int, 4 * j4 + 4>{});
          __builtin_amdgcn_sched_barrier(0);
        };
        static_assert(KPW == 16, "four row quads per wavefront");
        quad(std::integral_constant<int, 0>{});
        quad(std::integral_constant<int, 1>{});
        quad(std::integral_constant<int, 2>{});
        quad(std::integral_constant<int, 3>{});
#pragma unroll
        for (int hq = 0; hq < GQ / 4; ++hq)
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2)
#pragma unroll
            for (int t = 0; t < DPL; ++t) acc[4 * hq + i2][t] = pacc[hq][t][i2];
      } else {
        // head-major, one head's weights live at a time (the scheduling barrier
        // keeps the compiler from hoisting every head's LDS reads at once)
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
          float4 p4[KPW / 4];
#pragma unroll
          for (int j4 = 0; j4 < KPW / 4; ++j4) p4[j4] = ps4[(h * C + wave * KPW) / 4 + j4];
#pragma unroll
          for (int j4 = 0; j4 < KPW / 4; ++j4) {
            const float pv[4] = {p4[j4].x, p4[j4].y, p4[j4].z, p4[j4].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
              for (int t = 0; t < DPL; ++t)  // rows past the width carry p = 0
                acc[h][t] = __builtin_fmaf(pv[jj], vreg[4 * j4 + jj][t], acc[h][t]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (GQ % 4 != 0) {
        __builtin_amdgcn_sched_barrier(0);
        load_q(nxt);  // the next item's query heads, then its V, stream in under the rest
        __builtin_amdgcn_sched_barrier(0);
        load_v(nxt, cn_next, rs_next);
      }

      // at the range's last chunk: the wavefronts' states are exchanged,
      // rescaled to the range maximum and added in wavefront order, and the
      // range partial is stored; the state then restarts
      const int64_t slot0 =
          (cur.lrow * q_heads + (int64_t)cur.hk * GQ) * n_ranges + cur.chunk / RC;
      const bool range_end = pnx.sub == 0;
      if (range_end) {
        __syncthreads();  // every wavefront is done reading K: smem can hold the states
#pragma unroll
        for (int h = 0; h < GQ; ++h)
#pragma unroll
          for (int t = 0; t < DPL; ++t) smem[(wave * GQ + h) * D + lane * DPL + t] = acc[h][t];
        if (lq == 0 && hcol) {
          mw_sh[wave][li] = m_run;
          lw_sh[wave][li] = l_run;
        }
        __syncthreads();
        if (cn > 0) {
#pragma unroll
          for (int r = 0; r < OV4; ++r) {
            const int o4 = tid + r * NT;
            if (o4 < GQ * D / 4) {
              const int h = (4 * o4) / D;
              const int d = 4 * o4 - h * D;
              float mc = mw_sh[0][h];
#pragma unroll
              for (int w = 1; w < NW; ++w) mc = fmaxf(mc, mw_sh[w][h]);
              float ew[NW];
#pragma unroll
              for (int w = 0; w < NW; ++w) ew[w] = expf(mw_sh[w][h] - mc);
              const float4 t0 = smem4[(h * D + d) / 4];
              float4 sum = make_float4(t0.x * ew[0], t0.y * ew[0], t0.z * ew[0], t0.w * ew[0]);
              float lc = lw_sh[0][h] * ew[0];
#pragma unroll
              for (int ww = 1; ww < NW; ++ww) {
                const float4 t = smem4[((ww * GQ + h) * D + d) / 4];
                sum.x = __builtin_fmaf(t.x, ew[ww], sum.x);
                sum.y = __builtin_fmaf(t.y, ew[ww], sum.y);
                sum.z = __builtin_fmaf(t.z, ew[ww], sum.z);
                sum.w = __builtin_fmaf(t.w, ew[ww], sum.w);
                lc = __builtin_fmaf(lw_sh[ww][h], ew[ww], lc);
              }
              *reinterpret_cast<float4*>(part_acc + (slot0 + (int64_t)h * n_ranges) * D + d) = sum;
              if (d == 0)
                *reinterpret_cast<float2*>(part_ml + (slot0 + (int64_t)h * n_ranges) * 2) =
                    make_float2(mc, lc);
            }
          }
        }
        m_run = -INFINITY;
        l_run = 0.0f;
#pragma unroll
        for (int h = 0; h < GQ; ++h)
#pragma unroll
          for (int t = 0; t < DPL; ++t) acc[h][t] = 0.0f;
      }
      resolve_store(FUSED ? (j + 2) % 3 : 0, cn_next2);  // visible after the next item's first barrier
    }
    pcur = pnx;
    cur = nxt;
    cn = cn_next;
    ++j;
  }
}

// Merge of the range partials of one (query head, row): lane c holds range
// c's (m_c, l_c) and its weight a_c = exp(m_c - m); four wavefronts each fold
// a contiguous quarter of the ranges in ascending order (weights broadcast
// from their lanes), then the quarters are added in order.  Every load a
// wavefront needs -- all (m_c, l_c) and its quarter's accumulators -- is
// issued before the first use, so the merge costs one memory round trip.
constexpr int kMaxChunks = (4 * QSA_MAX_BUDGET + 3 + C - 1) / C;  // 65
constexpr int kMaxParts = attn_parts(kMaxChunks);                  // 9
constexpr int kMaxQuarter = (kMaxParts + 3) / 4;                   // 3

template <int D>
__global__ void __launch_bounds__(4 * kWave)
merge_kernel(const float* __restrict__ part_acc, const float* __restrict__ part_ml,
             const int32_t* __restrict__ width, int32_t q_heads, int32_t n_chunks,
             int32_t stride, int64_t row0, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int DPL = D / kWave;
  static_assert(kMaxParts <= kWave, "one range partial per lane at most");
  __shared__ float red[4][D + 1];
  const int wave = wave_id();
  const int lane = lane_id();
  const int64_t hq = blockIdx.x;
  const int64_t lrow = blockIdx.y;
  const int64_t row = row0 + lrow;
  const int32_t w = width[row];
  float* o = out + (row * q_heads + hq) * D;
  if (w <= 0 || w > stride - 1) {
    if (wave == 0) {
      const float fill = (w == 0) ? 0.0f : __int_as_float(0x7fc00000);
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[lane * DPL + j] = fill;
      if (lse && lane == 0) lse[row * q_heads + hq] = (w == 0) ? -INFINITY : fill;
    }
    return;
  }
  const int nc = attn_parts((w + C - 1) / C);  // range partials of this row
  const int64_t base = (lrow * q_heads + hq) * attn_parts(n_chunks);
  const int per = (nc + 3) / 4;
  const int cb = wave * per;
  const int cnt = (cb + per) < nc ? per : (nc > cb ? nc - cb : 0);
  // loads: (m, l) of range lane; this quarter's accumulators (indexes are
  // clamped to range nc-1, so every load is in bounds)
  const int c0 = lane < nc ? lane : nc - 1;
  float2 ml0 = *reinterpret_cast<const float2*>(part_ml + (base + c0) * 2);
  if (lane >= nc) ml0 = make_float2(-INFINITY, 0.0f);
  float pa[kMaxQuarter][DPL];
#pragma unroll
  for (int t = 0; t < kMaxQuarter; ++t) {
    const int c = t < cnt ? cb + t : nc - 1;
#pragma unroll
    for (int j = 0; j < DPL; ++j) pa[t][j] = part_acc[(base + c) * D + lane * DPL + j];
  }
  const float m = wave_max(ml0.x);
  const float a0 = lane < nc ? expf(ml0.x - m) : 0.0f;
  const float wl0 = ml0.y * a0;
  float l = 0.0f;
  float acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int t = 0; t < kMaxQuarter; ++t) {
    if (t < cnt) {  // uniform
      const int c = cb + t;
      const float a = read_lane(a0, c);
      l = l + read_lane(wl0, c);
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[j] = __builtin_fmaf(pa[t][j], a, acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < DPL; ++j) red[wave][lane * DPL + j] = acc[j];
  if (lane == 0) red[wave][D] = l;
  __syncthreads();
  if (wave == 0) {
    float lt = red[0][D];
    float at[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) at[j] = red[0][lane * DPL + j];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) {
      lt = lt + red[ww][D];
#pragma unroll
      for (int j = 0; j < DPL; ++j) at[j] = at[j] + red[ww][lane * DPL + j];
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[lane * DPL + j] = at[j] / lt;
    if (lse && lane == 0) lse[row * q_heads + hq] = m + logf(lt);
  }
}

}  // namespace

namespace {

// Persistent launch: as many workgroups as can be resident at once (queried
// once per kernel instance), each walking the work items with a stride of the
// grid size.

template <int D, int GQ, int MODE>
hipError_t launch_attend_t(const AttendArgs& a, hipStream_t s) {
  using A = AttnCfg<D, GQ>;
  // resident workgroups per compute unit for this instance; concurrent first
  // calls may both query it and store the same value
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attend_chunk_kernel<D, GQ, MODE>, A::NT,
                                                     0) != hipSuccess ||
        n < 1)
      n = 1;
    per_cu = n;
    per_cu_cache.store(n, std::memory_order_relaxed);
  }
  const int64_t items = (int64_t)attn_parts(a.n_chunks) * a.rows * a.kv_heads;
  const int64_t slots = (int64_t)device_cus() * per_cu;
  const unsigned grid = (unsigned)(items < slots ? items : slots);
  RowSource src{a.k_compact, a.v_compact, MODE == kUnion ? a.union_pos : a.token_ids, a.seq_len,
                a.slot_map, a.slot_off, a.k_cache, a.v_cache, a.kv_slots, a.queries};
  hipLaunchKernelGGL((attend_chunk_kernel<D, GQ, MODE>), dim3(grid), dim3(A::NT), 0, s, a.q, src,
                     a.width, a.q_heads, a.kv_heads, a.stride, a.n_chunks, a.scale, a.row0,
                     a.rows, a.part_acc, a.part_ml);
  return hipGetLastError();
}

template <int D, int GQ>
hipError_t launch_attend_f(const AttendArgs& a, hipStream_t s) {
  if (a.union_pos) return launch_attend_t<D, GQ, kUnion>(a, s);
  if (a.token_ids) return launch_attend_t<D, GQ, kFused>(a, s);
  return launch_attend_t<D, GQ, kCompact>(a, s);
}

template <int D>
hipError_t launch_attend_d(const AttendArgs& a, hipStream_t s) {
  switch (a.q_heads / a.kv_heads) {
    case 1: return launch_attend_f<D, 1>(a, s);
    case 2: return launch_attend_f<D, 2>(a, s);
    case 4: return launch_attend_f<D, 4>(a, s);
    case 8: return launch_attend_f<D, 8>(a, s);
    case 16: return launch_attend_f<D, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int launch_attend(const AttendArgs& a, void* stream) {
  if (a.rows == 0) return 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.head_dim) {
    case 64: return launch_attend_d<64>(a, s);
    case 128: return launch_attend_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

int launch_merge(const AttendArgs& a, void* stream) {
  if (a.rows == 0) return 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)a.q_heads, (unsigned)a.rows);
  switch (a.head_dim) {
    case 64:
      hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(4 * kWave), 0, s, a.part_acc, a.part_ml,
                         a.width, a.q_heads, a.n_chunks, a.stride, a.row0, a.out, a.lse);
      break;
    case 128:
      hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(4 * kWave), 0, s, a.part_acc, a.part_ml,
                         a.width, a.q_heads, a.n_chunks, a.stride, a.row0, a.out, a.lse);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
