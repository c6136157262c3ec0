// union.hip -- steps 6-7 for causal chunks with one gather per pass: the
// rows of a chunk (the queries of one sequence) choose almost the same
// groups, so the K/V rows they need are resolved through the slot map and
// copied once, into a union scratch, instead of once per row.  Each row then
// reads its chronological IDs through a per-row position list into that
// scratch.  The copy is still one explicit, bounded copy of only selected
// rows (AFN-016 "A sparse mask is not sparse attention", §Decision; §Why
// compact gather comes before fusion), and the K/V bits each row sees are
// those of its own compact row, so the attention result is unchanged.
//
// Union unit: the 4-token group.  A pass's union holds every group that
// some row of the pass (same sequence) selected or whose raw tail it reads;
// union group u of the pass occupies scratch rows 4u..4u+3, groups ordered
// by (sequence, group position).  Per pass:
//   union_mark_kernel    row bitmap of the groups the row's IDs touch
//   union_or_kernel      per sequence: OR of its rows' bitmaps
//   union_count_kernel   popcount per block of bitmap words
//   union_scan_kernel    exclusive scan of the block counts (one workgroup)
//   union_list_kernel    word prefixes and the list of union groups (alone
//                        when the bitmap fits one block)
//   union_gather_kernel  slot-map resolution and K/V copy per union group
//   union_pos_kernel     per row: ID -> scratch row (-1 when invalid)
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanWords = kUnionScanWords;  // bitmap words per count/list block
static_assert(kScanWords == 4 * kScanThreads, "four words per scan thread");

// Visible tokens of a row (negative: no such row in its sequence).
__device__ __forceinline__ int64_t row_visible(const int32_t* seq_len, int64_t row,
                                               int32_t queries, int32_t* b_out) {
  const int32_t b = (int32_t)(row / queries);
  *b_out = b;
  return (int64_t)seq_len[b] - queries + 1 + (row - (int64_t)b * queries);
}

// An ID the union can hold: visible to its row and inside the bitmap.
__device__ __forceinline__ bool id_ok(int32_t id, int64_t n, int64_t wps) {
  return id >= 0 && (int64_t)id < n && ((int64_t)id >> 7) < wps;
}

__device__ __forceinline__ bool width_ok(int32_t w, int32_t stride) {
  return w > 0 && w <= stride - 1;
}

// Row bitmaps of up to kMarkLdsWords words are built in LDS (LDS atomics,
// then one coalesced write of the whole bitmap); larger ones are built in
// place with global atomics.
constexpr int kMarkLdsWords = 8192;  // 32 KiB: max_groups up to 262,144

template <bool IN_LDS>
__global__ void __launch_bounds__(256)
union_mark_kernel(const int32_t* __restrict__ token_ids, const int32_t* __restrict__ width,
                  const int32_t* __restrict__ seq_len, int32_t queries, int32_t stride,
                  int64_t wps, int64_t row0, uint32_t* __restrict__ rbm) {
  __shared__ uint32_t sbm[IN_LDS ? kMarkLdsWords : 1];
  const int tid = (int)threadIdx.x;
  const int64_t lrow = blockIdx.x;
  const int64_t row = row0 + lrow;
  uint32_t* bm = rbm + lrow * wps;
  uint32_t* mark = IN_LDS ? sbm : bm;
  for (int64_t w = tid; w < wps; w += 256) mark[w] = 0u;
  if (!IN_LDS) __threadfence();
  __syncthreads();
  const int32_t wd = width[row];
  if (width_ok(wd, stride)) {  // an invalid row keeps an empty bitmap
    int32_t b;
    const int64_t n = row_visible(seq_len, row, queries, &b);
    const int32_t* ids = token_ids + row * stride;
    for (int i = tid; i < wd; i += 256) {
      const int32_t id = ids[i];
      if (id_ok(id, n, wps)) {
        const uint32_t g = (uint32_t)id >> 2;
        atomicOr(&mark[g >> 5], 1u << (g & 31));
      }
    }
  }
  if (IN_LDS) {
    __syncthreads();
    for (int64_t w = tid; w < wps; w += 256) bm[w] = sbm[w];
  }
}

// ubm[s][w] = OR over the pass rows of sequence b_first + s of rbm[row][w].
__global__ void __launch_bounds__(256)
union_or_kernel(const uint32_t* __restrict__ rbm, int32_t queries, int64_t wps, int64_t row0,
                int64_t rows, int64_t b_first, uint32_t* __restrict__ ubm) {
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= wps) return;
  const int64_t s = blockIdx.y;
  const int64_t b = b_first + s;
  const int64_t r_lo = b * queries > row0 ? b * queries : row0;
  const int64_t r_end = (b + 1) * queries < row0 + rows ? (b + 1) * queries : row0 + rows;
  // 32 rows' words in flight per round trip (the rows of a 256-query chunk
  // take eight round trips)
  uint32_t v = 0u;
#pragma unroll 32
  for (int64_t r = r_lo; r < r_end; ++r) v |= rbm[(r - row0) * wps + w];
  ubm[s * wps + w] = v;
}

__device__ __forceinline__ void load_words(const uint32_t* ubm, int64_t words, int64_t w0,
                                           uint32_t v[4], uint32_t* cnt) {
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = (w0 + e < words) ? ubm[w0 + e] : 0u;
    c += (uint32_t)__popc(v[e]);
  }
  *cnt = c;
}

__global__ void __launch_bounds__(kScanThreads)
union_count_kernel(const uint32_t* __restrict__ ubm, int64_t words, uint32_t* __restrict__ blk) {
  __shared__ uint32_t wave_tot[kScanThreads / kWave];
  const int64_t w0 = (int64_t)blockIdx.x * kScanWords + 4 * (int64_t)threadIdx.x;
  uint32_t v[4], c, tot;
  load_words(ubm, words, w0, v, &c);
  (void)block_exclusive_sum<kScanThreads>(c, wave_tot, &tot);
  if (threadIdx.x == 0) blk[blockIdx.x] = tot;
}

// blk[0..nb) -> exclusive prefix; blk[nb] = total union groups (also written
// to *count_out when given).
__global__ void __launch_bounds__(kScanThreads)
union_scan_kernel(uint32_t* __restrict__ blk, int64_t nb, int32_t* __restrict__ count_out) {
  __shared__ uint32_t wave_tot[kScanThreads / kWave];
  uint32_t run = 0;
  for (int64_t base = 0; base < nb; base += kScanThreads) {
    const int64_t i = base + threadIdx.x;
    const uint32_t c = i < nb ? blk[i] : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_sum<kScanThreads>(c, wave_tot, &tot);
    if (i < nb) blk[i] = run + ex;
    run += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    blk[nb] = run;
    if (count_out) *count_out = (int32_t)run;
  }
}

// upre[w] = union groups before word w; ulist[u] = (sequence slot, group).
// SINGLE: the bitmap fits one block, which then also writes the total to
// blk[1] and *count_out (the count and scan kernels are not launched).
template <bool SINGLE>
__global__ void __launch_bounds__(kScanThreads)
union_list_kernel(const uint32_t* __restrict__ ubm, int64_t words, int64_t wps,
                  uint32_t* __restrict__ blk, int32_t* __restrict__ count_out, uint32_t cap,
                  uint32_t* __restrict__ upre, int2* __restrict__ ulist) {
  __shared__ uint32_t wave_tot[kScanThreads / kWave];
  const int64_t w0 = (int64_t)blockIdx.x * kScanWords + 4 * (int64_t)threadIdx.x;
  uint32_t v[4], c, tot;
  load_words(ubm, words, w0, v, &c);
  uint32_t o = (SINGLE ? 0u : blk[blockIdx.x]) +
               block_exclusive_sum<kScanThreads>(c, wave_tot, &tot);
  if (SINGLE && threadIdx.x == 0) {
    blk[1] = tot;
    if (count_out) *count_out = (int32_t)tot;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t w = w0 + e;
    if (w >= words) break;
    upre[w] = o;
    const int32_t s = (int32_t)(w / wps);
    const int32_t gw = (int32_t)(w - (int64_t)s * wps) * 32;
    uint32_t bits = v[e];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1u;
      if (o < cap) ulist[o] = make_int2(s, gw + bit);
      ++o;
    }
  }
}

// Union groups two at a time (8 scratch rows): the first lanes resolve the
// slots into LDS, then every thread issues its float4 loads before any
// store.  Tokens past the last row of the pass that sees the most of the
// sequence are never read by any row and are skipped; an out-of-range slot
// gives NaN rows, as in the per-row gather.
__global__ void __launch_bounds__(256)
union_gather_kernel(const int2* __restrict__ ulist, const uint32_t* __restrict__ count,
                    const int32_t* __restrict__ seq_len, const int32_t* __restrict__ slot_map,
                    const int64_t* __restrict__ slot_off, const float4* __restrict__ k_cache,
                    const float4* __restrict__ v_cache, int32_t queries, int32_t row_f4,
                    int64_t kv_slots, int64_t row0, int64_t rows, int64_t b_first, uint32_t cap,
                    float4* __restrict__ k_out, float4* __restrict__ v_out) {
  constexpr int kTok = 8;
  __shared__ int32_t slot_sh[kTok];
  const int tid = (int)threadIdx.x;
  const uint32_t U = *count < cap ? *count : cap;
  const float nan = __int_as_float(0x7fc00000);
  for (int64_t p = blockIdx.x; 2 * p < (int64_t)U; p += gridDim.x) {
    __syncthreads();  // slot_sh of the previous pair is no longer read
    if (tid < kTok) {
      const int64_t u = 2 * p + (tid >> 2);
      int32_t slot = -2;  // -2: nothing to copy
      if (u < (int64_t)U) {
        const int2 en = ulist[u];
        const int64_t b = b_first + en.x;
        // visible tokens of the pass's last row of sequence b
        const int64_t r_end = (b + 1) * queries < row0 + rows ? (b + 1) * queries : row0 + rows;
        const int64_t n_max = (int64_t)seq_len[b] - queries + (r_end - b * queries);
        const int64_t t = 4 * (int64_t)en.y + (tid & 3);
        if (t < n_max) {
          const int32_t sl = slot_map[slot_off[b] + t];
          slot = (sl >= 0 && (int64_t)sl < kv_slots) ? sl : -1;
        }
      }
      slot_sh[tid] = slot;
    }
    __syncthreads();
    const int total = kTok * row_f4;
    constexpr int kPer = 8;
    for (int base = 0; base < total; base += kPer * 256) {
      float4 kv[kPer], vv[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int e0 = base + tid + r * 256;
        const int e = e0 < total ? e0 : total - 1;
        const int t = e / row_f4;
        const int c = e - t * row_f4;
        const int32_t slot = slot_sh[t];
        const int64_t src = (int64_t)(slot >= 0 ? slot : 0) * row_f4 + c;
        kv[r] = k_cache[src];
        vv[r] = v_cache[src];
      }
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int e = base + tid + r * 256;
        if (e < total) {
          const int t = e / row_f4;
          const int c = e - t * row_f4;
          const int32_t slot = slot_sh[t];
          if (slot != -2) {
            const int64_t dst = (8 * p + t) * (int64_t)row_f4 + c;
            k_out[dst] = slot >= 0 ? kv[r] : make_float4(nan, nan, nan, nan);
            v_out[dst] = slot >= 0 ? vv[r] : make_float4(nan, nan, nan, nan);
          }
        }
      }
    }
  }
}

// pos[row][i] = scratch row of the row's i-th ID: 4*(union groups before its
// group) + ID%4; -1 past the width or for an ID the row cannot see.
__global__ void __launch_bounds__(256)
union_pos_kernel(const int32_t* __restrict__ token_ids, const int32_t* __restrict__ width,
                 const int32_t* __restrict__ seq_len, const uint32_t* __restrict__ ubm,
                 const uint32_t* __restrict__ upre, int32_t queries, int32_t stride, int64_t wps,
                 int64_t row0, int64_t b_first, uint32_t cap, int32_t* __restrict__ pos) {
  const int64_t lrow = blockIdx.y;
  const int64_t row = row0 + lrow;
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (i >= stride) return;
  const int32_t wd = width[row];
  int32_t out = -1;
  if (width_ok(wd, stride) && i < wd) {
    int32_t b;
    const int64_t n = row_visible(seq_len, row, queries, &b);
    const int32_t id = token_ids[row * stride + i];
    if (id_ok(id, n, wps)) {
      const uint32_t g = (uint32_t)id >> 2;
      const int64_t w = (int64_t)(b - b_first) * wps + (g >> 5);
      const uint32_t below = ubm[w] & ((1u << (g & 31)) - 1u);
      const uint32_t u = upre[w] + (uint32_t)__popc(below);
      if (u < cap) out = (int32_t)(4u * u + ((uint32_t)id & 3u));
    }
  }
  pos[lrow * stride + i] = out;
}

}  // namespace

int launch_union(const UnionArgs& a, void* stream) {
  if (a.rows == 0) return 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int2* union_list = reinterpret_cast<int2*>(a.union_list);
  const int64_t wps = union_words_per_seq(a.max_groups);
  const int64_t b_first = a.row0 / a.queries;
  const int64_t b_last = (a.row0 + a.rows - 1) / a.queries;
  const int64_t seqs = b_last - b_first + 1;
  const int64_t words = seqs * wps;
  const int64_t nb = union_scan_blocks(words);
  if (wps <= kMarkLdsWords)
    hipLaunchKernelGGL(union_mark_kernel<true>, dim3((unsigned)a.rows), dim3(256), 0, s,
                       a.token_ids, a.width, a.seq_len, a.queries, a.stride, wps, a.row0,
                       a.row_bitmap);
  else
    hipLaunchKernelGGL(union_mark_kernel<false>, dim3((unsigned)a.rows), dim3(256), 0, s,
                       a.token_ids, a.width, a.seq_len, a.queries, a.stride, wps, a.row0,
                       a.row_bitmap);
  hipLaunchKernelGGL(union_or_kernel, dim3((unsigned)((wps + 255) / 256), (unsigned)seqs),
                     dim3(256), 0, s, a.row_bitmap, a.queries, wps, a.row0, a.rows, b_first,
                     a.union_bitmap);
  // capacity: a selection touches at most k+1 groups per row (k chosen, one
  // tail group); IDs from elsewhere may touch more, and groups past the
  // capacity are then neither listed nor copied, and their IDs get position -1
  const uint32_t cap = (uint32_t)(a.rows * (int64_t)(a.stride / 4));
  if (nb == 1) {
    hipLaunchKernelGGL(union_list_kernel<true>, dim3(1), dim3(kScanThreads), 0, s,
                       a.union_bitmap, words, wps, a.block_prefix, a.count_out, cap,
                       a.word_prefix, union_list);
  } else {
    hipLaunchKernelGGL(union_count_kernel, dim3((unsigned)nb), dim3(kScanThreads), 0, s,
                       a.union_bitmap, words, a.block_prefix);
    hipLaunchKernelGGL(union_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a.block_prefix, nb,
                       a.count_out);
    hipLaunchKernelGGL(union_list_kernel<false>, dim3((unsigned)nb), dim3(kScanThreads), 0, s,
                       a.union_bitmap, words, wps, a.block_prefix, nullptr, cap, a.word_prefix,
                       union_list);
  }
  const int32_t row_f4 = a.kv_heads * a.head_dim / 4;
  const int64_t pairs = ((int64_t)cap + 1) / 2;
  const int64_t max_grid = (int64_t)a.cus * 8;
  hipLaunchKernelGGL(union_gather_kernel, dim3((unsigned)(pairs < max_grid ? pairs : max_grid)),
                     dim3(256),
                     0, s, union_list, a.block_prefix + nb, a.seq_len, a.slot_map, a.slot_off,
                     reinterpret_cast<const float4*>(a.k_cache),
                     reinterpret_cast<const float4*>(a.v_cache), a.queries, row_f4, a.kv_slots,
                     a.row0, a.rows, b_first, cap, reinterpret_cast<float4*>(a.k_union),
                     reinterpret_cast<float4*>(a.v_union));
  hipLaunchKernelGGL(union_pos_kernel, dim3((unsigned)((a.stride + 255) / 256), (unsigned)a.rows),
                     dim3(256), 0, s, a.token_ids, a.width, a.seq_len, a.union_bitmap,
                     a.word_prefix, a.queries, a.stride, wps, a.row0, b_first, cap,
                     a.union_pos);
  return hipGetLastError();
}

}  // namespace qsa
