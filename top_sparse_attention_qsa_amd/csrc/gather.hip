// gather.hip -- steps 6-7: resolve each selected logical token ID once through
// the slot map and copy only those K/V cache rows into compact scratch, in
// row (chronological) order.  Only this step crosses from logical identity to
// physical cache layout, so selection never needs to know whether the cache
// wrapped, compacted or reused a slot (AFN-016 "A sparse mask is not sparse
// attention", §Decision; §Why compact gather comes before fusion: one
// explicit copy into bounded scratch).
//
// A workgroup handles kGatherTokens compact rows of one query row: the first
// lanes resolve the slots into LDS, then all 256 threads stream the H_kv*D
// floats of each K and V cache row with float4 loads (2 KiB contiguous per
// row at H_kv=4, D=128) and store each KV head's D floats into that head's
// run of the compact scratch ([row][KV head][position][dim]), which the
// attention then reads as one contiguous block per (row, head, chunk).
// Out-of-range IDs or slots produce NaN rows and slot -1 instead of a fault.
#include "qsa_internal.h"

namespace qsa {
namespace {

// Cache rows are read once per step: nontemporal loads keep them from
// displacing the compact rows, which the attention reads next.
__device__ __forceinline__ float4 load_stream(const float4* p) {
  typedef float v4 __attribute__((ext_vector_type(4)));
  const v4 v = __builtin_nontemporal_load(reinterpret_cast<const v4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__global__ void __launch_bounds__(256)
gather_kernel(const int32_t* __restrict__ token_ids, const int32_t* __restrict__ width,
              const int32_t* __restrict__ seq_len, const int32_t* __restrict__ slot_map,
              const int64_t* __restrict__ slot_off, const float4* __restrict__ k_cache,
              const float4* __restrict__ v_cache, int32_t queries, int32_t row_f4, int32_t head_f4,
              int32_t stride, int64_t kv_slots, int64_t row0, float4* __restrict__ k_out,
              float4* __restrict__ v_out, int32_t* __restrict__ phys_slots) {
  __shared__ int32_t slot_sh[kGatherTokens];
  const int tid = (int)threadIdx.x;
  const int64_t lrow = blockIdx.y;
  const int64_t row = row0 + lrow;
  const int32_t i0 = (int32_t)blockIdx.x * kGatherTokens;
  // The width, the token IDs (read speculatively, clamped to the row), the
  // sequence length and the slot-map offset do not depend on each other:
  // they are loaded together, then the slot map -- two dependent memory
  // round trips before the copy instead of four.
  const int32_t w = width[row];
  const int32_t b = (int32_t)(row / queries);
  const int32_t i = i0 + tid;
  int32_t id = -1, len = 0;
  int64_t soff = 0;
  if (tid < kGatherTokens) {
    id = token_ids[row * stride + (i < stride ? i : stride - 1)];
    len = seq_len[b];
    soff = slot_off[b];
  }
  if (w <= 0 || w > stride - 1 || i0 >= w) return;  // widths above 4k+3 are invalid
  if (tid < kGatherTokens) {
    int32_t slot = -2;  // -2: past the width, nothing to copy
    if (i < w) {
      const int64_t n = (int64_t)len - queries + 1 + (row - (int64_t)b * queries);
      slot = -1;
      if (id >= 0 && (int64_t)id < n) {
        const int32_t sl = slot_map[soff + id];
        if (sl >= 0 && (int64_t)sl < kv_slots) slot = sl;
      }
      if (phys_slots) phys_slots[row * stride + i] = slot;
    }
    slot_sh[tid] = slot;
  }
  __syncthreads();
  // All loads of a pass are issued before any store (slots that are out of
  // range or past the width read slot 0, which exists because kv_slots >= 1,
  // and are masked afterwards), so each pass costs one memory round trip.
  const float nan = __int_as_float(0x7fc00000);
  const int total = kGatherTokens * row_f4;
  constexpr int kPer = 4;  // float4 per thread per pass (one pass for H_kv x D = 512)
  for (int base = 0; base < total; base += kPer * 256) {
    float4 kv[kPer], vv[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int e0 = base + tid + r * 256;
      const int e = e0 < total ? e0 : total - 1;  // branch-free: the tail re-reads the last float4
      const int t = e / row_f4;
      const int c = e - t * row_f4;
      const int32_t slot = slot_sh[t];
      const int64_t src = (int64_t)(slot >= 0 ? slot : 0) * row_f4 + c;
      kv[r] = load_stream(k_cache + src);
      vv[r] = load_stream(v_cache + src);
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int e = base + tid + r * 256;
      if (e < total) {
        const int t = e / row_f4;
        const int c = e - t * row_f4;
        const int32_t slot = slot_sh[t];
        if (slot != -2) {
          // compact layout [row][KV head][position][dim]: a head's rows of one
          // query row are contiguous, so the attention streams them
          const int hk = c / head_f4;
          const int64_t dst = ((lrow * (row_f4 / head_f4) + hk) * stride + i0 + t) * head_f4 +
                              (c - hk * head_f4);
          k_out[dst] = slot >= 0 ? kv[r] : make_float4(nan, nan, nan, nan);
          v_out[dst] = slot >= 0 ? vv[r] : make_float4(nan, nan, nan, nan);
        }
      }
    }
  }
}

}  // namespace

int launch_gather(const GatherArgs& a, void* stream) {
  if (a.rows == 0) return 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t row_f4 = a.kv_heads * a.head_dim / 4;
  dim3 grid((unsigned)((a.stride + kGatherTokens - 1) / kGatherTokens), (unsigned)a.rows);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, s, a.token_ids, a.width, a.seq_len,
                     a.slot_map, a.slot_off, reinterpret_cast<const float4*>(a.k_cache),
                     reinterpret_cast<const float4*>(a.v_cache), a.queries, row_f4,
                     a.head_dim / 4, a.stride,
                     a.kv_slots, a.row0, reinterpret_cast<float4*>(a.k_compact),
                     reinterpret_cast<float4*>(a.v_compact), a.phys_slots);
  return hipGetLastError();
}

}  // namespace qsa
